// cp_build_meta kernel: validate cu_seqlens and emit per-rank local cu_seqlens.
//
// Dual-chunk-swap ("[PyTorch] Add experimental packed-contiguous THD
// all-gather CP", section "Why"; "Add stream-ordered CP gradient return
// primitive", author's reply on ownership): every document contributes two
// chunks of L_b/(2W) tokens to each rank, so each rank's local boundaries are
// cu/W.  Packed-contiguous (same PR, commit messages): rank r's slice is
// [rT/W, (r+1)T/W); its local boundaries are the global boundaries strictly
// inside the slice (first occurrence only, so empty documents vanish), shifted,
// between 0 and T/W.  The compaction is a wavefront ballot + popcount prefix,
// combined across the block's four waves through LDS.
#include "cpthd_internal.h"

namespace cpthd {
namespace {

__global__ void __launch_bounds__(kBlock)
build_meta_kernel(const int32_t* __restrict__ cu, int32_t B, int64_t T, int32_t W,
                  int32_t policy, char* __restrict__ meta) {
  const int r = blockIdx.x;  // one workgroup per rank
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t n = T / W;
  const int64_t lo = (int64_t)r * n;
  const int64_t hi = lo + n;

  int32_t* mcu = reinterpret_cast<int32_t*>(meta + meta_cu_offset());
  int32_t* lcu = reinterpret_cast<int32_t*>(meta + meta_local_cu_offset(B)) + (int64_t)r * (B + 1);
  int32_t* nloc = reinterpret_cast<int32_t*>(meta + meta_n_local_offset(B, W));

  __shared__ int s_wave_count[kWavesPerBlock];
  __shared__ int s_flags;
  if (tid == 0) s_flags = 0;
  __syncthreads();

  int flags = 0;
  int running = 0;  // packed-contiguous: boundaries kept so far
  for (int base = 0; base <= B; base += kBlock) {
    const int b = base + tid;
    const bool in = b <= B;
    const int32_t v = in ? cu[b] : 0;
    if (r == 0 && in) {
      mcu[b] = v;
      if (b == 0 && v != 0) flags |= CP_META_FIRST_NOT_ZERO;
      if (b == B && (int64_t)v != T) flags |= CP_META_LAST_NOT_TOTAL;
      if (b < B) {
        const int32_t next = cu[b + 1];
        if (next < v) flags |= CP_META_DECREASING;
        if (policy == CP_POLICY_DUAL_CHUNK_SWAP && ((int64_t)next - v) % (2 * W) != 0)
          flags |= CP_META_DOC_NOT_DIVISIBLE;
      }
    }
    if (policy == CP_POLICY_DUAL_CHUNK_SWAP) {
      if (in) lcu[b] = v / W;
    } else {
      bool keep = false;
      if (in) keep = (int64_t)v > lo && (int64_t)v < hi && (b == 0 || cu[b - 1] != v);
      const uint64_t ballot = __ballot(keep);
      const int lane_prefix = __popcll(ballot & ((1ull << lane) - 1ull));
      if (lane == 0) s_wave_count[wave] = __popcll(ballot);
      __syncthreads();
      int wave_prefix = 0, chunk_total = 0;
#pragma unroll
      for (int k = 0; k < kWavesPerBlock; ++k) {
        const int c = s_wave_count[k];
        wave_prefix += (k < wave) ? c : 0;
        chunk_total += c;
      }
      const int pos = 1 + running + wave_prefix + lane_prefix;
      if (keep && pos <= B) lcu[pos] = (int32_t)((int64_t)v - lo);
      running += chunk_total;
      __syncthreads();  // s_wave_count is reused by the next chunk
    }
  }

  if (policy == CP_POLICY_PACKED_CONTIGUOUS) {
    const int kept = running < B ? running : B;  // cannot exceed B-1 for valid input
    if (tid == 0) lcu[0] = 0;
    for (int k = kept + 1 + tid; k <= B; k += kBlock) lcu[k] = (int32_t)n;
    if (tid == 0) nloc[r] = (n == 0) ? 0 : (kept + 1 <= B ? kept + 1 : B);
  } else {
    if (tid == 0) nloc[r] = B;
  }

  if (r == 0) {
    if (flags) atomicOr(&s_flags, flags);
    __syncthreads();
    if (tid == 0) {
      cp_meta_header* h = reinterpret_cast<cp_meta_header*>(meta);
      h->flags = s_flags;
      h->policy = policy;
      h->cp_size = W;
      h->num_docs = B;
      h->reserved0 = 0;
      h->total_tokens = T;
      h->local_tokens = n;
      h->wait_timeout_ranks = 0;
      for (int k = 0; k < 4; ++k) h->reserved[k] = 0;
      h->magic = CP_META_MAGIC;
    }
  }
}

}  // namespace

hipError_t launch_build_meta(const int32_t* cu, int32_t B, int64_t T, int32_t W, int32_t policy,
                             void* meta, hipStream_t stream) {
  profile_before("build_meta", stream);
  hipLaunchKernelGGL(build_meta_kernel, dim3(W), dim3(kBlock), 0, stream, cu, B, T, W, policy,
                     static_cast<char*>(meta));
  hipError_t e = hipGetLastError();
  profile_after(stream);
  return e;
}

}  // namespace cpthd
