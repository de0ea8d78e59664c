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
//
// cp_build_attn_meta kernel: the query / key ranges of every rank's attention
// steps after the all-gather (same PR, "Why": two steps per rank under the
// per-document partition, one under packed-contiguous; "Scope and
// constraints": causal THD self-attention).  Chunk k of a document with chunk
// length c sees the document's first (k+1) c keys; a packed-contiguous segment
// sees its document from the first token on.  Every table entry has a closed
// form in cu, the rank's local cu and the look-back from the rank's first
// token to its document's start, so a thread per entry fills the tables.
#include "device_common.h"

namespace cpthd {
namespace {

__global__ void __launch_bounds__(kBlock)
build_meta_kernel(const int32_t* __restrict__ cu, int32_t B, int64_t T, int32_t W,
                  int32_t policy, int32_t row_maps, char* __restrict__ meta) {
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
  int64_t running = 0;  // packed-contiguous: boundaries kept so far
  // 64-bit document indexes throughout: B + kBlock may exceed 2^31 - 1.
  for (int64_t base = 0; base <= B; base += kBlock) {
    const int64_t b = base + tid;
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
      const int64_t pos = 1 + running + wave_prefix + lane_prefix;
      if (keep && pos <= B) lcu[pos] = (int32_t)((int64_t)v - lo);
      running += chunk_total;
      __syncthreads();  // s_wave_count is reused by the next chunk
    }
  }

  if (policy == CP_POLICY_PACKED_CONTIGUOUS) {
    const int64_t kept = running < B ? running : B;  // cannot exceed B-1 for valid input
    if (tid == 0) lcu[0] = 0;
    for (int64_t k = kept + 1 + tid; k <= B; k += kBlock) lcu[k] = (int32_t)n;
    if (tid == 0) nloc[r] = (n == 0) ? 0 : (int32_t)(kept + 1 <= B ? kept + 1 : B);
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
      h->row_maps = row_maps;
      for (int k = 0; k < 3; ++k) h->reserved[k] = 0;
      h->magic = CP_META_MAGIC;
    }
  }
}

// The dual-chunk-swap row maps after the tables (layout in cpthd.h): thread p
// maps flat local row p = r n + i to its global row through the rank-0 local
// cu (= cu / W) and writes both directions.  Runs after build_meta_kernel on
// the same stream; writes nothing when that kernel flagged the cu_seqlens.
__global__ void __launch_bounds__(kBlock) build_row_maps_kernel(char* __restrict__ meta) {
  const cp_meta_header* h = reinterpret_cast<const cp_meta_header*>(meta);
  if (h->magic != CP_META_MAGIC || (h->flags & CP_META_BUILD_MASK) != 0 || h->row_maps != 1) return;
  const int32_t W = h->cp_size;
  const int32_t B = h->num_docs;
  const int64_t T = h->total_tokens;
  const int64_t n = h->local_tokens;
  const int32_t* cu = reinterpret_cast<const int32_t*>(meta + meta_cu_offset());
  const int32_t* lcu = reinterpret_cast<const int32_t*>(meta + meta_local_cu_offset(B));
  int32_t* row_of_local = reinterpret_cast<int32_t*>(meta + meta_tables_bytes(B, W));
  int32_t* local_of_row = row_of_local + T;
  for (int64_t p = (int64_t)blockIdx.x * kBlock + threadIdx.x; p < T; p += (int64_t)gridDim.x * kBlock) {
    const int32_t r = (int32_t)(p / n);
    const int64_t i = p - (int64_t)r * n;
    const int32_t b = find_doc(lcu, B, i);
    const int64_t lstart = lcu[b];
    const int64_t c = (lcu[b + 1] - lstart) >> 1;
    const int64_t j = i - lstart;
    const int64_t g = j < c ? cu[b] + (int64_t)r * c + j : cu[b] + (int64_t)(2 * W - 1 - r) * c + (j - c);
    row_of_local[p] = (int32_t)g;
    local_of_row[g] = (int32_t)p;
  }
}

// Maximum over the workgroup (every thread gets it).
__device__ int32_t block_max(int32_t v) {
  __shared__ int32_t s_max[kWavesPerBlock];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = v;
  __syncthreads();
  int32_t m = s_max[0];
#pragma unroll
  for (int k = 1; k < kWavesPerBlock; ++k) m = max(m, s_max[k]);
  __syncthreads();  // s_max may be reused by the next call
  return m;
}

// One workgroup per (rank, step): blockIdx.x = 2 rank + step.
__global__ void __launch_bounds__(kBlock)
build_attn_meta_kernel(cp_meta_header* h, int32_t B, int32_t W, char* __restrict__ attn) {
  const int tid = threadIdx.x;
  const cp_meta_header hv = read_header(h);
  bool ok = meta_ok(h, hv, hv.total_tokens, W, -1);
  if (ok && hv.num_docs != B) {
    ok = false;
    if (blockIdx.x == 0 && tid == 0) atomicOr(&h->flags, CP_CALL_DOCS_MISMATCH);
  }
  if (blockIdx.x == 0 && tid == 0) {
    cp_attn_header* a = reinterpret_cast<cp_attn_header*>(attn);
    a->policy = ok ? hv.policy : -1;
    a->cp_size = W;
    a->num_docs = B;
    a->num_steps = ok ? (hv.policy == CP_POLICY_DUAL_CHUNK_SWAP ? 2 : 1) : 0;
    a->reserved0 = 0;
    a->total_tokens = ok ? hv.total_tokens : 0;
    a->local_tokens = ok ? hv.local_tokens : 0;
    for (int k = 0; k < 6; ++k) a->reserved[k] = 0;
    a->magic = ok ? CP_ATTN_MAGIC : 0u;
  }
  if (!ok) return;

  const int32_t r = blockIdx.x >> 1;
  const int32_t step = blockIdx.x & 1;
  const int32_t T = (int32_t)hv.total_tokens;
  const int32_t n = (int32_t)hv.local_tokens;
  const int32_t* cu = meta_cu(h);
  int32_t* scal = reinterpret_cast<int32_t*>(attn + attn_record_offset(B, blockIdx.x));
  int32_t* cuq = scal + 8;
  int32_t* cukv = cuq + (B + 1);
  int32_t* qoff = cukv + (B + 1);
  int32_t* kvoff = qoff + (B + 1);

  if (hv.policy == CP_POLICY_DUAL_CHUNK_SWAP) {
    const int32_t k = step == 0 ? r : 2 * W - 1 - r;  // the step's chunk index
    const int32_t two_w = 2 * W;
    int32_t max_c = 0;
    for (int64_t j = tid; j <= B; j += kBlock) {
      const int32_t v = cu[j];
      const int32_t before = v / two_w;  // chunk length summed over documents 0..j-1
      cuq[j] = before;
      cukv[j] = (k + 1) * before;
      if (j < B) {
        const int32_t c = (cu[j + 1] - v) / two_w;
        qoff[j] = v / W + step * c;
        kvoff[j] = v;
        max_c = max(max_c, c);
      } else {
        qoff[j] = n;
        kvoff[j] = T;
      }
    }
    max_c = block_max(max_c);
    if (tid == 0) {
      const int32_t total_c = cu[B] / two_w;
      scal[0] = B;
      scal[1] = max_c;
      scal[2] = (k + 1) * max_c;
      scal[3] = total_c;
      scal[4] = (k + 1) * total_c;
      scal[5] = scal[6] = scal[7] = 0;
    }
    return;
  }

  // packed-contiguous: one step; the second record of a rank is empty.
  if (step == 1) {
    for (int64_t j = tid; j <= B; j += kBlock) {
      cuq[j] = 0;
      cukv[j] = 0;
      qoff[j] = n;
      kvoff[j] = T;
    }
    if (tid < 8) scal[tid] = 0;
    return;
  }
  const int32_t* lcu = reinterpret_cast<const int32_t*>(reinterpret_cast<const char*>(h) +
                                                        meta_local_cu_offset(B)) + (int64_t)r * (B + 1);
  const int32_t m = reinterpret_cast<const int32_t*>(reinterpret_cast<const char*>(h) +
                                                     meta_n_local_offset(B, W))[r];
  const int32_t first = r * n;  // the rank's first global token
  int32_t doc_start = 0, back = 0;
  if (m > 0) {
    doc_start = cu[find_doc(cu, B, first)];
    back = first - doc_start;  // keys of the first segment before the rank's slice
  }
  int32_t max_q = 0, max_kv = 0;
  for (int64_t j = tid; j <= B; j += kBlock) {
    const int32_t l = lcu[j];  // padded with n after entry m
    cuq[j] = l;
    qoff[j] = l;
    cukv[j] = j == 0 ? 0 : l + back;
    kvoff[j] = j >= m ? T : (j == 0 ? doc_start : first + l);
    if (j < m) {
      const int32_t q_len = lcu[j + 1] - l;
      max_q = max(max_q, q_len);
      max_kv = max(max_kv, j == 0 ? q_len + back : q_len);
    }
  }
  max_q = block_max(max_q);
  max_kv = block_max(max_kv);
  if (tid == 0) {
    scal[0] = m;
    scal[1] = max_q;
    scal[2] = max_kv;
    scal[3] = m > 0 ? n : 0;
    scal[4] = m > 0 ? n + back : 0;
    scal[5] = scal[6] = scal[7] = 0;
  }
}

}  // namespace

hipError_t launch_build_attn_meta(cp_meta_header* meta, int32_t B, int32_t W, void* attn, hipStream_t stream) {
  profile_before("build_attn_meta", stream);
  hipLaunchKernelGGL(build_attn_meta_kernel, dim3(2 * W), dim3(kBlock), 0, stream, meta, B, W,
                     static_cast<char*>(attn));
  hipError_t e = hipGetLastError();
  profile_after(stream);
  return e;
}

hipError_t launch_build_meta(const int32_t* cu, int32_t B, int64_t T, int32_t W, int32_t policy,
                             bool row_maps, void* meta, hipStream_t stream) {
  profile_before("build_meta", stream);
  hipLaunchKernelGGL(build_meta_kernel, dim3(W), dim3(kBlock), 0, stream, cu, B, T, W, policy,
                     row_maps ? 1 : 0, static_cast<char*>(meta));
  hipError_t e = hipGetLastError();
  profile_after(stream);
  if (e != hipSuccess || !row_maps || T == 0) return e;
  int64_t blocks = (T + kBlock - 1) / kBlock;
  if (blocks > kMaxGrid) blocks = kMaxGrid;
  profile_before("build_row_maps", stream);
  hipLaunchKernelGGL(build_row_maps_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, stream, static_cast<char*>(meta));
  e = hipGetLastError();
  profile_after(stream);
  return e;
}

}  // namespace cpthd
