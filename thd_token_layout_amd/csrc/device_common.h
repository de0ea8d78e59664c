// Device helpers shared by the kernels: the metadata check every kernel runs
// first, and the dual-chunk-swap row map.
//
// Ownership ("[PyTorch] Add experimental packed-contiguous THD all-gather CP",
// section "Why"; "Add stream-ordered CP gradient return primitive", author's
// reply): every document b of length L_b is cut into 2W chunks of
// c_b = L_b / (2W) tokens; rank r holds chunk r then chunk 2W-1-r, document
// after document, so its local boundaries are local_cu = cu / W.  Local row i
// of rank r, in document b (local_cu[b] <= i < local_cu[b+1]) at offset
// j = i - local_cu[b], is global row
//     cu[b] + r c_b + j                 if j <  c_b
//     cu[b] + (2W-1-r) c_b + (j - c_b)  if j >= c_b.
#pragma once

#include "cpthd_internal.h"

namespace cpthd {

__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ const int32_t* meta_cu(const cp_meta_header* h) {
  return reinterpret_cast<const int32_t*>(reinterpret_cast<const char*>(h) + meta_cu_offset());
}
// local_cu of rank 0 (B documents); under dual-chunk-swap every rank's local_cu is cu / W.
__device__ __forceinline__ const int32_t* meta_local_cu0(const cp_meta_header* h, int32_t B) {
  return meta_cu(h) + (B + 1);
}

// A kernel's copy of the header: read once, before the kernel stores
// anything, so one 64-byte scalar read serves the check and every later use of
// a header field.  Measured on MI355X, per kernel: the slot sum runs 1-2%
// faster with the copy read first; the row-chunk permutation reads it while
// its data load is in flight; the row-tile permutation and the fused sum run
// 1-4% slower with a copy, so those read the fields from the metadata as the
// check reaches them (the overload below); the unit-tile permutation reads it
// through LDS (below).
__device__ __forceinline__ cp_meta_header read_header(const cp_meta_header* h) {
  typedef uint32_t u32x16 __attribute__((ext_vector_type(16), aligned(8)));
  static_assert(sizeof(cp_meta_header) == sizeof(u32x16), "the header is 64 bytes");
  const u32x16 w = *reinterpret_cast<const u32x16*>(h);
  cp_meta_header v;
  __builtin_memcpy(&v, &w, sizeof(v));
  return v;
}

// The same copy read in two steps, through vector memory into LDS: each wave
// issues one 64-byte load straight into its own 16 LDS words
// (load_header_lds), and later reads them back (header_from_lds, after
// waiting for everything in flight).  Scalar loads return out of order and
// share their counter with LDS accesses, so a kernel that waits for anything
// scalar or in LDS also waits for a scalar header read in flight; a vector
// load completes in order with the kernel's other global loads, so the header
// can stay in flight during lookups issued after it, and landing in LDS it
// holds no registers meanwhile.  `words` is the wave's 16 words of LDS.
__device__ __forceinline__ void load_header_lds(const cp_meta_header* h, uint32_t* words) {
  static_assert(sizeof(cp_meta_header) == 64, "the header is 64 bytes");
  const int lane = threadIdx.x & 63;
  if (lane < 4)
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint32_t*>(h) + 4 * lane, words, 16, 0, 0);
}
__device__ __forceinline__ cp_meta_header header_from_lds(const uint32_t* words) {
  __builtin_amdgcn_s_waitcnt(0);
  uint32_t u[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) u[k] = (uint32_t)__builtin_amdgcn_readfirstlane((int)words[k]);
  cp_meta_header v;
  __builtin_memcpy(&v, u, sizeof(v));
  return v;
}

// Returns false, and records why in the sticky call flags of `h`, when a
// kernel must not write any output: metadata never built, built from invalid
// cu_seqlens, or built for another token count, CP size (expect_W >= 0) or
// policy (expect_policy >= 0).  `v` is the kernel's copy of *h.  Every
// workgroup evaluates the same header, so all of them take the same decision;
// one thread records it.
__device__ __forceinline__ bool meta_ok(cp_meta_header* h, const cp_meta_header& v, int64_t T,
                                        int32_t expect_W, int32_t expect_policy) {
  int code = 0;
  if (v.magic != CP_META_MAGIC) code = CP_CALL_BAD_MAGIC;
  else if (v.flags & CP_META_BUILD_MASK) code = CP_CALL_USED_INVALID_META;
  else if (v.total_tokens != T) code = CP_CALL_TOKENS_MISMATCH;
  else if (expect_W >= 0 && v.cp_size != expect_W) code = CP_CALL_CP_SIZE_MISMATCH;
  else if (expect_policy >= 0 && v.policy != expect_policy) code = CP_CALL_POLICY_MISMATCH;
  if (code != 0 && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) atomicOr(&h->flags, code);
  return code == 0;
}
// The same check reading each header field from the metadata when it is needed.
__device__ __forceinline__ bool meta_ok(cp_meta_header* h, int64_t T, int32_t expect_W, int32_t expect_policy) {
  return meta_ok(h, *h, T, expect_W, expect_policy);
}

// Largest b in [0, B) with bound[b] <= v, for a nondecreasing bound[] with
// bound[0] <= v < bound[B]: the non-empty document holding position v.
// `bound` is a pointer or anything indexable; the midpoint is formed without
// overflow for every B up to 2^31 - 1 (callable on the host, so this holds in
// a CPU test near that size).
template <typename Bound>
__host__ __device__ __forceinline__ int32_t find_doc(const Bound& bound, int32_t B, int64_t v) {
  int32_t lo = 0, hi = B - 1;
  while (lo < hi) {
    const int32_t mid = lo + ((hi - lo + 1) >> 1);
    if ((int64_t)bound[mid] <= v) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Global row of local row i of rank r under dual-chunk-swap.
__device__ __forceinline__ int64_t dcs_global_row(int32_t r, int64_t i, int32_t W, int32_t B,
                                                  const int32_t* cu, const int32_t* lcu) {
  const int b = find_doc(lcu, B, i);
  const int64_t lstart = lcu[b];
  const int64_t c = (lcu[b + 1] - lstart) >> 1;
  const int64_t j = i - lstart;
  return j < c ? cu[b] + (int64_t)r * c + j : cu[b] + (int64_t)(2 * W - 1 - r) * c + (j - c);
}

// Global row of owner r's local row i under the metadata's policy: the
// dual-chunk-swap map above, or r n + i under packed-contiguous (n = T / W).
__device__ __forceinline__ int64_t owner_global_row(int32_t policy, int32_t r, int64_t i, int64_t n,
                                                    int32_t W, int32_t B, const int32_t* cu,
                                                    const int32_t* lcu) {
  return policy == CP_POLICY_DUAL_CHUNK_SWAP ? dcs_global_row(r, i, W, B, cu, lcu) : (int64_t)r * n + i;
}

}  // namespace cpthd
