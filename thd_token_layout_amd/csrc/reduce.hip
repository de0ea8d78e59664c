// Owner-side reductions and the writer/owner epoch protocol.
//
// "Add stream-ordered CP gradient return primitive", sections "Description"
// and "Sequence Diagram": every writer scatters its global dK/dV into the
// owners' slots [owner][writer], publishes an epoch to every owner, each owner
// waits until all of its epoch entries are >= epoch, then accumulates slots
// 0..cp_size-1 into its dK/dV.  The sum here is fixed-order fp32: the
// accumulator starts as slot 0 (widened exactly) and each further slot is added
// once, in writer order; the result is rounded once to the output type
// (bf16: round-to-nearest-even on the bit pattern, NaN kept quiet with its sign).
//
// On one GPU the writers' and owners' streams share one HBM; an epoch store is
// an agent-scope release store, the wait is a bounded spin with agent-scope
// acquire loads (gfx950 has one L2 per XCD, so plain loads could stay stale).
//
// Design: HBM-bound streaming.  A thread handles units of 8 elements (16 B of
// bf16, 32 B of fp32 per slot), issues the loads of a batch of WB slots before
// adding them in order, and writes 16-byte vectors with non-temporal stores.
#include "cpthd_internal.h"

#include <mutex>

namespace cpthd {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ float bf16_bits_to_f32(unsigned int bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits; NaN becomes a quiet NaN, sign kept.
__device__ __forceinline__ unsigned int f32_to_bf16_bits(float f) {
  const unsigned int u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x0040u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---- 8-element units -------------------------------------------------------
struct F8 {
  float v[8];
};

template <int IN>  // IN: CP_F32 or CP_BF16
__device__ __forceinline__ void load_unit(F8& x, const char* base, int64_t unit) {
  if constexpr (IN == CP_F32) {
    const u32x4* p = reinterpret_cast<const u32x4*>(base) + 2 * unit;
    const u32x4 a = __builtin_nontemporal_load(p);
    const u32x4 b = __builtin_nontemporal_load(p + 1);
    x.v[0] = __uint_as_float(a.x); x.v[1] = __uint_as_float(a.y);
    x.v[2] = __uint_as_float(a.z); x.v[3] = __uint_as_float(a.w);
    x.v[4] = __uint_as_float(b.x); x.v[5] = __uint_as_float(b.y);
    x.v[6] = __uint_as_float(b.z); x.v[7] = __uint_as_float(b.w);
  } else {
    const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base) + unit);
    const unsigned int w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x.v[2 * k] = bf16_bits_to_f32(w[k] & 0xFFFFu);
      x.v[2 * k + 1] = bf16_bits_to_f32(w[k] >> 16);
    }
  }
}

template <int OUT>
__device__ __forceinline__ void store_unit(char* base, int64_t unit, const F8& x) {
  if constexpr (OUT == CP_F32) {
    u32x4* p = reinterpret_cast<u32x4*>(base) + 2 * unit;
    u32x4 a, b;
    a.x = __float_as_uint(x.v[0]); a.y = __float_as_uint(x.v[1]);
    a.z = __float_as_uint(x.v[2]); a.w = __float_as_uint(x.v[3]);
    b.x = __float_as_uint(x.v[4]); b.y = __float_as_uint(x.v[5]);
    b.z = __float_as_uint(x.v[6]); b.w = __float_as_uint(x.v[7]);
    __builtin_nontemporal_store(a, p);
    __builtin_nontemporal_store(b, p + 1);
  } else {
    u32x4 a;
    a.x = f32_to_bf16_bits(x.v[0]) | (f32_to_bf16_bits(x.v[1]) << 16);
    a.y = f32_to_bf16_bits(x.v[2]) | (f32_to_bf16_bits(x.v[3]) << 16);
    a.z = f32_to_bf16_bits(x.v[4]) | (f32_to_bf16_bits(x.v[5]) << 16);
    a.w = f32_to_bf16_bits(x.v[6]) | (f32_to_bf16_bits(x.v[7]) << 16);
    __builtin_nontemporal_store(a, reinterpret_cast<u32x4*>(base) + unit);
  }
}

// Scalar element access (unaligned / tail path).
template <int IN>
__device__ __forceinline__ float load_elem(const char* base, int64_t k) {
  if constexpr (IN == CP_F32) return reinterpret_cast<const float*>(base)[k];
  else return bf16_bits_to_f32(reinterpret_cast<const unsigned short*>(base)[k]);
}
template <int OUT>
__device__ __forceinline__ void store_elem(char* base, int64_t k, float f) {
  if constexpr (OUT == CP_F32) reinterpret_cast<float*>(base)[k] = f;
  else reinterpret_cast<unsigned short*>(base)[k] = (unsigned short)f32_to_bf16_bits(f);
}

// Sum one 8-element unit over slots 0..W-1 in order: batches of WB loads in
// flight, then the adds of that batch in slot order.  `in` is the kernel
// argument table (uniform), `off` a byte offset applied to every slot.
template <int IN, int WB>
__device__ __forceinline__ void sum_unit(F8& acc, const ConstRankPtrs& in, int W, int64_t off,
                                         int64_t unit) {
  {
    F8 x[WB];
#pragma unroll
    for (int w = 0; w < WB; ++w)
      if (w < W) load_unit<IN>(x[w], in.p[w] + off, unit);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc.v[e] = x[0].v[e];
#pragma unroll
    for (int w = 1; w < WB; ++w)
      if (w < W) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc.v[e] = acc.v[e] + x[w].v[e];
      }
  }
  for (int w0 = WB; w0 < W; w0 += WB) {
    F8 x[WB];
#pragma unroll
    for (int w = 0; w < WB; ++w)
      if (w0 + w < W) load_unit<IN>(x[w], in.p[w0 + w] + off, unit);
#pragma unroll
    for (int w = 0; w < WB; ++w)
      if (w0 + w < W) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc.v[e] = acc.v[e] + x[w].v[e];
      }
  }
}

__device__ __forceinline__ bool grad_meta_ok(cp_meta_header* h, int64_t T, int32_t W) {
  int code = 0;
  if (h->magic != CP_META_MAGIC) code = CP_CALL_BAD_MAGIC;
  else if (h->flags & CP_META_BUILD_MASK) code = CP_CALL_USED_INVALID_META;
  else if (h->total_tokens != T) code = CP_CALL_TOKENS_MISMATCH;
  else if (h->cp_size != W) code = CP_CALL_CP_SIZE_MISMATCH;
  else if (h->policy != CP_POLICY_DUAL_CHUNK_SWAP) code = CP_CALL_POLICY_MISMATCH;
  if (code != 0 && blockIdx.x == 0 && threadIdx.x == 0) atomicOr(&h->flags, code);
  return code == 0;
}

// ---- slot sum ----------------------------------------------------------------
template <int IN, int OUT, int WB, bool VEC>
__global__ void __launch_bounds__(kBlock) slot_sum_kernel(SlotSumArgs a) {
  if (a.gate_meta != nullptr) {
    cp_meta_header* h = a.gate_meta;
    if (!grad_meta_ok(h, a.gate_T, a.num_slots)) return;
    if (a.owner >= 0 && ((h->wait_timeout_ranks >> a.owner) & 1ull)) return;
  }
  const int W = a.num_slots;
  const int64_t gtid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const int64_t gstride = (int64_t)gridDim.x * kBlock;
  int64_t done = 0;
  if constexpr (VEC) {
    const int64_t nunits = a.n_elems / 8;
    for (int64_t u = gtid; u < nunits; u += gstride) {
      F8 acc;
      sum_unit<IN, WB>(acc, a.in, W, 0, u);
      store_unit<OUT>(a.out, u, acc);
    }
    done = nunits * 8;
  }
  for (int64_t k = done + gtid; k < a.n_elems; k += gstride) {
    float acc = load_elem<IN>(a.in.p[0], k);
    for (int w = 1; w < W; ++w) acc = acc + load_elem<IN>(a.in.p[w], k);
    store_elem<OUT>(a.out, k, acc);
  }
}

// ---- fused scatter + sum ---------------------------------------------------
// Same row map as the permutation engine, restricted to dual-chunk-swap.
struct DocCursor {
  int32_t r;
  int64_t i, lstart, lend, gstart, c;
  int32_t b;
};

__device__ __forceinline__ void doc_load(DocCursor& k, const int32_t* cu, const int32_t* lcu) {
  k.lstart = lcu[k.b];
  k.lend = lcu[k.b + 1];
  k.gstart = cu[k.b];
  k.c = (k.lend - k.lstart) >> 1;
}

__device__ __forceinline__ int64_t owner_row_to_global(int32_t o, int64_t i, int32_t W, int32_t B,
                                                       const int32_t* cu, const int32_t* lcu) {
  DocCursor k;
  k.r = o;
  k.i = i;
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)lcu[mid] <= i) lo = mid; else hi = mid - 1;
  }
  k.b = lo;
  doc_load(k, cu, lcu);
  const int64_t j = i - k.lstart;
  return j < k.c ? k.gstart + (int64_t)o * k.c + j
                 : k.gstart + (int64_t)(2 * W - 1 - o) * k.c + (j - k.c);
}

template <int IN, int OUT, int WB, bool VEC>
__global__ void __launch_bounds__(kBlock) fused_kernel(FusedArgs a) {
  cp_meta_header* h = a.meta;
  if (!grad_meta_ok(h, a.total_tokens, a.cp_size)) return;
  const int32_t W = a.cp_size;
  const int32_t B = h->num_docs;
  const int64_t n = h->local_tokens;
  const int32_t* cu = reinterpret_cast<const int32_t*>(reinterpret_cast<const char*>(h) + 64);
  const int32_t* lcu = cu + (B + 1);
  const int in_bytes = IN == CP_F32 ? 4 : 2;
  const int out_bytes = OUT == CP_F32 ? 4 : 2;

  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * kWavesPerBlock + uniform(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
  const int64_t rows = (int64_t)(a.owner_end - a.owner_begin) * n;

  for (int64_t q = wave; q < rows; q += nwaves) {
    const int32_t o = a.owner_begin + (int32_t)(q / n);
    const int64_t i = q - (int64_t)(o - a.owner_begin) * n;
    const int64_t g = owner_row_to_global(o, i, W, B, cu, lcu);
    const int64_t src_off = g * a.row_elems * in_bytes;  // same row in every writer's view
    char* row_dst = a.out.p[o] + i * a.row_elems * out_bytes;
    if constexpr (VEC) {
      const int64_t units = a.row_elems / 8;
      for (int64_t u = lane; u < units; u += 64) {
        F8 acc;
        sum_unit<IN, WB>(acc, a.grads, W, src_off, u);
        store_unit<OUT>(row_dst, u, acc);
      }
    } else {
      for (int64_t k = lane; k < a.row_elems; k += 64) {
        float acc = load_elem<IN>(a.grads.p[0] + src_off, k);
        for (int w = 1; w < W; ++w) acc = acc + load_elem<IN>(a.grads.p[w] + src_off, k);
        store_elem<OUT>(row_dst, k, acc);
      }
    }
  }
}

// ---- epochs -------------------------------------------------------------------
__global__ void epoch_publish_kernel(uint32_t* epochs, int32_t W, int32_t writer, uint32_t epoch) {
  const int t = threadIdx.x;
  if (writer >= 0) {
    for (int o = t; o < W; o += blockDim.x)
      __hip_atomic_store(&epochs[o * W + writer], epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    for (int k = t; k < W * W; k += blockDim.x)
      __hip_atomic_store(&epochs[k], epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// One wave.  Every lane checks some (owner, writer) entries; the wave ORs the
// pending-owner masks.  The loop always ends: when all entries are ready or
// when the wall clock passes the limit.
__global__ void __launch_bounds__(64)
epoch_wait_kernel(const uint32_t* epochs, int32_t W, int32_t owner, uint32_t epoch,
                  int64_t timeout_ticks, cp_meta_header* h) {
  const int lane = threadIdx.x;
  const int o_begin = owner >= 0 ? owner : 0;
  const int o_count = owner >= 0 ? 1 : W;
  const int64_t start = wall_clock64();
  unsigned long long pending;
  while (true) {
    pending = 0;
    for (int k = lane; k < o_count * W; k += 64) {
      const int o = o_begin + k / W;
      const int w = k - (k / W) * W;
      const uint32_t v = __hip_atomic_load(&epochs[o * W + w], __ATOMIC_ACQUIRE,
                                           __HIP_MEMORY_SCOPE_AGENT);
      if (v < epoch) pending |= 1ull << o;
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) pending |= __shfl_xor(pending, s, 64);
    if (pending == 0) break;
    if (wall_clock64() - start > timeout_ticks) break;
    __builtin_amdgcn_s_sleep(16);
  }
  if (lane == 0) {
    if (owner >= 0) {
      const unsigned long long bit = 1ull << owner;
      if (pending) __hip_atomic_fetch_or(&h->wait_timeout_ranks, bit, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
      else __hip_atomic_fetch_and(&h->wait_timeout_ranks, ~bit, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
    } else {
      __hip_atomic_store(&h->wait_timeout_ranks, pending, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---- dispatch -------------------------------------------------------------------
template <typename K>
int occupancy(K fn, int* cache, std::mutex& m) {
  std::lock_guard<std::mutex> lock(m);
  if (*cache == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, kBlock, 0) != hipSuccess || nb < 1) nb = 1;
    *cache = nb;
  }
  return *cache;
}

std::mutex g_mutex;


template <int IN, int OUT>
struct SumTable {
  void (*fn[2][4])(SlotSumArgs);
  int occ[2][4];
  const char* name[2][4];
};

#define CP_SUM_ROW(IN, OUT, VEC, TAG)                                                        \
  {slot_sum_kernel<IN, OUT, 1, VEC>, slot_sum_kernel<IN, OUT, 2, VEC>,                      \
   slot_sum_kernel<IN, OUT, 4, VEC>, slot_sum_kernel<IN, OUT, 8, VEC>}

#define CP_SUM_NAMES(TAG, VEC)                                                               \
  {"slot_sum<" TAG ",1," VEC ">", "slot_sum<" TAG ",2," VEC ">", "slot_sum<" TAG ",4," VEC ">", \
   "slot_sum<" TAG ",8," VEC ">"}

SumTable<CP_F32, CP_F32> g_sum_ff = {{CP_SUM_ROW(CP_F32, CP_F32, false, ""),
                                      CP_SUM_ROW(CP_F32, CP_F32, true, "")},
                                     {{0}},
                                     {CP_SUM_NAMES("f32,f32", "s"), CP_SUM_NAMES("f32,f32", "v")}};
SumTable<CP_F32, CP_BF16> g_sum_fb = {{CP_SUM_ROW(CP_F32, CP_BF16, false, ""),
                                       CP_SUM_ROW(CP_F32, CP_BF16, true, "")},
                                      {{0}},
                                      {CP_SUM_NAMES("f32,bf16", "s"), CP_SUM_NAMES("f32,bf16", "v")}};
SumTable<CP_BF16, CP_BF16> g_sum_bb = {{CP_SUM_ROW(CP_BF16, CP_BF16, false, ""),
                                        CP_SUM_ROW(CP_BF16, CP_BF16, true, "")},
                                       {{0}},
                                       {CP_SUM_NAMES("bf16,bf16", "s"), CP_SUM_NAMES("bf16,bf16", "v")}};
SumTable<CP_BF16, CP_F32> g_sum_bf = {{CP_SUM_ROW(CP_BF16, CP_F32, false, ""),
                                       CP_SUM_ROW(CP_BF16, CP_F32, true, "")},
                                      {{0}},
                                      {CP_SUM_NAMES("bf16,f32", "s"), CP_SUM_NAMES("bf16,f32", "v")}};

template <int IN, int OUT>
struct FusedTable {
  void (*fn[2][4])(FusedArgs);
  int occ[2][4];
  const char* name[2][4];
};

#define CP_FUSED_ROW(IN, OUT, VEC)                                                           \
  {fused_kernel<IN, OUT, 1, VEC>, fused_kernel<IN, OUT, 2, VEC>, fused_kernel<IN, OUT, 4, VEC>, \
   fused_kernel<IN, OUT, 8, VEC>}
#define CP_FUSED_NAMES(TAG, VEC)                                                             \
  {"fused_grad_return<" TAG ",1," VEC ">", "fused_grad_return<" TAG ",2," VEC ">",            \
   "fused_grad_return<" TAG ",4," VEC ">", "fused_grad_return<" TAG ",8," VEC ">"}

FusedTable<CP_F32, CP_F32> g_fused_ff = {{CP_FUSED_ROW(CP_F32, CP_F32, false),
                                          CP_FUSED_ROW(CP_F32, CP_F32, true)},
                                         {{0}},
                                         {CP_FUSED_NAMES("f32,f32", "s"), CP_FUSED_NAMES("f32,f32", "v")}};
FusedTable<CP_F32, CP_BF16> g_fused_fb = {{CP_FUSED_ROW(CP_F32, CP_BF16, false),
                                          CP_FUSED_ROW(CP_F32, CP_BF16, true)},
                                         {{0}},
                                         {CP_FUSED_NAMES("f32,bf16", "s"), CP_FUSED_NAMES("f32,bf16", "v")}};
FusedTable<CP_BF16, CP_BF16> g_fused_bb = {{CP_FUSED_ROW(CP_BF16, CP_BF16, false),
                                            CP_FUSED_ROW(CP_BF16, CP_BF16, true)},
                                           {{0}},
                                           {CP_FUSED_NAMES("bf16,bf16", "s"),
                                            CP_FUSED_NAMES("bf16,bf16", "v")}};
FusedTable<CP_BF16, CP_F32> g_fused_bf = {{CP_FUSED_ROW(CP_BF16, CP_F32, false),
                                           CP_FUSED_ROW(CP_BF16, CP_F32, true)},
                                          {{0}},
                                          {CP_FUSED_NAMES("bf16,f32", "s"),
                                           CP_FUSED_NAMES("bf16,f32", "v")}};

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

template <typename Table, typename Args>
hipError_t run_sum(Table& tab, const Args& ka, bool vec, int W, int64_t n_elems, hipStream_t stream) {
  const int v = vec ? 1 : 0;
  const int wi = W <= 1 ? 0 : W <= 2 ? 1 : W <= 4 ? 2 : 3;
  const int occ = occupancy(tab.fn[v][wi], &tab.occ[v][wi], g_mutex);
  const int64_t work = vec ? (n_elems / 8 + (n_elems % 8)) : n_elems;
  int64_t want = (work + kBlock - 1) / kBlock;
  const int64_t cap = (int64_t)device_cu_count() * occ;
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  profile_before(tab.name[v][wi], stream);
  hipLaunchKernelGGL(tab.fn[v][wi], dim3((unsigned)want), dim3(kBlock), 0, stream, ka);
  hipError_t e = hipGetLastError();
  profile_after(stream);
  return e;
}

template <typename Table>
hipError_t run_fused(Table& tab, const FusedArgs& a, bool vec, hipStream_t stream) {
  const int v = vec ? 1 : 0;
  const int W = a.cp_size;
  const int wi = W <= 1 ? 0 : W <= 2 ? 1 : W <= 4 ? 2 : 3;
  const int occ = occupancy(tab.fn[v][wi], &tab.occ[v][wi], g_mutex);
  const int64_t rows = (int64_t)(a.owner_end - a.owner_begin) * (a.total_tokens / W);
  int64_t want = (rows + kWavesPerBlock - 1) / kWavesPerBlock;
  const int64_t cap = (int64_t)device_cu_count() * occ;
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  profile_before(tab.name[v][wi], stream);
  hipLaunchKernelGGL(tab.fn[v][wi], dim3((unsigned)want), dim3(kBlock), 0, stream, a);
  hipError_t e = hipGetLastError();
  profile_after(stream);
  return e;
}

}  // namespace

hipError_t launch_slot_sum(const SlotSumArgs& a, hipStream_t stream) {
  if (a.n_elems == 0) return hipSuccess;
  bool vec = aligned16(a.out);
  for (int w = 0; w < a.num_slots; ++w) vec = vec && aligned16(a.in.p[w]);
  if (a.in_dtype == CP_F32 && a.out_dtype == CP_F32) return run_sum(g_sum_ff, a, vec, a.num_slots, a.n_elems, stream);
  if (a.in_dtype == CP_F32 && a.out_dtype == CP_BF16) return run_sum(g_sum_fb, a, vec, a.num_slots, a.n_elems, stream);
  if (a.in_dtype == CP_BF16 && a.out_dtype == CP_BF16) return run_sum(g_sum_bb, a, vec, a.num_slots, a.n_elems, stream);
  if (a.in_dtype == CP_BF16 && a.out_dtype == CP_F32) return run_sum(g_sum_bf, a, vec, a.num_slots, a.n_elems, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_fused(const FusedArgs& a, hipStream_t stream) {
  if (a.total_tokens == 0 || a.row_elems == 0 || a.owner_end <= a.owner_begin) return hipSuccess;
  const int in_b = a.in_dtype == CP_F32 ? 4 : 2;
  const int out_b = a.out_dtype == CP_F32 ? 4 : 2;
  bool vec = a.row_elems % 8 == 0 && (a.row_elems * in_b) % 16 == 0 && (a.row_elems * out_b) % 16 == 0;
  for (int w = 0; w < a.cp_size; ++w) vec = vec && aligned16(a.grads.p[w]);
  for (int o = a.owner_begin; o < a.owner_end; ++o) vec = vec && aligned16(a.out.p[o]);
  if (a.in_dtype == CP_F32 && a.out_dtype == CP_F32) return run_fused(g_fused_ff, a, vec, stream);
  if (a.in_dtype == CP_F32 && a.out_dtype == CP_BF16) return run_fused(g_fused_fb, a, vec, stream);
  if (a.in_dtype == CP_BF16 && a.out_dtype == CP_BF16) return run_fused(g_fused_bb, a, vec, stream);
  if (a.in_dtype == CP_BF16 && a.out_dtype == CP_F32) return run_fused(g_fused_bf, a, vec, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_epoch_publish(uint32_t* epochs, int32_t W, int32_t writer, uint32_t epoch,
                                hipStream_t stream) {
  profile_before("epoch_publish", stream);
  hipLaunchKernelGGL(epoch_publish_kernel, dim3(1), dim3(kBlock), 0, stream, epochs, W, writer, epoch);
  hipError_t e = hipGetLastError();
  profile_after(stream);
  return e;
}

hipError_t launch_epoch_wait(const uint32_t* epochs, int32_t W, int32_t owner, uint32_t epoch,
                             int64_t timeout_ticks, cp_meta_header* meta, hipStream_t stream) {
  profile_before("epoch_wait", stream);
  hipLaunchKernelGGL(epoch_wait_kernel, dim3(1), dim3(64), 0, stream, epochs, W, owner, epoch,
                     timeout_ticks, meta);
  hipError_t e = hipGetLastError();
  profile_after(stream);
  return e;
}

}  // namespace cpthd
