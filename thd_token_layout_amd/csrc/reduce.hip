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
// In the accumulate mode the accumulator starts from the owner's current value
// (widened) and slots 0..cp_size-1 are all added, one at a time, in order.
// The owner's rows follow the metadata's policy (two-chunk layout under
// dual-chunk-swap, the contiguous slice under packed-contiguous).
//
// On one GPU the writers' and owners' streams share one HBM; an epoch store is
// an agent-scope release store, the wait is a bounded spin with agent-scope
// acquire loads (gfx950 has one L2 per XCD, so plain loads could stay stale).
//
// Design: HBM-bound streaming.  A thread handles units of 8 elements (laid out
// so that every wave instruction touches one contiguous span, see below),
// issues the loads of a batch of WB slots before adding them in order, and
// writes with non-temporal stores.
// Launches cover all work with one small contiguous tile per workgroup (a full
// grid rather than a resident-capacity persistent loop, which streams HBM less
// contiguously and measured slower on MI355X).
#include "device_common.h"

#include <atomic>
#include <string>
#include <type_traits>


namespace cpthd {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

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
// Element layout of unit u.  Contiguous (bf16 -> bf16): elements [8u, 8u+8),
// one 16-byte access per lane.  Split (whenever fp32 data is involved): units
// come in groups of 64, and unit u = 64g + l holds the pieces
// [512g + 4l, +4) and [512g + 256 + 4l, +4), so each load or store instruction
// of a wave covers one contiguous span of 64 pieces (16 B per lane for fp32,
// 8 B for bf16).  With 32 contiguous bytes per lane instead, every store
// instruction half-filled each cache line: measured 8-10% extra HBM write
// traffic.  The split layout needs whole groups: 512 elements.
struct F8 {
  float v[8];
};

template <int IN, int OUT>
constexpr bool split_layout() { return IN == CP_F32 || OUT == CP_F32; }
template <int IN, int OUT>
constexpr int64_t unit_group_elems() { return split_layout<IN, OUT>() ? 512 : 8; }

__device__ __forceinline__ int64_t split_piece(int64_t unit) { return (unit >> 6) * 128 + (unit & 63); }

__device__ __forceinline__ void bf16x4_to_f32(float* v, u32x2 w) {
  v[0] = bf16_bits_to_f32(w.x & 0xFFFFu);
  v[1] = bf16_bits_to_f32(w.x >> 16);
  v[2] = bf16_bits_to_f32(w.y & 0xFFFFu);
  v[3] = bf16_bits_to_f32(w.y >> 16);
}

__device__ __forceinline__ void f32x4_from(float* v, u32x4 a) {
  v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
  v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
}

template <int IN, bool SPLIT>
__device__ __forceinline__ void load_unit(F8& x, const char* base, int64_t unit) {
  if constexpr (SPLIT) {
    const int64_t p0 = split_piece(unit);
    if constexpr (IN == CP_F32) {
      const u32x4* p = reinterpret_cast<const u32x4*>(base);
      f32x4_from(x.v, __builtin_nontemporal_load(p + p0));
      f32x4_from(x.v + 4, __builtin_nontemporal_load(p + p0 + 64));
    } else {
      const u32x2* p = reinterpret_cast<const u32x2*>(base);
      bf16x4_to_f32(x.v, __builtin_nontemporal_load(p + p0));
      bf16x4_to_f32(x.v + 4, __builtin_nontemporal_load(p + p0 + 64));
    }
  } else {
    static_assert(IN == CP_BF16, "the contiguous layout is bf16 only");
    const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base) + unit);
    bf16x4_to_f32(x.v, u32x2{a.x, a.y});
    bf16x4_to_f32(x.v + 4, u32x2{a.z, a.w});
  }
}

__device__ __forceinline__ u32x4 f32x4_bits(const float* v) {
  return u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
               __float_as_uint(v[3])};
}
__device__ __forceinline__ u32x2 bf16x4_bits(const float* v) {
  return u32x2{f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16),
               f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16)};
}

template <int OUT, bool SPLIT>
__device__ __forceinline__ void store_unit(char* base, int64_t unit, const F8& x) {
  if constexpr (SPLIT) {
    const int64_t p0 = split_piece(unit);
    if constexpr (OUT == CP_F32) {
      u32x4* p = reinterpret_cast<u32x4*>(base);
      __builtin_nontemporal_store(f32x4_bits(x.v), p + p0);
      __builtin_nontemporal_store(f32x4_bits(x.v + 4), p + p0 + 64);
    } else {
      u32x2* p = reinterpret_cast<u32x2*>(base);
      __builtin_nontemporal_store(bf16x4_bits(x.v), p + p0);
      __builtin_nontemporal_store(bf16x4_bits(x.v + 4), p + p0 + 64);
    }
  } else {
    static_assert(OUT == CP_BF16, "the contiguous layout is bf16 only");
    const u32x2 lo = bf16x4_bits(x.v), hi = bf16x4_bits(x.v + 4);
    __builtin_nontemporal_store(u32x4{lo.x, lo.y, hi.x, hi.y}, reinterpret_cast<u32x4*>(base) + unit);
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

// Sum UPT 8-element units over slots 0..W-1 in order.  The loads of a batch
// of WB slots (for all UPT units) are issued before that batch's adds, which
// then run in slot order.  `in` is the kernel argument table (uniform), off[u]
// a byte offset applied to every slot for unit u, ok[u] masks units past the end.
// Without ACC the accumulator is seeded with slot 0; with ACC the caller has
// seeded it (with the owner's current values) and every slot is added.
template <int IN, bool SPLIT, int WB, int UPT, bool ACC>
__device__ __forceinline__ void sum_units(F8 (&acc)[UPT], const ConstRankPtrs& in, int W,
                                          const int64_t (&off)[UPT], const int64_t (&unit)[UPT],
                                          const bool (&ok)[UPT]) {
  {
    F8 x[UPT][WB];
#pragma unroll
    for (int u = 0; u < UPT; ++u)
#pragma unroll
      for (int w = 0; w < WB; ++w)
        if (ok[u] && w < W) load_unit<IN, SPLIT>(x[u][w], in.p[w] + off[u], unit[u]);
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      if constexpr (ACC) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[u].v[e] = acc[u].v[e] + x[u][0].v[e];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[u].v[e] = x[u][0].v[e];
      }
#pragma unroll
      for (int w = 1; w < WB; ++w)
        if (w < W) {
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[u].v[e] = acc[u].v[e] + x[u][w].v[e];
        }
    }
  }
  for (int w0 = WB; w0 < W; w0 += WB) {
    F8 x[UPT][WB];
#pragma unroll
    for (int u = 0; u < UPT; ++u)
#pragma unroll
      for (int w = 0; w < WB; ++w)
        if (ok[u] && w0 + w < W) load_unit<IN, SPLIT>(x[u][w], in.p[w0 + w] + off[u], unit[u]);
#pragma unroll
    for (int u = 0; u < UPT; ++u)
#pragma unroll
      for (int w = 0; w < WB; ++w)
        if (w0 + w < W) {
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[u].v[e] = acc[u].v[e] + x[u][w].v[e];
        }
  }
}

// Seed of the accumulate mode: the owner's current values, widened to fp32.
template <int OUT, bool SPLIT, int UPT>
__device__ __forceinline__ void seed_units(F8 (&acc)[UPT], const char* out, const int64_t (&unit)[UPT],
                                           const bool (&ok)[UPT]) {
#pragma unroll
  for (int u = 0; u < UPT; ++u)
    if (ok[u]) load_unit<OUT, SPLIT>(acc[u], out, unit[u]);
}

// Gradient-return kernels need metadata built for W ranks and T tokens (either
// policy: the owner's rows are those the partition gives it).
__device__ __forceinline__ bool grad_meta_ok(cp_meta_header* h, int64_t T, int32_t W) {
  return meta_ok(h, T, W, -1);
}

// ---- slot sum ----------------------------------------------------------------
// A workgroup owns a tile of kBlock*UPT consecutive 8-element units; thread t
// takes units t, t + kBlock, ... of the tile (coalesced per load instruction).
template <int IN, int OUT, int WB, bool VEC, int UPT, bool ACC>
__global__ void __launch_bounds__(kBlock) slot_sum_kernel(SlotSumArgs a) {
  if (a.gate_meta != nullptr) {
    cp_meta_header* h = a.gate_meta;
    if (!grad_meta_ok(h, a.gate_T, a.num_slots)) return;
    if (a.owner >= 0 && ((h->wait_timeout_ranks >> a.owner) & 1ull)) return;
  }
  const int W = a.num_slots;
  constexpr bool SPLIT = split_layout<IN, OUT>();
  int64_t done = 0;
  if constexpr (VEC) {
    const int64_t nunits = a.n_elems / unit_group_elems<IN, OUT>() * (unit_group_elems<IN, OUT>() / 8);
    const int64_t ntiles = (nunits + (int64_t)kBlock * UPT - 1) / ((int64_t)kBlock * UPT);
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
      int64_t unit[UPT], off[UPT];
      bool ok[UPT];
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
        unit[u] = tile * kBlock * UPT + (int64_t)u * kBlock + threadIdx.x;
        ok[u] = unit[u] < nunits;
        off[u] = 0;
      }
      F8 acc[UPT];
      if constexpr (ACC) seed_units<OUT, SPLIT, UPT>(acc, a.out, unit, ok);
      sum_units<IN, SPLIT, WB, UPT, ACC>(acc, a.in, W, off, unit, ok);
#pragma unroll
      for (int u = 0; u < UPT; ++u)
        if (ok[u]) store_unit<OUT, SPLIT>(a.out, unit[u], acc[u]);
    }
    done = nunits * 8;
  }
  const int64_t gtid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const int64_t gstride = (int64_t)gridDim.x * kBlock;
  for (int64_t k = done + gtid; k < a.n_elems; k += gstride) {
    float acc = ACC ? load_elem<OUT>(a.out, k) + load_elem<IN>(a.in.p[0], k) : load_elem<IN>(a.in.p[0], k);
    for (int w = 1; w < W; ++w) acc = acc + load_elem<IN>(a.in.p[w], k);
    store_elem<OUT>(a.out, k, acc);
  }
}

// ---- fused scatter + sum ---------------------------------------------------
// Owner o's local row i reads global row owner_global_row(o, i) of every writer.

// A workgroup owns (4 / WPR) output rows; WPR waves share a row, each taking
// column passes of 64*UPL units (8 elements each) so a lane has UPL*W loads in
// flight per pass.
template <int IN, int OUT, int WB, bool VEC, int WPR, int UPL, bool ACC>
__global__ void __launch_bounds__(kBlock) fused_kernel(FusedArgs a) {
  constexpr int kRowsPerTile = kWavesPerBlock / WPR;
  cp_meta_header* h = a.meta;
  if (!grad_meta_ok(h, a.total_tokens, a.cp_size)) return;
  const int32_t W = a.cp_size;
  const int32_t B = h->num_docs;
  const int64_t n = h->local_tokens;
  const int32_t* cu = meta_cu(h);
  const int32_t* lcu = meta_local_cu0(h);
  const int in_bytes = IN == CP_F32 ? 4 : 2;
  const int out_bytes = OUT == CP_F32 ? 4 : 2;

  const int lane = threadIdx.x & 63;
  const int wave = wave_uniform(threadIdx.x >> 6);
  const int row_slot = wave / WPR;
  const int chunk = wave % WPR;
  const int64_t rows = (int64_t)(a.owner_end - a.owner_begin) * n;
  const int64_t ntiles = (rows + kRowsPerTile - 1) / kRowsPerTile;

  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t q = tile * kRowsPerTile + row_slot;
    if (q >= rows) continue;
    const int32_t o = a.owner_begin + (int32_t)(q / n);
    const int64_t i = q - (int64_t)(o - a.owner_begin) * n;
    const int64_t g = owner_global_row(h->policy, o, i, n, W, B, cu, lcu);
    const int64_t src_off = g * a.row_elems * in_bytes;  // same row in every writer's view
    char* row_dst = a.out.p[o] + i * a.row_elems * out_bytes;
    if constexpr (VEC) {
      const int64_t units = a.row_elems / 8;
      for (int64_t cb = (int64_t)chunk * 64 * UPL; cb < units; cb += (int64_t)WPR * 64 * UPL) {
        int64_t unit[UPL], off[UPL];
        bool ok[UPL];
#pragma unroll
        for (int m = 0; m < UPL; ++m) {
          unit[m] = cb + lane + 64 * m;
          ok[m] = unit[m] < units;
          off[m] = src_off;
        }
        F8 acc[UPL];
        if constexpr (ACC) seed_units<OUT, split_layout<IN, OUT>(), UPL>(acc, row_dst, unit, ok);
        sum_units<IN, split_layout<IN, OUT>(), WB, UPL, ACC>(acc, a.grads, W, off, unit, ok);
#pragma unroll
        for (int m = 0; m < UPL; ++m)
          if (ok[m]) store_unit<OUT, split_layout<IN, OUT>()>(row_dst, unit[m], acc[m]);
      }
    } else if (chunk == 0) {
      for (int64_t k = lane; k < a.row_elems; k += 64) {
        float acc = ACC ? load_elem<OUT>(row_dst, k) + load_elem<IN>(a.grads.p[0] + src_off, k)
                        : load_elem<IN>(a.grads.p[0] + src_off, k);
        for (int w = 1; w < W; ++w) acc = acc + load_elem<IN>(a.grads.p[w] + src_off, k);
        store_elem<OUT>(row_dst, k, acc);
      }
    }
  }
}

// Flat-tile variant: the owners' output rows are one flat range of
// rows * units_per_row 8-element units, and a workgroup owns kBlock*NP
// consecutive units of it (a tile may start and end inside a row), so every
// thread does exactly NP units in one pass, as in the slot sum.  The first
// threads look up the source offset and destination of the <= kMaxTileRows
// rows the tile touches and share them through LDS.  The row of a unit is
// found with a multiply-high by `upr_magic` = ceil(2^32 / units_per_row),
// exact while the in-tile offset times units_per_row stays below 2^32.
constexpr int kMaxTileRows = 16;

template <int IN, int OUT, int WB, int NP, bool ACC>
__global__ void __launch_bounds__(kBlock) fused_flat_kernel(FusedArgs a, uint32_t upr_magic) {
  __shared__ int64_t s_src[kMaxTileRows];
  __shared__ char* s_dst[kMaxTileRows];
  cp_meta_header* h = a.meta;
  if (!grad_meta_ok(h, a.total_tokens, a.cp_size)) return;
  const int32_t W = a.cp_size;
  const int32_t B = h->num_docs;
  const int64_t n = h->local_tokens;
  const int32_t* cu = meta_cu(h);
  const int32_t* lcu = meta_local_cu0(h);
  const int in_bytes = IN == CP_F32 ? 4 : 2;
  const int out_bytes = OUT == CP_F32 ? 4 : 2;
  const int64_t upr = a.row_elems / 8;
  const int64_t rows = (int64_t)(a.owner_end - a.owner_begin) * n;
  const int64_t total = rows * upr;
  constexpr int64_t kTileUnits = (int64_t)kBlock * NP;
  const int64_t ntiles = (total + kTileUnits - 1) / kTileUnits;

  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t u0 = tile * kTileUnits;
    const int64_t row0 = u0 / upr;
    const int64_t u_end = u0 + kTileUnits < total ? u0 + kTileUnits : total;
    const int nrows = (int)((u_end - 1) / upr - row0 + 1);
    if ((int)threadIdx.x < nrows) {
      const int64_t q = row0 + threadIdx.x;
      const int32_t o = a.owner_begin + (int32_t)(q / n);
      const int64_t i = q - (int64_t)(o - a.owner_begin) * n;
      s_src[threadIdx.x] = owner_global_row(h->policy, o, i, n, W, B, cu, lcu) * a.row_elems * in_bytes;
      s_dst[threadIdx.x] = a.out.p[o] + i * a.row_elems * out_bytes;
    }
    __syncthreads();
    const int64_t base = u0 - row0 * upr;  // offset of the tile's first unit inside row0
    int64_t unit[NP], off[NP];
    int row[NP];
    bool ok[NP];
#pragma unroll
    for (int m = 0; m < NP; ++m) {
      const uint32_t f = (uint32_t)(base + (int64_t)m * kBlock + threadIdx.x);
      ok[m] = u0 + (int64_t)m * kBlock + threadIdx.x < u_end;
      row[m] = ok[m] ? (int)__umulhi(f, upr_magic) : 0;
      unit[m] = (int64_t)f - (int64_t)row[m] * upr;
      off[m] = s_src[row[m]];
    }
    F8 acc[NP];
    if constexpr (ACC) {
#pragma unroll
      for (int m = 0; m < NP; ++m)
        if (ok[m]) load_unit<OUT, split_layout<IN, OUT>()>(acc[m], s_dst[row[m]], unit[m]);
    }
    sum_units<IN, split_layout<IN, OUT>(), WB, NP, ACC>(acc, a.grads, W, off, unit, ok);
#pragma unroll
    for (int m = 0; m < NP; ++m)
      if (ok[m]) store_unit<OUT, split_layout<IN, OUT>()>(s_dst[row[m]], unit[m], acc[m]);
    __syncthreads();  // s_src / s_dst are rewritten by the next tile
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

// ---- all-reduce: one-shot and ring ---------------------------------------------
// "Low Latency Communication Kernels with NVSHMEM": the all-reduce algorithms
// picked by message size and the exercise comparing a one-shot all-reduce
// with a ring over 1 KB - 16 MB.  One-shot: every rank sums all W buffers
// itself.  Ring: a reduce-scatter then an all-gather, W-1 steps each, every
// rank passing one chunk to rank r+1 per step; partials travel in the buffer
// type, so a bf16 ring rounds after each add.
// All W ranks' buffers sit in this device's HBM; each launch does one step of
// the algorithm for every rank, ranks in blockIdx.y (dispatch runs rank by
// rank, as W devices would each do their own share).

// One-shot: rank r's workgroups sum all W inputs in rank order (seeded with
// input 0, one fp32 add per further input) and write out[r].
template <int T, int WB, bool VEC, int UPT>
__global__ void __launch_bounds__(kBlock) allreduce_one_shot_kernel(AllreduceArgs a) {
  const int W = a.cp_size;
  char* const out = a.out.p[blockIdx.y];
  constexpr bool SPLIT = split_layout<T, T>();
  int64_t done = 0;
  if constexpr (VEC) {
    constexpr int64_t G = unit_group_elems<T, T>();
    const int64_t nunits = a.n_elems / G * (G / 8);
    const int64_t ntiles = (nunits + (int64_t)kBlock * UPT - 1) / ((int64_t)kBlock * UPT);
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
      int64_t unit[UPT], off[UPT];
      bool ok[UPT];
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
        unit[u] = tile * kBlock * UPT + (int64_t)u * kBlock + threadIdx.x;
        ok[u] = unit[u] < nunits;
        off[u] = 0;
      }
      F8 acc[UPT];
      sum_units<T, SPLIT, WB, UPT, false>(acc, a.in, W, off, unit, ok);
#pragma unroll
      for (int u = 0; u < UPT; ++u)
        if (ok[u]) store_unit<T, SPLIT>(out, unit[u], acc[u]);
    }
    done = nunits * 8;
  }
  const int64_t gstride = (int64_t)gridDim.x * kBlock;
  for (int64_t k = done + (int64_t)blockIdx.x * kBlock + threadIdx.x; k < a.n_elems; k += gstride) {
    float acc = load_elem<T>(a.in.p[0], k);
    for (int w = 1; w < W; ++w) acc = acc + load_elem<T>(a.in.p[w], k);
    store_elem<T>(out, k, acc);
  }
}

// Chunk c of the ring: [lo, hi) elements.
__device__ __forceinline__ void ring_chunk(const AllreduceArgs& a, int c, int64_t& lo, int64_t& hi) {
  lo = (int64_t)c * a.chunk;
  hi = lo + a.chunk;
  if (lo > a.n_elems) lo = a.n_elems;
  if (hi > a.n_elems) hi = a.n_elems;
}

// Ring reduce-scatter step: rank r receives chunk c = (r-1-step) mod W from
// rank r-1 (its input at step 0, its working buffer after) and stores
// received + own input, rounded to the buffer type.
template <int T, bool VEC, int UPT>
__global__ void __launch_bounds__(kBlock) ring_reduce_step_kernel(AllreduceArgs a, int32_t step) {
  const int W = a.cp_size;
  const int r = blockIdx.y;
  const int prev = r == 0 ? W - 1 : r - 1;
  const int c = ((r - 1 - step) % W + W) % W;
  int64_t lo, hi;
  ring_chunk(a, c, lo, hi);
  const int64_t len = hi - lo;
  constexpr int64_t eb = T == CP_F32 ? 4 : 2;
  const char* const recv = (step == 0 ? a.in.p[prev] : a.out.p[prev]) + lo * eb;
  const char* const own = a.in.p[r] + lo * eb;
  char* const dst = a.out.p[r] + lo * eb;
  constexpr bool SPLIT = split_layout<T, T>();
  int64_t done = 0;
  if constexpr (VEC) {
    constexpr int64_t G = unit_group_elems<T, T>();
    const int64_t nunits = len / G * (G / 8);
    const int64_t ntiles = (nunits + (int64_t)kBlock * UPT - 1) / ((int64_t)kBlock * UPT);
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
      F8 x[UPT], y[UPT];
      int64_t unit[UPT];
      bool ok[UPT];
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
        unit[u] = tile * kBlock * UPT + (int64_t)u * kBlock + threadIdx.x;
        ok[u] = unit[u] < nunits;
        if (ok[u]) {
          load_unit<T, SPLIT>(x[u], recv, unit[u]);
          load_unit<T, SPLIT>(y[u], own, unit[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < UPT; ++u)
        if (ok[u]) {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[u].v[e] = x[u].v[e] + y[u].v[e];
          store_unit<T, SPLIT>(dst, unit[u], x[u]);
        }
    }
    done = nunits * 8;
  }
  const int64_t gstride = (int64_t)gridDim.x * kBlock;
  for (int64_t k = done + (int64_t)blockIdx.x * kBlock + threadIdx.x; k < len; k += gstride)
    store_elem<T>(dst, k, load_elem<T>(recv, k) + load_elem<T>(own, k));
}

// Ring all-gather step: rank r copies chunk c = (r-step) mod W from rank
// r-1's working buffer, bit for bit.  FROM_IN (one rank): copy the input.
template <int EB, bool VEC, bool FROM_IN>
__global__ void __launch_bounds__(kBlock) ring_gather_step_kernel(AllreduceArgs a, int32_t step) {
  const int W = a.cp_size;
  const int r = blockIdx.y;
  const int prev = r == 0 ? W - 1 : r - 1;
  const int c = ((r - step) % W + W) % W;
  int64_t lo, hi;
  ring_chunk(a, c, lo, hi);
  const char* const src = (FROM_IN ? a.in.p[r] : a.out.p[prev]) + lo * EB;
  char* const dst = a.out.p[r] + lo * EB;
  const int64_t len = hi - lo;
  int64_t done = 0;
  if constexpr (VEC) {
    constexpr int kUpt = 4;  // 16-byte units per thread and tile
    const int64_t n16 = len * EB / 16;
    const int64_t ntiles = (n16 + (int64_t)kBlock * kUpt - 1) / ((int64_t)kBlock * kUpt);
    const u32x4* s16 = reinterpret_cast<const u32x4*>(src);
    u32x4* d16 = reinterpret_cast<u32x4*>(dst);
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
      u32x4 v[kUpt];
      int64_t unit[kUpt];
#pragma unroll
      for (int u = 0; u < kUpt; ++u) {
        unit[u] = tile * kBlock * kUpt + (int64_t)u * kBlock + threadIdx.x;
        if (unit[u] < n16) v[u] = __builtin_nontemporal_load(s16 + unit[u]);
      }
#pragma unroll
      for (int u = 0; u < kUpt; ++u)
        if (unit[u] < n16) __builtin_nontemporal_store(v[u], d16 + unit[u]);
    }
    done = n16 * 16 / EB;
  }
  typedef typename std::conditional<EB == 4, unsigned int, unsigned short>::type E;
  const E* se = reinterpret_cast<const E*>(src);
  E* de = reinterpret_cast<E*>(dst);
  const int64_t gstride = (int64_t)gridDim.x * kBlock;
  for (int64_t k = done + (int64_t)blockIdx.x * kBlock + threadIdx.x; k < len; k += gstride) de[k] = se[k];
}


// The ring in one launch (the persistent, in-kernel-signalling form of the
// pages' design): workgroup (t, r) is rank r's share of tile t of every chunk.
// It runs rank r's W-1 reduce-scatter and W-1 all-gather steps in order; before
// step k > 0 one lane waits until rank r-1's workgroup of the same tile has
// finished k steps, and after each step the workgroup publishes k+1.  Every
// dependency of the ring is within one tile, so tiles proceed independently.
// Data written in a step is made visible at agent scope by the flag store with
// release after a workgroup barrier; the waiter polls with relaxed loads and
// acquires once.  Waits are bounded by the device wall clock; a timeout, or a
// stale epoch (a flag already at or above this call's base), is recorded in the
// status words and every workgroup stops.  The grid is sized to at most half of
// what can be resident at once, so every workgroup a wait depends on runs; a
// cooperative launch would guarantee that too but costs ~20 us on this chip,
// which is more than the whole ring of a small message.
__device__ __forceinline__ void atomic_max_u64(uint64_t* p, uint64_t v) {
  __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int T>
__global__ void __launch_bounds__(kBlock) ring_signal_kernel(AllreduceArgs a, RingSignalArgs g) {
  const int W = a.cp_size;
  const int r = blockIdx.y;
  const int t = blockIdx.x;
  const int prev = r == 0 ? W - 1 : r - 1;
  uint64_t* const words = g.signals;
  uint64_t* const mine = g.signals + 2 + (int64_t)r * kSignalTiles + t;
  const uint64_t* const theirs = g.signals + 2 + (int64_t)prev * kSignalTiles + t;
  const uint64_t base = g.epoch << 8;
  __shared__ int s_go;
  if (threadIdx.x == 0) {
    const uint64_t v = __hip_atomic_load(mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_go = v < base;
    if (!s_go) atomic_max_u64(&words[1], g.epoch);
  }
  __syncthreads();
  if (!s_go) return;
  constexpr int64_t eb = T == CP_F32 ? 4 : 2;
  constexpr bool SPLIT = split_layout<T, T>();
  constexpr int64_t G = unit_group_elems<T, T>();
  // The four buffers this workgroup touches, read once from the argument tables
  // (indexing the tables inside the loop would copy them to scratch memory).
  const char* const in_prev = a.in.p[prev];
  const char* const in_mine = a.in.p[r];
  const char* const out_prev = a.out.p[prev];
  char* const out_mine = a.out.p[r];
  const int64_t n = a.n_elems, chunk = a.chunk;
  const bool vec = a.vec != 0;
  const int steps = 2 * (W - 1);
  for (int k = 0; k < steps; ++k) {
    if (k > 0) {
      if (threadIdx.x == 0) {
        int ok = 1;
        const int64_t start = wall_clock64();
        while (__hip_atomic_load(theirs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < base + (uint64_t)k) {
          if (__hip_atomic_load(&words[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= g.epoch ||
              __hip_atomic_load(&words[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= g.epoch) {
            ok = 0;  // another workgroup has stopped the call
            break;
          }
          if (wall_clock64() - start > g.timeout_ticks) {
            atomic_max_u64(&words[0], g.epoch);
            ok = 0;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        // One acquire for the workgroup: the cache invalidation it implies is
        // cache-wide, and the barrier orders every wave's loads after it.
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        s_go = ok;
      }
      __syncthreads();
      if (!s_go) return;
    }
    const bool reduce = k < W - 1;
    const int s = reduce ? k : k - (W - 1);
    const int c = reduce ? ((r - 1 - s) % W + W) % W : ((r - s) % W + W) % W;
    const int64_t lo = (int64_t)c * chunk < n ? (int64_t)c * chunk : n;
    const int64_t hi = lo + chunk < n ? lo + chunk : n;
    int64_t tlo = lo + (int64_t)t * g.tile_elems;
    if (tlo > hi) tlo = hi;
    int64_t thi = tlo + g.tile_elems;
    if (thi > hi) thi = hi;
    const int64_t len = thi - tlo;
    char* const dst = out_mine + tlo * eb;
    if (reduce) {
      const char* const recv = (s == 0 ? in_prev : out_prev) + tlo * eb;
      const char* const own = in_mine + tlo * eb;
      const int64_t nunits = vec ? len / G * (G / 8) : 0;
      constexpr int kU = 4;  // units in flight per thread
      for (int64_t u0 = threadIdx.x; u0 < nunits; u0 += kBlock * kU) {
        F8 x[kU], y[kU];
#pragma unroll
        for (int m = 0; m < kU; ++m) {
          const int64_t u = u0 + (int64_t)m * kBlock;
          if (u < nunits) {
            load_unit<T, SPLIT>(x[m], recv, u);
            load_unit<T, SPLIT>(y[m], own, u);
          }
        }
#pragma unroll
        for (int m = 0; m < kU; ++m) {
          const int64_t u = u0 + (int64_t)m * kBlock;
          if (u < nunits) {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[m].v[e] = x[m].v[e] + y[m].v[e];
            store_unit<T, SPLIT>(dst, u, x[m]);
          }
        }
      }
      for (int64_t q = nunits * 8 + threadIdx.x; q < len; q += kBlock)
        store_elem<T>(dst, q, load_elem<T>(recv, q) + load_elem<T>(own, q));
    } else {
      const char* const src = out_prev + tlo * eb;
      const int64_t n16 = vec ? len * eb / 16 : 0;
      constexpr int kC = 8;  // 16-byte units in flight per thread
      for (int64_t u0 = threadIdx.x; u0 < n16; u0 += kBlock * kC) {
        u32x4 v[kC];
#pragma unroll
        for (int m = 0; m < kC; ++m) {
          const int64_t u = u0 + (int64_t)m * kBlock;
          if (u < n16) v[m] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + u);
        }
#pragma unroll
        for (int m = 0; m < kC; ++m) {
          const int64_t u = u0 + (int64_t)m * kBlock;
          if (u < n16) __builtin_nontemporal_store(v[m], reinterpret_cast<u32x4*>(dst) + u);
        }
      }
      typedef typename std::conditional<eb == 4, unsigned int, unsigned short>::type E;
      for (int64_t q = n16 * 16 / eb + threadIdx.x; q < len; q += kBlock)
        reinterpret_cast<E*>(dst)[q] = reinterpret_cast<const E*>(src)[q];
    }
    // The barrier completes every wave's stores into this XCD's L2; lane 0's
    // agent-scope release then writes the L2 back before the flag is stored.
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_store(mine, base + (uint64_t)(k + 1), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---- dispatch -------------------------------------------------------------------
bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

const char* dtype_tag(int dt) { return dt == CP_F32 ? "f32" : "bf16"; }

// Tile shapes (units of 8 elements per thread / per lane, waves per row).
// Chosen from a sweep on MI355X; see the kernels' comments.
// At most 8 slots x 8 floats of loaded data per thread and pass: more raises
// register use enough to lower occupancy (a W=8 bf16 sum with 2 units per
// thread measured 25% slower).
constexpr int sum_upt(int wb) { return wb <= 2 ? 4 : wb <= 4 ? 2 : 1; }
constexpr int fused_upl(int wb) { return wb <= 2 ? 2 : 1; }
constexpr int kFusedWpr = 4;
// Fused shapes, from a sweep on the S=262144 (W=4 fp32) and S=131072 (W=8
// bf16) shapes: flat unit tiles, 2 units per thread for W <= 4 (6.20 TB/s,
// against 6.05 for a wave per row), 1 unit per thread above.

template <int IN, int OUT, int WB, bool ACC>
hipError_t launch_sum_wb(const SlotSumArgs& a, bool vec, hipStream_t stream) {
  constexpr int UPT = sum_upt(WB);
  const std::string tag = std::string(ACC ? "slot_sum_acc<" : "slot_sum<") + dtype_tag(IN) + "," +
                          dtype_tag(OUT) + "," + std::to_string(WB) + ",";
  static const std::string names[2] = {tag + "s>", tag + "v" + std::to_string(UPT) + ">"};
  int64_t blocks;
  if (vec) {
    constexpr int64_t G = unit_group_elems<IN, OUT>();
    const int64_t units = a.n_elems / G * (G / 8);
    blocks = (units + (int64_t)kBlock * UPT - 1) / ((int64_t)kBlock * UPT);
    const int64_t tail = a.n_elems - units * 8;  // elements left to the scalar loop
    if (blocks == 0 && tail > 0) blocks = 1;
  } else {
    blocks = (a.n_elems + kBlock - 1) / kBlock;
  }
  if (blocks > kMaxGrid) blocks = kMaxGrid;
  if (blocks < 1) blocks = 1;
  profile_before(names[vec ? 1 : 0].c_str(), stream);
  if (vec)
    hipLaunchKernelGGL((slot_sum_kernel<IN, OUT, WB, true, UPT, ACC>), dim3((unsigned)blocks), dim3(kBlock), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((slot_sum_kernel<IN, OUT, WB, false, 1, ACC>), dim3((unsigned)blocks), dim3(kBlock), 0,
                       stream, a);
  hipError_t e = hipGetLastError();
  profile_after(stream);
  return e;
}

template <int IN, int OUT, bool ACC>
hipError_t launch_sum_acc(const SlotSumArgs& a, bool vec, hipStream_t stream) {
  const int W = a.num_slots;
  if (W <= 1) return launch_sum_wb<IN, OUT, 1, ACC>(a, vec, stream);
  if (W <= 2) return launch_sum_wb<IN, OUT, 2, ACC>(a, vec, stream);
  if (W <= 4) return launch_sum_wb<IN, OUT, 4, ACC>(a, vec, stream);
  return launch_sum_wb<IN, OUT, 8, ACC>(a, vec, stream);
}

template <int IN, int OUT>
hipError_t launch_sum_typed(const SlotSumArgs& a, bool vec, hipStream_t stream) {
  return a.accumulate ? launch_sum_acc<IN, OUT, true>(a, vec, stream)
                      : launch_sum_acc<IN, OUT, false>(a, vec, stream);
}

template <int IN, int OUT, int WB, bool ACC>
hipError_t launch_fused_wb(const FusedArgs& a, bool vec, hipStream_t stream) {
  const std::string tag = std::string(ACC ? "fused_grad_return_acc<" : "fused_grad_return<") + dtype_tag(IN) +
                          "," + dtype_tag(OUT) + "," + std::to_string(WB) + ",";
  static const std::string names[4] = {tag + "s>", tag + "flat1>", tag + "flat2>",
                                       tag + "v" + std::to_string(fused_upl(WB)) + "/" +
                                           std::to_string(kFusedWpr) + ">"};
  vec = vec && a.row_elems % unit_group_elems<IN, OUT>() == 0;  // whole unit groups per row
  const int64_t rows = (int64_t)(a.owner_end - a.owner_begin) * (a.total_tokens / a.cp_size);
  const int64_t upr = a.row_elems / 8;
  const int np = a.cp_size <= 4 ? 2 : 1;
  const int64_t tile_units = (int64_t)kBlock * np;
  // Flat unit tiles need the rows a tile touches to fit kMaxTileRows and
  // (tile units + units_per_row) * units_per_row < 2^32 for the row split.
  const bool flat_ok = upr > 0 && tile_units / upr + 2 <= kMaxTileRows &&
                       (tile_units + upr) * upr < (int64_t(1) << 32);
  // kind 0: scalar; 1, 2: flat unit tiles with NP = 1, 2; 3: 4 waves per row (very long rows)
  const int kind = !vec ? 0 : !flat_ok ? 3 : np;
  int64_t blocks;
  if (kind == 1 || kind == 2) {
    blocks = (rows * upr + tile_units - 1) / tile_units;
  } else {
    const int64_t rows_per_block = kind == 3 ? kWavesPerBlock / kFusedWpr : kWavesPerBlock;
    blocks = (rows + rows_per_block - 1) / rows_per_block;
  }
  if (blocks > kMaxGrid) blocks = kMaxGrid;
  if (blocks < 1) blocks = 1;
  const uint32_t magic = upr > 0 ? (uint32_t)(((uint64_t(1) << 32) + (uint64_t)upr - 1) / (uint64_t)upr) : 0;
  profile_before(names[kind].c_str(), stream);
  if (kind == 1) {
    hipLaunchKernelGGL((fused_flat_kernel<IN, OUT, WB, 1, ACC>), dim3((unsigned)blocks), dim3(kBlock), 0, stream,
                       a, magic);
  } else if (kind == 2) {
    hipLaunchKernelGGL((fused_flat_kernel<IN, OUT, WB, 2, ACC>), dim3((unsigned)blocks), dim3(kBlock), 0, stream,
                       a, magic);
  } else if (kind == 3) {
    hipLaunchKernelGGL((fused_kernel<IN, OUT, WB, true, kFusedWpr, fused_upl(WB), ACC>),
                       dim3((unsigned)blocks), dim3(kBlock), 0, stream, a);
  } else {
    hipLaunchKernelGGL((fused_kernel<IN, OUT, WB, false, 1, 1, ACC>), dim3((unsigned)blocks), dim3(kBlock), 0,
                       stream, a);
  }
  hipError_t e = hipGetLastError();
  profile_after(stream);
  return e;
}

// Writers are summed in batches of at most 4 (W = 8 bf16 measured 6.08 TB/s
// with two batches of 4, 5.03 TB/s with one batch of 8: register pressure).
template <int IN, int OUT, bool ACC>
hipError_t launch_fused_acc(const FusedArgs& a, bool vec, hipStream_t stream) {
  const int W = a.cp_size;
  if (W <= 1) return launch_fused_wb<IN, OUT, 1, ACC>(a, vec, stream);
  if (W <= 2) return launch_fused_wb<IN, OUT, 2, ACC>(a, vec, stream);
  return launch_fused_wb<IN, OUT, 4, ACC>(a, vec, stream);
}

template <int IN, int OUT>
hipError_t launch_fused_typed(const FusedArgs& a, bool vec, hipStream_t stream) {
  return a.accumulate ? launch_fused_acc<IN, OUT, true>(a, vec, stream)
                      : launch_fused_acc<IN, OUT, false>(a, vec, stream);
}


// ---- all-reduce launches --------------------------------------------------------
template <int T, int WB>
hipError_t launch_one_shot_wb(const AllreduceArgs& a, bool vec, hipStream_t stream) {
  constexpr int UPT = sum_upt(WB);
  static const std::string names[2] = {
      std::string("allreduce_one_shot<") + dtype_tag(T) + "," + std::to_string(WB) + ",s>",
      std::string("allreduce_one_shot<") + dtype_tag(T) + "," + std::to_string(WB) + ",v" +
          std::to_string(UPT) + ">"};
  int64_t blocks;
  if (vec) {
    constexpr int64_t G = unit_group_elems<T, T>();
    blocks = (a.n_elems / G * (G / 8) + (int64_t)kBlock * UPT - 1) / ((int64_t)kBlock * UPT);
  } else {
    blocks = (a.n_elems + kBlock - 1) / kBlock;
  }
  if (blocks > kMaxGrid) blocks = kMaxGrid;
  if (blocks < 1) blocks = 1;
  const dim3 grid((unsigned)blocks, (unsigned)a.cp_size);
  profile_before(names[vec ? 1 : 0].c_str(), stream);
  if (vec)
    hipLaunchKernelGGL((allreduce_one_shot_kernel<T, WB, true, UPT>), grid, dim3(kBlock), 0, stream, a);
  else
    hipLaunchKernelGGL((allreduce_one_shot_kernel<T, WB, false, 1>), grid, dim3(kBlock), 0, stream, a);
  hipError_t e = hipGetLastError();
  profile_after(stream);
  return e;
}

template <int T>
hipError_t launch_one_shot_typed(const AllreduceArgs& a, bool vec, hipStream_t stream) {
  const int W = a.cp_size;
  if (W <= 1) return launch_one_shot_wb<T, 1>(a, vec, stream);
  if (W <= 2) return launch_one_shot_wb<T, 2>(a, vec, stream);
  if (W <= 4) return launch_one_shot_wb<T, 4>(a, vec, stream);
  return launch_one_shot_wb<T, 8>(a, vec, stream);
}

bool allreduce_aligned(const AllreduceArgs& a) {
  bool vec = true;
  for (int w = 0; w < a.cp_size; ++w) vec = vec && aligned16(a.in.p[w]) && aligned16(a.out.p[w]);
  return vec;
}

constexpr int kRingUpt = 2;  // 8-element units per thread in a reduce-scatter step

template <int T>
hipError_t launch_ring_reduce_typed(const AllreduceArgs& a, int32_t step, bool vec, hipStream_t stream) {
  static const std::string names[2] = {std::string("ring_reduce_step<") + dtype_tag(T) + ",s>",
                                       std::string("ring_reduce_step<") + dtype_tag(T) + ",v>"};
  const int64_t len = a.chunk < a.n_elems ? a.chunk : a.n_elems;  // longest chunk
  int64_t blocks;
  if (vec) {
    constexpr int64_t G = unit_group_elems<T, T>();
    blocks = (len / G * (G / 8) + (int64_t)kBlock * kRingUpt - 1) / ((int64_t)kBlock * kRingUpt);
  } else {
    blocks = (len + kBlock - 1) / kBlock;
  }
  if (blocks > kMaxGrid) blocks = kMaxGrid;
  if (blocks < 1) blocks = 1;
  const dim3 grid((unsigned)blocks, (unsigned)a.cp_size);
  profile_before(names[vec ? 1 : 0].c_str(), stream);
  if (vec)
    hipLaunchKernelGGL((ring_reduce_step_kernel<T, true, kRingUpt>), grid, dim3(kBlock), 0, stream, a, step);
  else
    hipLaunchKernelGGL((ring_reduce_step_kernel<T, false, 1>), grid, dim3(kBlock), 0, stream, a, step);
  hipError_t e = hipGetLastError();
  profile_after(stream);
  return e;
}

template <int EB, bool FROM_IN>
hipError_t launch_ring_gather_typed(const AllreduceArgs& a, int32_t step, bool vec, hipStream_t stream) {
  static const std::string names[2] = {std::string("ring_gather_step<") + std::to_string(EB) + "B,s>",
                                       std::string("ring_gather_step<") + std::to_string(EB) + "B,v>"};
  const int64_t len = a.chunk < a.n_elems ? a.chunk : a.n_elems;
  int64_t blocks = vec ? (len * EB / 16 + (int64_t)kBlock * 4 - 1) / ((int64_t)kBlock * 4)
                       : (len + kBlock - 1) / kBlock;
  if (blocks > kMaxGrid) blocks = kMaxGrid;
  if (blocks < 1) blocks = 1;
  const dim3 grid((unsigned)blocks, (unsigned)a.cp_size);
  profile_before(names[vec ? 1 : 0].c_str(), stream);
  if (vec)
    hipLaunchKernelGGL((ring_gather_step_kernel<EB, true, FROM_IN>), grid, dim3(kBlock), 0, stream, a, step);
  else
    hipLaunchKernelGGL((ring_gather_step_kernel<EB, false, FROM_IN>), grid, dim3(kBlock), 0, stream, a, step);
  hipError_t e = hipGetLastError();
  profile_after(stream);
  return e;
}


template <int T>
int ring_signal_resident_blocks() {
  // Workgroups of this kernel that fit on the current device at once, kept per
  // device (the first 64 device indices; others are queried every time).
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  if (dev >= 0 && dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(&ring_signal_kernel<T>),
                                                   kBlock, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  if (dev >= 0 && dev < 64) cached[dev].store(per_cu * cus, std::memory_order_relaxed);
  return per_cu * cus;
}

}  // namespace

hipError_t launch_slot_sum(const SlotSumArgs& a, hipStream_t stream) {
  if (a.n_elems == 0) return hipSuccess;
  bool vec = aligned16(a.out);
  for (int w = 0; w < a.num_slots; ++w) vec = vec && aligned16(a.in.p[w]);
  if (a.in_dtype == CP_F32 && a.out_dtype == CP_F32) return launch_sum_typed<CP_F32, CP_F32>(a, vec, stream);
  if (a.in_dtype == CP_F32 && a.out_dtype == CP_BF16) return launch_sum_typed<CP_F32, CP_BF16>(a, vec, stream);
  if (a.in_dtype == CP_BF16 && a.out_dtype == CP_BF16) return launch_sum_typed<CP_BF16, CP_BF16>(a, vec, stream);
  if (a.in_dtype == CP_BF16 && a.out_dtype == CP_F32) return launch_sum_typed<CP_BF16, CP_F32>(a, vec, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_fused(const FusedArgs& a, hipStream_t stream) {
  if (a.total_tokens == 0 || a.row_elems == 0 || a.owner_end <= a.owner_begin) return hipSuccess;
  const int in_b = a.in_dtype == CP_F32 ? 4 : 2;
  const int out_b = a.out_dtype == CP_F32 ? 4 : 2;
  bool vec = a.row_elems % 8 == 0 && (a.row_elems * in_b) % 16 == 0 && (a.row_elems * out_b) % 16 == 0;
  for (int w = 0; w < a.cp_size; ++w) vec = vec && aligned16(a.grads.p[w]);
  for (int o = a.owner_begin; o < a.owner_end; ++o) vec = vec && aligned16(a.out.p[o]);
  if (a.in_dtype == CP_F32 && a.out_dtype == CP_F32) return launch_fused_typed<CP_F32, CP_F32>(a, vec, stream);
  if (a.in_dtype == CP_F32 && a.out_dtype == CP_BF16) return launch_fused_typed<CP_F32, CP_BF16>(a, vec, stream);
  if (a.in_dtype == CP_BF16 && a.out_dtype == CP_BF16) return launch_fused_typed<CP_BF16, CP_BF16>(a, vec, stream);
  if (a.in_dtype == CP_BF16 && a.out_dtype == CP_F32) return launch_fused_typed<CP_BF16, CP_F32>(a, vec, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_allreduce_one_shot(const AllreduceArgs& a, hipStream_t stream) {
  if (a.n_elems == 0) return hipSuccess;
  const bool vec = allreduce_aligned(a);
  if (a.dtype == CP_F32) return launch_one_shot_typed<CP_F32>(a, vec, stream);
  if (a.dtype == CP_BF16) return launch_one_shot_typed<CP_BF16>(a, vec, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_ring_reduce_step(const AllreduceArgs& a, int32_t step, hipStream_t stream) {
  if (a.n_elems == 0) return hipSuccess;
  const bool vec = allreduce_aligned(a);
  if (a.dtype == CP_F32) return launch_ring_reduce_typed<CP_F32>(a, step, vec, stream);
  if (a.dtype == CP_BF16) return launch_ring_reduce_typed<CP_BF16>(a, step, vec, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_ring_gather_step(const AllreduceArgs& a, int32_t step, bool from_input,
                                   hipStream_t stream) {
  if (a.n_elems == 0) return hipSuccess;
  const bool vec = allreduce_aligned(a);
  if (a.dtype == CP_F32)
    return from_input ? launch_ring_gather_typed<4, true>(a, step, vec, stream)
                      : launch_ring_gather_typed<4, false>(a, step, vec, stream);
  if (a.dtype == CP_BF16)
    return from_input ? launch_ring_gather_typed<2, true>(a, step, vec, stream)
                      : launch_ring_gather_typed<2, false>(a, step, vec, stream);
  return hipErrorInvalidValue;
}

int ring_signal_tiles(const AllreduceArgs& a, int64_t* tile_elems) {
  const int resident = a.dtype == CP_F32 ? ring_signal_resident_blocks<CP_F32>()
                                         : ring_signal_resident_blocks<CP_BF16>();
  int cap = resident / 2 / a.cp_size;  // at most half of the resident capacity
  if (cap > kSignalTiles) cap = kSignalTiles;
  if (cap < 1) return 0;
  const int64_t q = a.chunk < a.n_elems ? a.chunk : a.n_elems;
  // About sqrt(q / 2048) tiles, at most 16: every agent-scope release and
  // acquire acts on a whole L2, so more workgroups per hop cost more than they
  // stream (W = 8 fp32, measured best: 1 tile up to 64 KiB per rank, 2 at
  // 256 KiB, 4 at 1 MiB, 8 at 4 MiB, 16 at 16 MiB).
  int tiles = 1;
  while (tiles < 16 && (int64_t)(tiles + 1) * (tiles + 1) * 2048 <= q) ++tiles;
  if (tiles > cap) tiles = cap;
  int64_t te = (q + tiles - 1) / tiles;
  te = (te + 511) / 512 * 512;
  if (te < 512) te = 512;
  *tile_elems = te;
  return (int)((q + te - 1) / te);
}

hipError_t launch_ring_signal(const AllreduceArgs& a, const RingSignalArgs& g, int tiles, hipStream_t stream) {
  if (a.n_elems == 0) return hipSuccess;
  const dim3 grid((unsigned)tiles, (unsigned)a.cp_size);
  AllreduceArgs args = a;
  args.vec = allreduce_aligned(a) ? 1 : 0;
  RingSignalArgs sig = g;
  void* params[2] = {&args, &sig};
  static const std::string names[2] = {"ring_signal<f32>", "ring_signal<bf16>"};
  profile_before(names[a.dtype == CP_F32 ? 0 : 1].c_str(), stream);
  hipError_t e;
  if (a.dtype == CP_F32)
    e = hipLaunchKernel(reinterpret_cast<const void*>(&ring_signal_kernel<CP_F32>), grid, dim3(kBlock), params, 0,
                        stream);
  else
    e = hipLaunchKernel(reinterpret_cast<const void*>(&ring_signal_kernel<CP_BF16>), grid, dim3(kBlock), params, 0,
                        stream);
  if (e == hipSuccess) e = hipGetLastError();
  else (void)hipGetLastError();
  profile_after(stream);
  return e;
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
