// All-reduce of W rank buffers held on one device: one-shot, ring (one launch
// per step), two-shot, and the ring in one launch with in-kernel signalling.
#include "units.h"

#include <atomic>
#include <string>
#include <type_traits>

namespace cpthd {
namespace {

// ---- element ranges that start anywhere -------------------------------------------
// The ring's chunks start at multiples of ceil(n / W) elements, so a chunk need
// not start on a 16-byte boundary even when every buffer does.  A range
// [lo, hi) is split into a head [lo, vlo) up to the first 16-byte boundary, a
// vector section [vlo, vend) of whole unit groups, and a tail [vend, hi); the
// head and tail are done element by element.  Without the vector path the whole
// range is scalar (vlo = vend = lo).
struct Span {
  int64_t lo, vlo, vend, hi;
  int64_t nunits;  // vector units (8 elements, or 16 bytes for copies) in [vlo, vend)
};

// A = elements per 16 bytes, G = elements per vector unit group, U = elements per unit.
template <int64_t A, int64_t G, int64_t U>
__device__ __forceinline__ Span split_span(int64_t lo, int64_t hi, bool vec) {
  Span s{lo, lo, lo, hi, 0};
  if (!vec || hi <= lo) return s;
  int64_t v = (lo + A - 1) / A * A;
  if (v > hi) v = hi;
  s.vlo = v;
  s.nunits = (hi - v) / G * (G / U);
  s.vend = v + s.nunits * U;
  return s;
}
__device__ __forceinline__ int64_t span_scalar_count(const Span& s) { return (s.vlo - s.lo) + (s.hi - s.vend); }
// Element index of the j-th scalar element: the head first, then the tail.
__device__ __forceinline__ int64_t span_scalar(const Span& s, int64_t j) {
  const int64_t h = s.vlo - s.lo;
  return j < h ? s.lo + j : s.vend + (j - h);
}
template <int T>
constexpr int64_t elems_per_16B() { return T == CP_F32 ? 4 : 8; }

// ---- all-reduce: one-shot, ring, two-shot ----------------------------------------
// "Low Latency Communication Kernels with NVSHMEM": the all-reduce algorithms
// picked by message size and the exercise comparing a one-shot all-reduce
// with a ring over 1 KB - 16 MB.  One-shot: every rank sums all W buffers
// itself.  Ring: a reduce-scatter then an all-gather, W-1 steps each, every
// rank passing one chunk to rank r+1 per step; partials travel in the buffer
// type, so a bf16 ring rounds after each add.  Two-shot (not named by the
// pages; the direct algorithm between the two): rank r sums chunk r of all
// buffers, then every rank copies every reduced chunk.
// All W ranks' buffers sit in this device's HBM; each launch does one step of
// the algorithm for every rank, ranks in blockIdx.y (dispatch runs rank by
// rank, as W devices would each do their own share).

// One-shot: rank r's workgroups sum all W inputs in rank order (seeded with
// input 0, one fp32 add per further input) and write out[r].  CHUNKED (the
// two-shot's reduce-scatter): rank r sums and writes only chunk r.
template <int T, int WB, bool VEC, int UPT, bool CHUNKED>
__global__ void __launch_bounds__(kBlock) allreduce_one_shot_kernel(AllreduceArgs a) {
  const int W = a.cp_size;
  const int r = blockIdx.y;
  constexpr int64_t eb = T == CP_F32 ? 4 : 2;
  int64_t lo = 0, hi = a.n_elems;
  if constexpr (CHUNKED) {
    lo = (int64_t)r * a.chunk < a.n_elems ? (int64_t)r * a.chunk : a.n_elems;
    hi = lo + a.chunk < a.n_elems ? lo + a.chunk : a.n_elems;
  }
  constexpr bool SPLIT = split_layout<T, T>();
  const Span sp = split_span<elems_per_16B<T>(), unit_group_elems<T, T>(), 8>(lo, hi, VEC);
  const int64_t off0 = sp.vlo * eb;
  char* const out = a.out.p[r] + off0;
  if constexpr (VEC) {
    const int64_t nunits = sp.nunits;
    const int64_t ntiles = (nunits + (int64_t)kBlock * UPT - 1) / ((int64_t)kBlock * UPT);
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
      int64_t unit[UPT], off[UPT];
      bool ok[UPT];
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
        unit[u] = tile * kBlock * UPT + (int64_t)u * kBlock + threadIdx.x;
        ok[u] = unit[u] < nunits;
        off[u] = off0;
      }
      F8 acc[UPT];
      sum_units<T, SPLIT, WB, UPT, false>(acc, a.in, W, off, unit, ok);
#pragma unroll
      for (int u = 0; u < UPT; ++u)
        if (ok[u]) store_unit<T, SPLIT>(out, unit[u], acc[u]);
    }
  }
  const int64_t gstride = (int64_t)gridDim.x * kBlock;
  const int64_t nscalar = span_scalar_count(sp);
  for (int64_t j = (int64_t)blockIdx.x * kBlock + threadIdx.x; j < nscalar; j += gstride) {
    const int64_t k = span_scalar(sp, j);
    float acc = load_elem<T>(a.in.p[0], k);
    for (int w = 1; w < W; ++w) acc = acc + load_elem<T>(a.in.p[w], k);
    store_elem<T>(a.out.p[r], k, acc);
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
  constexpr int64_t eb = T == CP_F32 ? 4 : 2;
  const Span sp = split_span<elems_per_16B<T>(), unit_group_elems<T, T>(), 8>(lo, hi, VEC);
  const char* const recv_base = step == 0 ? a.in.p[prev] : a.out.p[prev];
  const char* const recv = recv_base + sp.vlo * eb;
  const char* const own = a.in.p[r] + sp.vlo * eb;
  char* const dst = a.out.p[r] + sp.vlo * eb;
  constexpr bool SPLIT = split_layout<T, T>();
  if constexpr (VEC) {
    const int64_t nunits = sp.nunits;
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
  }
  const int64_t gstride = (int64_t)gridDim.x * kBlock;
  const int64_t nscalar = span_scalar_count(sp);
  for (int64_t j = (int64_t)blockIdx.x * kBlock + threadIdx.x; j < nscalar; j += gstride) {
    const int64_t k = span_scalar(sp, j);
    store_elem<T>(a.out.p[r], k, load_elem<T>(recv_base, k) + load_elem<T>(a.in.p[r], k));
  }
}

// Copy elements [lo, hi) of EB bytes from buffer src to buffer dst, bit for
// bit: 16-byte units (4 per thread and tile) from the first 16-byte boundary
// when VEC, the head and tail element by element; tiles over blockIdx.x.
template <int EB, bool VEC>
__device__ __forceinline__ void copy_range(const char* src, char* dst, int64_t lo, int64_t hi) {
  const Span sp = split_span<16 / EB, 16 / EB, 16 / EB>(lo, hi, VEC);
  if constexpr (VEC) {
    constexpr int kUpt = 4;
    const int64_t n16 = sp.nunits;
    const int64_t ntiles = (n16 + (int64_t)kBlock * kUpt - 1) / ((int64_t)kBlock * kUpt);
    const u32x4* s16 = reinterpret_cast<const u32x4*>(src + sp.vlo * EB);
    u32x4* d16 = reinterpret_cast<u32x4*>(dst + sp.vlo * EB);
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
  }
  typedef typename std::conditional<EB == 4, unsigned int, unsigned short>::type E;
  const E* se = reinterpret_cast<const E*>(src);
  E* de = reinterpret_cast<E*>(dst);
  const int64_t gstride = (int64_t)gridDim.x * kBlock;
  const int64_t nscalar = span_scalar_count(sp);
  for (int64_t j = (int64_t)blockIdx.x * kBlock + threadIdx.x; j < nscalar; j += gstride) {
    const int64_t k = span_scalar(sp, j);
    de[k] = se[k];
  }
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
  copy_range<EB, VEC>(FROM_IN ? a.in.p[r] : a.out.p[prev], a.out.p[r], lo, hi);
}

// Two-shot all-gather: rank r (blockIdx.y) copies chunk c = (r+1+z) mod W
// (z = blockIdx.z < W-1) from its owner's output, bit for bit.
template <int EB, bool VEC>
__global__ void __launch_bounds__(kBlock) two_shot_gather_kernel(AllreduceArgs a) {
  const int W = a.cp_size;
  const int r = blockIdx.y;
  const int c = (r + 1 + (int)blockIdx.z) % W;
  int64_t lo, hi;
  ring_chunk(a, c, lo, hi);
  copy_range<EB, VEC>(a.out.p[c], a.out.p[r], lo, hi);
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
    if (reduce) {
      const Span sp = split_span<elems_per_16B<T>(), G, 8>(tlo, thi, vec);
      const char* const recv_base = s == 0 ? in_prev : out_prev;
      const char* const recv = recv_base + sp.vlo * eb;
      const char* const own = in_mine + sp.vlo * eb;
      char* const dst = out_mine + sp.vlo * eb;
      const int64_t nunits = sp.nunits;
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
      const int64_t nscalar = span_scalar_count(sp);
      for (int64_t j = threadIdx.x; j < nscalar; j += kBlock) {
        const int64_t q = span_scalar(sp, j);
        store_elem<T>(out_mine, q, load_elem<T>(recv_base, q) + load_elem<T>(in_mine, q));
      }
    } else {
      const Span sp = split_span<16 / eb, 16 / eb, 16 / eb>(tlo, thi, vec);
      const char* const src = out_prev + sp.vlo * eb;
      char* const dst = out_mine + sp.vlo * eb;
      const int64_t n16 = sp.nunits;
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
      const int64_t nscalar = span_scalar_count(sp);
      for (int64_t j = threadIdx.x; j < nscalar; j += kBlock) {
        const int64_t q = span_scalar(sp, j);
        reinterpret_cast<E*>(out_mine)[q] = reinterpret_cast<const E*>(out_prev)[q];
      }
    }
    // The barrier completes every wave's stores into this XCD's L2; lane 0's
    // agent-scope release then writes the L2 back before the flag is stored.
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_store(mine, base + (uint64_t)(k + 1), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---- all-reduce launches --------------------------------------------------------
template <int T, int WB, bool CHUNKED>
hipError_t launch_one_shot_wb(const AllreduceArgs& a, bool vec, hipStream_t stream) {
  constexpr int UPT = sum_upt(WB);
  const std::string tag = std::string(CHUNKED ? "two_shot_reduce<" : "allreduce_one_shot<") + dtype_tag(T) +
                          "," + std::to_string(WB) + ",";
  static const std::string names[2] = {tag + "s>", tag + "v" + std::to_string(UPT) + ">"};
  const int64_t len = CHUNKED ? (a.chunk < a.n_elems ? a.chunk : a.n_elems) : a.n_elems;  // longest range
  int64_t blocks;
  if (vec) {
    constexpr int64_t G = unit_group_elems<T, T>();
    blocks = (len / G * (G / 8) + (int64_t)kBlock * UPT - 1) / ((int64_t)kBlock * UPT);
  } else {
    blocks = (len + kBlock - 1) / kBlock;
  }
  if (blocks > kMaxGrid) blocks = kMaxGrid;
  if (blocks < 1) blocks = 1;
  const dim3 grid((unsigned)blocks, (unsigned)a.cp_size);
  profile_before(names[vec ? 1 : 0].c_str(), stream);
  if (vec)
    hipLaunchKernelGGL((allreduce_one_shot_kernel<T, WB, true, UPT, CHUNKED>), grid, dim3(kBlock), 0, stream, a);
  else
    hipLaunchKernelGGL((allreduce_one_shot_kernel<T, WB, false, 1, CHUNKED>), grid, dim3(kBlock), 0, stream, a);
  hipError_t e = hipGetLastError();
  profile_after(stream);
  return e;
}

template <int T, bool CHUNKED>
hipError_t launch_one_shot_typed(const AllreduceArgs& a, bool vec, hipStream_t stream) {
  const int W = a.cp_size;
  if (W <= 1) return launch_one_shot_wb<T, 1, CHUNKED>(a, vec, stream);
  if (W <= 2) return launch_one_shot_wb<T, 2, CHUNKED>(a, vec, stream);
  if (W <= 4) return launch_one_shot_wb<T, 4, CHUNKED>(a, vec, stream);
  return launch_one_shot_wb<T, 8, CHUNKED>(a, vec, stream);
}

template <int EB>
hipError_t launch_two_shot_gather_typed(const AllreduceArgs& a, bool vec, hipStream_t stream) {
  static const std::string names[2] = {std::string("two_shot_gather<") + std::to_string(EB) + "B,s>",
                                       std::string("two_shot_gather<") + std::to_string(EB) + "B,v>"};
  const int64_t len = a.chunk < a.n_elems ? a.chunk : a.n_elems;
  int64_t blocks = vec ? (len * EB / 16 + (int64_t)kBlock * 4 - 1) / ((int64_t)kBlock * 4)
                       : (len + kBlock - 1) / kBlock;
  if (blocks > kMaxGrid) blocks = kMaxGrid;
  if (blocks < 1) blocks = 1;
  const dim3 grid((unsigned)blocks, (unsigned)a.cp_size, (unsigned)(a.cp_size - 1));
  profile_before(names[vec ? 1 : 0].c_str(), stream);
  if (vec)
    hipLaunchKernelGGL((two_shot_gather_kernel<EB, true>), grid, dim3(kBlock), 0, stream, a);
  else
    hipLaunchKernelGGL((two_shot_gather_kernel<EB, false>), grid, dim3(kBlock), 0, stream, a);
  hipError_t e = hipGetLastError();
  profile_after(stream);
  return e;
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

hipError_t launch_allreduce_one_shot(const AllreduceArgs& a, hipStream_t stream) {
  if (a.n_elems == 0) return hipSuccess;
  const bool vec = allreduce_aligned(a);
  if (a.dtype == CP_F32) return launch_one_shot_typed<CP_F32, false>(a, vec, stream);
  if (a.dtype == CP_BF16) return launch_one_shot_typed<CP_BF16, false>(a, vec, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_allreduce_two_shot(const AllreduceArgs& a, hipStream_t stream) {
  if (a.n_elems == 0) return hipSuccess;
  const bool vec = allreduce_aligned(a);
  hipError_t e;
  if (a.dtype == CP_F32) e = launch_one_shot_typed<CP_F32, true>(a, vec, stream);
  else if (a.dtype == CP_BF16) e = launch_one_shot_typed<CP_BF16, true>(a, vec, stream);
  else return hipErrorInvalidValue;
  if (e != hipSuccess || a.cp_size == 1) return e;
  return a.dtype == CP_F32 ? launch_two_shot_gather_typed<4>(a, vec, stream)
                           : launch_two_shot_gather_typed<2>(a, vec, stream);
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

}  // namespace cpthd
