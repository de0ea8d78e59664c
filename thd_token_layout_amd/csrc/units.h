// Element-unit helpers shared by the reduction kernels (owner sums, fused
// gradient return, all-reduce): bf16 <-> fp32 on the bit pattern, the 8-element
// unit layouts, unit loads and stores, and the in-order slot sum.
#pragma once

#include "device_common.h"

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

// ---- 16-byte input pieces ----------------------------------------------------
// The layout with one load per lane and slot: a piece is the elements one
// 16-byte load of the input holds (4 fp32 or 8 bf16), piece p being elements
// [E p, E p + E), and the output keeps them at the same positions in its own
// type (16 bytes for fp32 -> fp32 and bf16 -> bf16, 8 bytes for fp32 -> bf16),
// so every wave instruction covers one contiguous span on both sides.  bf16 ->
// fp32 would store 32 bytes per lane and keeps the split units above.
template <int IN, int OUT>
constexpr bool piece_layout() { return !(IN == CP_BF16 && OUT == CP_F32); }
template <int IN>
constexpr int piece_elems() { return IN == CP_F32 ? 4 : 8; }

template <int IN>
__device__ __forceinline__ void load_in_piece(F8& x, const char* base, int64_t piece) {
  const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base) + piece);
  if constexpr (IN == CP_F32) {
    f32x4_from(x.v, a);
  } else {
    bf16x4_to_f32(x.v, u32x2{a.x, a.y});
    bf16x4_to_f32(x.v + 4, u32x2{a.z, a.w});
  }
}

// The output's piece (the accumulate mode's seed), widened to fp32.
template <int IN, int OUT>
__device__ __forceinline__ void load_out_piece(F8& x, const char* base, int64_t piece) {
  static_assert(piece_layout<IN, OUT>(), "no piece layout for bf16 -> fp32");
  if constexpr (OUT == CP_BF16 && IN == CP_F32)
    bf16x4_to_f32(x.v, __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(base) + piece));
  else
    load_in_piece<OUT>(x, base, piece);
}

template <int IN, int OUT>
__device__ __forceinline__ void store_piece(char* base, int64_t piece, const F8& x) {
  static_assert(piece_layout<IN, OUT>(), "no piece layout for bf16 -> fp32");
  if constexpr (OUT == CP_F32) {
    __builtin_nontemporal_store(f32x4_bits(x.v), reinterpret_cast<u32x4*>(base) + piece);
  } else if constexpr (IN == CP_F32) {
    __builtin_nontemporal_store(bf16x4_bits(x.v), reinterpret_cast<u32x2*>(base) + piece);
  } else {
    const u32x2 lo = bf16x4_bits(x.v), hi = bf16x4_bits(x.v + 4);
    __builtin_nontemporal_store(u32x4{lo.x, lo.y, hi.x, hi.y}, reinterpret_cast<u32x4*>(base) + piece);
  }
}

// Sum NP pieces over slots 0..W-1 in order, with one load in flight per lane:
// every load is waited for before the next is issued.  Measured on MI355X
// (plain 4:1 streams, 2.7 GB buffers): one 16-byte load in flight per lane
// streams 6.4 TB/s, two 6.1, four 5.9-6.0.  `in` is the kernel argument table
// (uniform), off[m] a byte offset applied to every slot for piece m, ok[m]
// masks pieces past the end.  Without ACC the accumulator is seeded with slot
// 0; with ACC the caller has seeded it and every slot is added.
template <int IN, int WB, int NP, bool ACC>
__device__ __forceinline__ void sum_pieces(F8 (&acc)[NP], const ConstRankPtrs& in, int W,
                                           const int64_t (&off)[NP], const int64_t (&piece)[NP],
                                           const bool (&ok)[NP]) {
  constexpr int E = piece_elems<IN>();
  auto add = [&](const char* slot, bool first) {
#pragma unroll
    for (int m = 0; m < NP; ++m) {
      F8 x{};
      if (ok[m]) load_in_piece<IN>(x, slot + off[m], piece[m]);
      __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[m].v[e] = first && !ACC ? x.v[e] : acc[m].v[e] + x.v[e];
    }
  };
#pragma unroll
  for (int w = 0; w < WB; ++w)
    if (w < W) add(in.p[w], w == 0);
  for (int w0 = WB; w0 < W; w0 += WB)
#pragma unroll
    for (int w = 0; w < WB; ++w)
      if (w0 + w < W) add(in.p[w0 + w], false);
}

// Seed of the accumulate mode: the owner's current values, widened to fp32.
template <int OUT, bool SPLIT, int UPT>
__device__ __forceinline__ void seed_units(F8 (&acc)[UPT], const char* out, const int64_t (&unit)[UPT],
                                           const bool (&ok)[UPT]) {
#pragma unroll
  for (int u = 0; u < UPT; ++u)
    if (ok[u]) load_unit<OUT, SPLIT>(acc[u], out, unit[u]);
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

inline const char* dtype_tag(int dt) { return dt == CP_F32 ? "f32" : "bf16"; }

// Tile shapes (units of 8 elements per thread / per lane, waves per row).
// Chosen from a sweep on MI355X; see the kernels' comments.
// At most 8 slots x 8 floats of loaded data per thread and pass: more raises
// register use enough to lower occupancy (a W=8 bf16 sum with 2 units per
// thread measured 25% slower).
constexpr int sum_upt(int wb) { return wb <= 2 ? 4 : wb <= 4 ? 2 : 1; }
// The piece layout (one load in flight per lane) serves sums of at most
// kPieceMaxSlots slots of at least kPieceMinBytes each; smaller ones are
// latency-bound, and with eight slots the serial chain per lane grows long
// enough that a batch of loads in flight streams better (measured on MI355X:
// eight 134 MB bf16 slots 197 us batched against 212 us one at a time; fused
// return of eight 1 GiB writers 1552 against 1580 us), so those keep the
// units.  Pieces per thread from a sweep (owner sum of four 671 MB fp32
// slots: 536 us with one, 550 with two; fused return of four 2.7 GB writers:
// 2105 us with two, 2288 with one, 2142-2164 with three or four): the owner
// sum streams best with one, the fused return, which looks up its rows per
// tile, with two.
constexpr int64_t kPieceMinBytes = int64_t(32) << 20;
constexpr int kPieceMaxSlots = 4;
constexpr int kSumPiecesPerThread = 1;
constexpr int kFusedPiecesPerThread = 2;
// Threads per workgroup of the owner sums' and the fused return's flat tiles
// from kPieceMinBytes per slot or writer: one wave.  Measured on MI355X
// against 256 threads: owner sum of four 671 MB fp32 slots 537 -> 522 us,
// fused return of four 2.7 GB writers 2119 -> 2036 us (with two pieces per
// thread; four 2127, eight 2300), eight 134 MB bf16 slots 197 -> 195 us, eight
// 1 GiB bf16 writers 1545 -> 1519 us; plain streams too run 1.5% faster in
// 64-thread workgroups.  Smaller sums keep 256 threads (eight 8 MiB fp32 slots
// took 17 us in one-wave workgroups, 14 us in 256-thread ones).
constexpr int kSumBlock = 64;

}  // namespace
}  // namespace cpthd
