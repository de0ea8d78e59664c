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
// Design: HBM-bound streaming, two unit layouts (units.h), every wave
// instruction touching one contiguous span.  Large sums of at most four slots
// read 16-byte pieces, one load in flight per lane, slot after slot; other
// sums handle units of 8 elements and issue the loads of a batch of WB slots
// before adding them in order.  Both write with non-temporal stores.  Large
// sums run in one-wave workgroups, smaller ones in 256-thread workgroups.
// Launches cover all work with one small contiguous tile per workgroup (a full
// grid rather than a resident-capacity persistent loop, which streams HBM less
// contiguously and measured slower on MI355X).
#include "units.h"

#include <string>


namespace cpthd {
namespace {

// Gradient-return kernels need metadata built for W ranks and T tokens (either
// policy: the owner's rows are those the partition gives it).
__device__ __forceinline__ bool grad_meta_ok(cp_meta_header* h, const cp_meta_header& v, int64_t T, int32_t W) {
  return meta_ok(h, v, T, W, -1);
}
__device__ __forceinline__ bool grad_meta_ok(cp_meta_header* h, int64_t T, int32_t W) {
  return meta_ok(h, T, W, -1);
}

// ---- slot sum ----------------------------------------------------------------
// A workgroup of BS threads owns a tile of BS*UPT consecutive units (8-element
// units, or 16-byte pieces); thread t takes units t, t + BS, ... of the tile
// (coalesced per load instruction).
// MODE 0: elements (unaligned pointers); 1: 8-element units, the loads of a
// batch of slots in flight together; 2: 16-byte pieces, one load in flight.
template <int IN, int OUT, int WB, int MODE, int UPT, bool ACC, int BS = kBlock>
__global__ void __launch_bounds__(BS) slot_sum_kernel(SlotSumArgs a) {
  if (a.gate_meta != nullptr) {
    cp_meta_header* h = a.gate_meta;
    const cp_meta_header hv = read_header(h);
    if (!grad_meta_ok(h, hv, a.gate_T, a.num_slots)) return;
    if (a.owner >= 0 && ((hv.wait_timeout_ranks >> a.owner) & 1ull)) return;
  }
  const int W = a.num_slots;
  constexpr bool SPLIT = split_layout<IN, OUT>();
  int64_t done = 0;
  if constexpr (MODE == 2) {
    static_assert(piece_layout<IN, OUT>(), "no piece layout for bf16 -> fp32");
    // 16-byte input pieces, one load in flight per lane (units.h)
    constexpr int E = piece_elems<IN>();
    const int64_t npieces = a.n_elems / E;
    const int64_t ntiles = (npieces + (int64_t)BS * UPT - 1) / ((int64_t)BS * UPT);
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
      int64_t piece[UPT], off[UPT];
      bool ok[UPT];
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
        piece[u] = tile * BS * UPT + (int64_t)u * BS + threadIdx.x;
        ok[u] = piece[u] < npieces;
        off[u] = 0;
      }
      F8 acc[UPT] = {};
      if constexpr (ACC) {
#pragma unroll
        for (int u = 0; u < UPT; ++u)
          if (ok[u]) load_out_piece<IN, OUT>(acc[u], a.out, piece[u]);
      }
      sum_pieces<IN, WB, UPT, ACC>(acc, a.in, W, off, piece, ok);
#pragma unroll
      for (int u = 0; u < UPT; ++u)
        if (ok[u]) store_piece<IN, OUT>(a.out, piece[u], acc[u]);
    }
    done = npieces * E;
  } else if constexpr (MODE == 1) {
    const int64_t nunits = a.n_elems / unit_group_elems<IN, OUT>() * (unit_group_elems<IN, OUT>() / 8);
    const int64_t ntiles = (nunits + (int64_t)BS * UPT - 1) / ((int64_t)BS * UPT);
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
      int64_t unit[UPT], off[UPT];
      bool ok[UPT];
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
        unit[u] = tile * BS * UPT + (int64_t)u * BS + threadIdx.x;
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
  const int64_t gtid = (int64_t)blockIdx.x * BS + threadIdx.x;
  const int64_t gstride = (int64_t)gridDim.x * BS;
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
  const int32_t policy = h->policy;
  const int32_t* cu = meta_cu(h);
  const int32_t* lcu = meta_local_cu0(h, B);
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
    const int64_t g = owner_global_row(policy, o, i, n, W, B, cu, lcu);
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
// rows * units_per_row units (8 elements, or 16-byte pieces), and a workgroup
// of BS threads owns BS*NP consecutive units of it (a tile may start and end
// inside a row), so every thread does exactly NP units in one pass, as in the
// slot sum.  The first
// threads look up the source offset and destination of the <= kMaxTileRows
// rows the tile touches and share them through LDS.  The row of a unit is
// found with a multiply-high by `upr_magic` = ceil(2^32 / units_per_row),
// exact while the in-tile offset times units_per_row stays below 2^32.
constexpr int kMaxTileRows = 16;

// PIECES: 16-byte pieces with one load in flight (units.h), else 8-element
// units with the loads of a batch of writers in flight together.
template <int IN, int OUT, int WB, int NP, bool ACC, bool PIECES, int BS = kBlock>
__global__ void __launch_bounds__(BS) fused_flat_kernel(FusedArgs a, uint32_t upr_magic) {
  static_assert(!PIECES || piece_layout<IN, OUT>(), "no piece layout for bf16 -> fp32");
  __shared__ int64_t s_src[kMaxTileRows];
  __shared__ char* s_dst[kMaxTileRows];
  cp_meta_header* h = a.meta;
  if (!grad_meta_ok(h, a.total_tokens, a.cp_size)) return;
  const int32_t W = a.cp_size;
  const int32_t B = h->num_docs;
  const int64_t n = h->local_tokens;
  const int32_t policy = h->policy;
  const int32_t* cu = meta_cu(h);
  const int32_t* lcu = meta_local_cu0(h, B);
  const int in_bytes = IN == CP_F32 ? 4 : 2;
  const int out_bytes = OUT == CP_F32 ? 4 : 2;
  const int64_t upr = a.row_elems / (PIECES ? piece_elems<IN>() : 8);  // units (pieces) per row
  const int64_t rows = (int64_t)(a.owner_end - a.owner_begin) * n;
  const int64_t total = rows * upr;
  constexpr int64_t kTileUnits = (int64_t)BS * NP;
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
      s_src[threadIdx.x] = owner_global_row(policy, o, i, n, W, B, cu, lcu) * a.row_elems * in_bytes;
      s_dst[threadIdx.x] = a.out.p[o] + i * a.row_elems * out_bytes;
    }
    __syncthreads();
    const int64_t base = u0 - row0 * upr;  // offset of the tile's first unit inside row0
    int64_t unit[NP], off[NP];
    int row[NP];
    bool ok[NP];
#pragma unroll
    for (int m = 0; m < NP; ++m) {
      const uint32_t f = (uint32_t)(base + (int64_t)m * BS + threadIdx.x);
      ok[m] = u0 + (int64_t)m * BS + threadIdx.x < u_end;
      row[m] = ok[m] ? (int)__umulhi(f, upr_magic) : 0;
      unit[m] = (int64_t)f - (int64_t)row[m] * upr;
      off[m] = s_src[row[m]];
    }
    F8 acc[NP] = {};
    if constexpr (PIECES) {
      if constexpr (ACC) {
#pragma unroll
        for (int m = 0; m < NP; ++m)
          if (ok[m]) load_out_piece<IN, OUT>(acc[m], s_dst[row[m]], unit[m]);
      }
      sum_pieces<IN, WB, NP, ACC>(acc, a.grads, W, off, unit, ok);
#pragma unroll
      for (int m = 0; m < NP; ++m)
        if (ok[m]) store_piece<IN, OUT>(s_dst[row[m]], unit[m], acc[m]);
    } else {
      if constexpr (ACC) {
#pragma unroll
        for (int m = 0; m < NP; ++m)
          if (ok[m]) load_unit<OUT, split_layout<IN, OUT>()>(acc[m], s_dst[row[m]], unit[m]);
      }
      sum_units<IN, split_layout<IN, OUT>(), WB, NP, ACC>(acc, a.grads, W, off, unit, ok);
#pragma unroll
      for (int m = 0; m < NP; ++m)
        if (ok[m]) store_unit<OUT, split_layout<IN, OUT>()>(s_dst[row[m]], unit[m], acc[m]);
    }
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

// ---- dispatch -------------------------------------------------------------------
constexpr int fused_upl(int wb) { return wb <= 2 ? 2 : 1; }
constexpr int kFusedWpr = 4;
// Fused shapes of the batched units, from a sweep on the S=262144 (W=4 fp32)
// and S=131072 (W=8 bf16) shapes: flat unit tiles, 2 units per thread for
// W <= 4 (6.20 TB/s, against 6.05 for a wave per row), 1 unit per thread
// above.  The piece layout's shape is in units.h.

template <int IN, int OUT, int WB, bool ACC>
hipError_t launch_sum_wb(const SlotSumArgs& a, bool vec, hipStream_t stream) {
  constexpr int UPT_UNITS = sum_upt(WB);
  constexpr int UPT_PIECES = kSumPiecesPerThread;
  const std::string tag = std::string(ACC ? "slot_sum_acc<" : "slot_sum<") + dtype_tag(IN) + "," +
                          dtype_tag(OUT) + "," + std::to_string(WB) + ",";
  static const std::string names[3] = {tag + "s>", tag + "v" + std::to_string(UPT_UNITS) + ">",
                                       tag + "p" + std::to_string(UPT_PIECES) + ">"};
  const int64_t slot_bytes = a.n_elems * (IN == CP_F32 ? 4 : 2);
  const bool large = slot_bytes >= kPieceMinBytes;  // one-wave workgroups, pieces for <= kPieceMaxSlots slots
  const int mode = !vec ? 0 : piece_layout<IN, OUT>() && large && a.num_slots <= kPieceMaxSlots ? 2 : 1;
  const int64_t bs = large ? kSumBlock : kBlock;
  int64_t blocks;
  if (mode == 2) {
    const int64_t pieces = a.n_elems / piece_elems<IN>();
    blocks = (pieces + (int64_t)kSumBlock * UPT_PIECES - 1) / ((int64_t)kSumBlock * UPT_PIECES);
  } else if (mode == 1) {
    constexpr int64_t G = unit_group_elems<IN, OUT>();
    const int64_t units = a.n_elems / G * (G / 8);
    blocks = (units + bs * UPT_UNITS - 1) / (bs * UPT_UNITS);
    const int64_t tail = a.n_elems - units * 8;  // elements left to the scalar loop
    if (blocks == 0 && tail > 0) blocks = 1;
  } else {
    blocks = (a.n_elems + kBlock - 1) / kBlock;
  }
  if (blocks > kMaxGrid) blocks = kMaxGrid;
  if (blocks < 1) blocks = 1;
  profile_before(names[mode].c_str(), stream);
  if constexpr (piece_layout<IN, OUT>()) {
    if (mode == 2)
      hipLaunchKernelGGL((slot_sum_kernel<IN, OUT, WB, 2, UPT_PIECES, ACC, kSumBlock>), dim3((unsigned)blocks),
                         dim3(kSumBlock), 0, stream, a);
  }
  if (mode == 1 && large)
    hipLaunchKernelGGL((slot_sum_kernel<IN, OUT, WB, 1, UPT_UNITS, ACC, kSumBlock>), dim3((unsigned)blocks),
                       dim3(kSumBlock), 0, stream, a);
  else if (mode == 1)
    hipLaunchKernelGGL((slot_sum_kernel<IN, OUT, WB, 1, UPT_UNITS, ACC>), dim3((unsigned)blocks), dim3(kBlock), 0,
                       stream, a);
  else if (mode == 0)
    hipLaunchKernelGGL((slot_sum_kernel<IN, OUT, WB, 0, 1, ACC>), dim3((unsigned)blocks), dim3(kBlock), 0,
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

template <int IN, int OUT, int WB, int NP, bool ACC, bool PIECES, int BS = kBlock>
void launch_fused_flat(const FusedArgs& a, int64_t blocks, uint32_t magic, hipStream_t stream) {
  hipLaunchKernelGGL((fused_flat_kernel<IN, OUT, WB, NP, ACC, PIECES, BS>), dim3((unsigned)blocks), dim3(BS), 0,
                     stream, a, magic);
}

template <int IN, int OUT, int WB, bool ACC>
hipError_t launch_fused_wb(const FusedArgs& a, bool vec, hipStream_t stream) {
  const int64_t rows = (int64_t)(a.owner_end - a.owner_begin) * (a.total_tokens / a.cp_size);
  const int64_t writer_bytes = rows * a.row_elems * (IN == CP_F32 ? 4 : 2);  // read from each writer
  // one-wave workgroups by size, pieces also by writer count (layout checked below)
  const bool large = writer_bytes >= kPieceMinBytes;
  const bool large_pieces = piece_layout<IN, OUT>() && large && a.cp_size <= kPieceMaxSlots;
  const std::string tag = std::string(ACC ? "fused_grad_return_acc<" : "fused_grad_return<") + dtype_tag(IN) +
                          "," + dtype_tag(OUT) + "," + std::to_string(WB) + ",";
  // [scalar, 4 waves per row, flat tiles of 1 or 2 units per thread, of pieces]
  static const std::string names[5] = {
      tag + "s>", tag + "v" + std::to_string(fused_upl(WB)) + "/" + std::to_string(kFusedWpr) + ">",
      tag + "flat1>", tag + "flat2>", tag + "pieces" + std::to_string(kFusedPiecesPerThread) + ">"};
  // Flat tiles need the rows a tile touches to fit kMaxTileRows and
  // (tile units + units_per_row) * units_per_row < 2^32 for the row split.
  auto flat_fits = [](int64_t upr, int64_t tile_units) {
    return upr > 0 && tile_units / upr + 2 <= kMaxTileRows && (tile_units + upr) * upr < (int64_t(1) << 32);
  };
  const bool vec_units = vec && a.row_elems % unit_group_elems<IN, OUT>() == 0;  // whole unit groups per row
  const bool pieces = large_pieces && vec && a.row_elems % piece_elems<IN>() == 0 &&
                      flat_fits(a.row_elems / piece_elems<IN>(), (int64_t)kSumBlock * kFusedPiecesPerThread);
  const int64_t upr = a.row_elems / (pieces ? piece_elems<IN>() : 8);  // units (pieces) per row
  const int np = pieces ? kFusedPiecesPerThread : a.cp_size <= 4 ? 2 : 1;
  const int64_t tile_units = (int64_t)(large ? kSumBlock : kBlock) * np;
  // kind 0: scalar; 1: 4 waves per row (very long rows); 2: flat tiles
  const int kind = pieces ? 2 : !vec_units ? 0 : !flat_fits(upr, tile_units) ? 1 : 2;
  int64_t blocks;
  if (kind == 2) {
    blocks = (rows * upr + tile_units - 1) / tile_units;
  } else {
    const int64_t rows_per_block = kind == 1 ? kWavesPerBlock / kFusedWpr : kWavesPerBlock;
    blocks = (rows + rows_per_block - 1) / rows_per_block;
  }
  if (blocks > kMaxGrid) blocks = kMaxGrid;
  if (blocks < 1) blocks = 1;
  const uint32_t magic = upr > 0 ? (uint32_t)(((uint64_t(1) << 32) + (uint64_t)upr - 1) / (uint64_t)upr) : 0;
  profile_before(names[kind == 2 ? (pieces ? 4 : 1 + np) : kind].c_str(), stream);
  if (kind == 2 && pieces) {
    if constexpr (piece_layout<IN, OUT>())
      launch_fused_flat<IN, OUT, WB, kFusedPiecesPerThread, ACC, true, kSumBlock>(a, blocks, magic, stream);
  } else if (kind == 2) {
    if (large) {
      if (np == 1) launch_fused_flat<IN, OUT, WB, 1, ACC, false, kSumBlock>(a, blocks, magic, stream);
      else launch_fused_flat<IN, OUT, WB, 2, ACC, false, kSumBlock>(a, blocks, magic, stream);
    } else {
      if (np == 1) launch_fused_flat<IN, OUT, WB, 1, ACC, false>(a, blocks, magic, stream);
      else launch_fused_flat<IN, OUT, WB, 2, ACC, false>(a, blocks, magic, stream);
    }
  } else if (kind == 1) {
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
