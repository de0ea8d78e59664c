// Internal interface between the C-ABI layer (abi.cpp) and the HIP kernels.
// Host code only sees launch functions; kernels live in the .hip files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cpthd.h"

namespace cpthd {

constexpr int kMaxRanks = CP_MAX_CP_SIZE;
constexpr int kBlock = 256;           // threads per workgroup: 4 wave64s
constexpr int kWavesPerBlock = kBlock / 64;
// Largest grid launched; kernels loop (grid-stride) over work beyond it.  Keeps
// blocks * kBlock well inside the 32-bit grid size.
constexpr int64_t kMaxGrid = int64_t(1) << 22;

// Byte offsets inside the metadata buffer (layout documented in cpthd.h).
__host__ __device__ inline int64_t meta_cu_offset() { return 64; }
__host__ __device__ inline int64_t meta_local_cu_offset(int32_t B) { return 64 + 4 * ((int64_t)B + 1); }
__host__ __device__ inline int64_t meta_n_local_offset(int32_t B, int32_t W) {
  return 64 + 4 * ((int64_t)B + 1) * ((int64_t)W + 1);
}
// Unit tiles stage the dual-chunk-swap document tables of up to this many
// documents in LDS (when they do not use the row maps).
constexpr int32_t kStagedMaxDocs = 64;

// cp_meta_bytes(B, W): header and tables, rounded up to 256 bytes; the
// optional row maps (row_of_local[T], then local_of_row[T]) start there.
__host__ __device__ inline int64_t meta_tables_bytes(int32_t B, int32_t W) {
  return (meta_n_local_offset(B, W) + 4 * (int64_t)W + 255) / 256 * 256;
}

// Fixed-capacity pointer table passed by value in the kernel arguments.
struct RankPtrs {
  char* p[kMaxRanks];
};
struct ConstRankPtrs {
  const char* p[kMaxRanks];
};

// Bytes per element of a cp_dtype (0 for unsupported).
inline int dtype_bytes(int32_t dt) {
  switch (dt) {
    case CP_F32: return 4;
    case CP_BF16: return 2;
    case CP_F16: return 2;
    default: return 0;
  }
}

// ---------------------------------------------------------------- metadata
// row_maps: also write the row maps after the tables (dual-chunk-swap only;
// the caller has checked that the buffer holds them).
hipError_t launch_build_meta(const int32_t* cu, int32_t B, int64_t T, int32_t W, int32_t policy,
                             bool row_maps, void* meta, hipStream_t stream);

// Attention-step records (layout documented in cpthd.h): 64-byte header, then
// 2W records of 32 + 16(B+1) bytes.
__host__ __device__ inline int64_t attn_record_bytes(int32_t B) { return 32 + 16 * ((int64_t)B + 1); }
__host__ __device__ inline int64_t attn_record_offset(int32_t B, int32_t index) {
  return 64 + (int64_t)index * attn_record_bytes(B);
}
hipError_t launch_build_attn_meta(cp_meta_header* meta, int32_t B, int32_t W, void* attn, hipStream_t stream);

// ---------------------------------------------------------------- row permutation
// One launch moves all T rows of n_tensors tensors (same T, row size and
// layout) between the global layout and the per-rank layout.  global[t] is
// tensor t's x ([T, row]); the local side is either one contiguous
// [W, T/W, row] buffer per tensor (local_table == false, local[t]) or, for a
// single tensor, one [T/W, row] buffer per rank (local_table == true, table).
// to_local: partition / scatter (global -> local); otherwise gather.
constexpr int kMaxLayoutTensors = 8;
struct PermuteArgs {
  cp_meta_header* meta;
  int32_t n_tensors;
  char* global[kMaxLayoutTensors];
  char* local[kMaxLayoutTensors];
  RankPtrs table;
  bool local_table;
  bool to_local;
  int64_t total_tokens;
  int64_t row_bytes;
  int32_t expect_cp_size;   // -1: any
  int32_t expect_policy;    // -1: any
  // Host-side record of the metadata (policy, document count and CP size when
  // the host built it at this address; -1 / 0: unknown).  Chooses the tile
  // shape; the unit-tile kernels also start their first lookups from it and
  // check it against the header before they touch the tensors.
  int32_t hint_policy;
  int32_t hint_docs;
  int32_t hint_cp_size;
  int64_t hint_local_tokens;  // T / W of the record
  bool hint_row_maps;         // the metadata was built with its row maps
};
hipError_t launch_permute(const PermuteArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- reductions
// out[k] = sum_w in[w][k] in fp32, w = 0..W-1 in order, seeded with in[0].
struct SlotSumArgs {
  ConstRankPtrs in;
  char* out;
  int32_t num_slots;
  int64_t n_elems;
  int32_t in_dtype;
  int32_t out_dtype;
  // Optional fail-closed gate (gradient return): when gate_meta is set the
  // kernel writes nothing unless the meta is valid metadata for gate_T tokens
  // and num_slots ranks, and, when owner >= 0, bit `owner` of
  // meta->wait_timeout_ranks is clear.
  cp_meta_header* gate_meta;
  int64_t gate_T;
  int32_t owner;
  int32_t accumulate;  // nonzero: out = ((out + s_0) + s_1) + ... (out read first)
};
hipError_t launch_slot_sum(const SlotSumArgs& a, hipStream_t stream);

// Fused scatter+sum: out[o][i] = sum_w grads[w][g_o(i)] for owners o in
// [owner_begin, owner_end).
struct FusedArgs {
  cp_meta_header* meta;
  ConstRankPtrs grads;  // [W] writer views, [T, row]
  RankPtrs out;         // [W] owner outputs, [T/W, row] (entries outside the owner range unused)
  int32_t cp_size;
  int32_t owner_begin;
  int32_t owner_end;
  int64_t total_tokens;
  int64_t row_elems;
  int32_t in_dtype;
  int32_t out_dtype;
  int32_t accumulate;  // nonzero: the owner's current out seeds the sum
};
hipError_t launch_fused(const FusedArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- all-reduce
// W rank buffers of n elements (f32 or bf16), every rank's out = the sum of
// all W inputs.  One-shot: one launch, rank r reads all inputs and sums them
// in rank order.  Ring: W chunks of `chunk` elements (the last ones possibly
// short or empty); a reduce-scatter step s has rank r add its own input to
// chunk (r-1-s) mod W received from rank r-1; an all-gather step s has rank r
// copy chunk (r-s) mod W from rank r-1.
struct AllreduceArgs {
  ConstRankPtrs in;   // [W] inputs, n elements each
  RankPtrs out;       // [W] outputs, n elements each (ring: the working buffers)
  int32_t cp_size;
  int64_t n_elems;
  int64_t chunk;      // ring chunk length in elements, ceil(n / W); chunks start anywhere
  int32_t dtype;      // CP_F32 or CP_BF16, inputs and outputs alike
  int32_t vec;        // all pointers 16-byte aligned (set by the launch functions)
};
hipError_t launch_allreduce_one_shot(const AllreduceArgs& a, hipStream_t stream);
// Two-shot: rank r sums chunk r of all inputs in rank order into out[r]
// (one launch), then every rank copies the other ranks' chunks (one launch).
hipError_t launch_allreduce_two_shot(const AllreduceArgs& a, hipStream_t stream);
// Reduce-scatter step `step` (0..W-2) of the ring for all ranks in one launch.
hipError_t launch_ring_reduce_step(const AllreduceArgs& a, int32_t step, hipStream_t stream);
// All-gather step `step` (0..W-2) for all ranks; with from_input (W = 1 only)
// every rank copies its own input instead.
hipError_t launch_ring_gather_step(const AllreduceArgs& a, int32_t step, bool from_input,
                                   hipStream_t stream);

// The ring in one launch.  Workgroup (rank r, tile t) runs rank r's 2(W-1)
// steps on tile t of each chunk and signals every finished step through a
// device flag; before a step it waits for rank r-1's flag of the same tile.
// signals (uint64 words): [0] largest epoch in which a wait timed out, [1]
// largest epoch found stale (not above the flags left by an earlier call),
// [2 + r * kSignalTiles + t] = (epoch << 8) + steps finished by (r, t).
constexpr int kSignalTiles = 256;
inline int64_t signal_words(int32_t W) { return 2 + (int64_t)W * kSignalTiles; }
struct RingSignalArgs {
  uint64_t* signals;
  uint64_t epoch;
  int64_t timeout_ticks;  // per wait, device wall-clock ticks
  int64_t tile_elems;     // elements per tile, a multiple of 512
};
// Tiles per rank, from co-residency on the current device and the chunk length.
int ring_signal_tiles(const AllreduceArgs& a, int64_t* tile_elems);
hipError_t launch_ring_signal(const AllreduceArgs& a, const RingSignalArgs& g, int tiles, hipStream_t stream);

// ---------------------------------------------------------------- epochs
// Writer `writer` (or every writer when writer < 0) stores `epoch` into
// epochs[o][writer] for every owner o, with release ordering.
hipError_t launch_epoch_publish(uint32_t* epochs, int32_t W, int32_t writer, uint32_t epoch,
                                hipStream_t stream);
// Owner `owner` (or every owner when owner < 0) waits until epochs[o][w] >=
// epoch for all w, or until timeout_ticks of the device wall clock pass; then
// records the owners still pending in meta->wait_timeout_ranks.
hipError_t launch_epoch_wait(const uint32_t* epochs, int32_t W, int32_t owner, uint32_t epoch,
                             int64_t timeout_ticks, cp_meta_header* meta, hipStream_t stream);

// ---------------------------------------------------------------- static workspace
// Device address (on the current device) of the library's static workspace of
// kNoallocScratchBytes bytes, 256-byte aligned (scratch.hip); looked up once
// per device.
constexpr int64_t kNoallocScratchBytes = (int64_t)CP_NOALLOC_SCRATCH_BYTES;
hipError_t noalloc_scratch(void** ptr);

// ---------------------------------------------------------------- timing hooks
// Called by every launch function around its kernel launch.
void profile_before(const char* name, hipStream_t stream);
void profile_after(hipStream_t stream);

}  // namespace cpthd
