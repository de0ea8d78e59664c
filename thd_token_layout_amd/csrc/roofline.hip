// Plain streaming kernels for the benchmark's ceiling measurement: what one
// MI355X streams for a given read/write mix and size with the library's
// schedule (a full grid, one contiguous tile of kBlock * NP 16-byte units per
// workgroup, non-temporal loads) and the best of NP = 1, 2, 3 units per thread,
// of two store policies (non-temporal global stores, or buffer stores over the
// workgroup's tile with the nt and sc1 cache policy, measured faster on MI355X
// for a copy) and of two load schedules (a thread's loads all in flight, or one
// at a time, each waited for before the next: measured faster on MI355X for
// every mix with several loads per thread) and, with one unit per thread, of
// 256- and 64-thread workgroups.  A plain copy streams best with one unit per
// thread in 64-thread workgroups (1 KiB each); the library's kernels need 8-20
// KiB tiles to amortise their per-tile row lookup, so the ceiling is taken over
// the tile shapes, not at the library's.  The layout, scatter and sum kernels
// are compared with the stream of the same mix and size.  Built into its own
// library (libcpthd_roofline.so), not part of the cpthd boundary.
//
//   n_in inputs, an output:   out[u] = in_0[u] ^ ... ^ in_{n_in-1}[u]
//   n_in inputs, no output:   read only (each workgroup folds what it read
//                             into one word, stored only if it equals a value
//                             no input holds, so the loads stay)
//   no input, an output:      write only (a pattern of the unit index)
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 256;
constexpr int kMaxIn = 9;  // the W = 8 accumulate mix reads 8 gradients and the output
constexpr int64_t kMaxGrid = int64_t(1) << 22;

struct InPtrs {
  const u32x4* p[kMaxIn];
};

// Raw buffer descriptor word 3 (32-bit data format, no swizzle) and the store
// cache policy nt | sc1.
constexpr int kRawBufferWord3 = 0x00020000;
constexpr int kStoreNtSc1 = 2 | 16;

template <int NIN, bool WRITE, int NP, bool SC1, bool SER, int BS>
__global__ void __launch_bounds__(BS) stream_kernel(InPtrs in, u32x4* out, int64_t units, uint32_t* sink) {
  constexpr int64_t kTile = (int64_t)BS * NP;
  const int64_t ntiles = (units + kTile - 1) / kTile;
  u32x4 fold = {0u, 0u, 0u, 0u};
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    u32x4 v[NP];
    bool ok[NP];
#pragma unroll
    for (int m = 0; m < NP; ++m) {
      const int64_t u = tile * kTile + (int64_t)m * BS + threadIdx.x;
      ok[m] = u < units;
      v[m] = u32x4{(uint32_t)u, (uint32_t)(u >> 32), 0x9E3779B9u, 0x7F4A7C15u};
      if (NIN > 0 && ok[m]) {
        v[m] = __builtin_nontemporal_load(in.p[0] + u);
        if constexpr (SER) __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
        for (int k = 1; k < NIN; ++k) {
          v[m] ^= __builtin_nontemporal_load(in.p[k] + u);
          if constexpr (SER) __builtin_amdgcn_s_waitcnt(0);
        }
      }
    }
    if constexpr (WRITE && SC1) {
      // the tile's units [tile * kTile, min(+kTile, units)) through one buffer resource
      const int64_t t_units = units - tile * kTile < kTile ? units - tile * kTile : kTile;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          reinterpret_cast<char*>(out + tile * kTile), 0, (int)(t_units * 16), kRawBufferWord3);
#pragma unroll
      for (int m = 0; m < NP; ++m)
        if (ok[m]) __builtin_amdgcn_raw_buffer_store_b128(v[m], rs, (m * BS + (int)threadIdx.x) * 16, 0, kStoreNtSc1);
    } else {
#pragma unroll
      for (int m = 0; m < NP; ++m) {
        const int64_t u = tile * kTile + (int64_t)m * BS + threadIdx.x;
        if (WRITE && ok[m]) __builtin_nontemporal_store(v[m], out + u);
        if (!WRITE && ok[m]) fold ^= v[m];
      }
    }
  }
  if (!WRITE && fold.x == 0xFFFFFFFFu && fold.y == 0x00000001u && fold.z == 0xFFFFFFFFu && fold.w == 0x00000001u)
    sink[blockIdx.x & 1023] = fold.x ^ fold.w;
}

typedef void (*StreamFn)(InPtrs, u32x4*, int64_t, uint32_t*);

template <int NIN, int NP, bool SER, int BS = kBlock>
StreamFn pick_np(bool write, bool sc1) {
  return !write ? stream_kernel<NIN, false, NP, false, SER, BS>
                : sc1 ? stream_kernel<NIN, true, NP, true, SER, BS> : stream_kernel<NIN, true, NP, false, SER, BS>;
}

template <int NIN, bool SER>
StreamFn pick_ser(bool write, int np, bool sc1) {
  return np == 1   ? pick_np<NIN, 1, SER>(write, sc1)
         : np == 2 ? pick_np<NIN, 2, SER>(write, sc1)
                   : pick_np<NIN, 3, SER>(write, sc1);
}

// 64-thread workgroups: one unit per thread only.
template <int NIN>
StreamFn pick(bool write, int np, bool sc1, bool ser, bool small) {
  if (small) return ser ? pick_np<NIN, 1, true, 64>(write, sc1) : pick_np<NIN, 1, false, 64>(write, sc1);
  return ser ? pick_ser<NIN, true>(write, np, sc1) : pick_ser<NIN, false>(write, np, sc1);
}

}  // namespace

extern "C" {

// Stream n_in (0..9) inputs of `bytes` each into `out` (NULL: read only), or
// write `out` alone (n_in = 0), with `units_per_thread` (1..3) 16-byte units
// per thread and tile.  `policy` bit 0: buffer stores with nt | sc1 (else
// non-temporal global stores); bit 1: one load in flight per thread (else all
// of a thread's loads in flight together); bit 2: 64-thread workgroups (else
// 256; with one unit per thread only).  bytes must be a positive multiple
// of 16 and every pointer 16-byte aligned; read-only runs need `sink` (>= 4
// KiB, never written in practice).  Asynchronous on `stream`.  Returns 0, or -1
// on bad arguments (nothing launched), or the HIP error of the launch.
int cprl_stream(int n_in, const void* const* in, void* out, int64_t bytes, int units_per_thread, void* sink,
                int policy, hipStream_t stream) {
  if (n_in < 0 || n_in > kMaxIn || bytes <= 0 || bytes % 16 != 0) return -1;
  if (units_per_thread < 1 || units_per_thread > 3) return -1;
  if (policy < 0 || policy > 7) return -1;
  const bool small = (policy & 4) != 0;
  if (small && units_per_thread != 1) return -1;
  if (n_in == 0 && out == nullptr) return -1;
  if (out == nullptr && sink == nullptr) return -1;
  InPtrs p{};
  for (int k = 0; k < n_in; ++k) {
    if (in == nullptr || in[k] == nullptr || (reinterpret_cast<uintptr_t>(in[k]) & 15) != 0) return -1;
    p.p[k] = static_cast<const u32x4*>(in[k]);
  }
  if (out != nullptr && (reinterpret_cast<uintptr_t>(out) & 15) != 0) return -1;
  const int64_t units = bytes / 16;
  const int np = units_per_thread;
  const int64_t bs = small ? 64 : kBlock;
  int64_t blocks = (units + bs * np - 1) / (bs * np);
  if (blocks > kMaxGrid) blocks = kMaxGrid;
  const bool w = out != nullptr;
  const bool sc1 = (policy & 1) != 0;
  const bool ser = (policy & 2) != 0;
  StreamFn fns[kMaxIn + 1] = {
      pick<0>(true, np, sc1, ser, small), pick<1>(w, np, sc1, ser, small), pick<2>(w, np, sc1, ser, small),
      pick<3>(w, np, sc1, ser, small),    pick<4>(w, np, sc1, ser, small), pick<5>(w, np, sc1, ser, small),
      pick<6>(w, np, sc1, ser, small),    pick<7>(w, np, sc1, ser, small), pick<8>(w, np, sc1, ser, small),
      pick<9>(w, np, sc1, ser, small)};
  hipLaunchKernelGGL(fns[n_in], dim3((unsigned)blocks), dim3((unsigned)bs), 0, stream, p, static_cast<u32x4*>(out),
                     units, static_cast<uint32_t*>(sink));
  return (int)hipGetLastError();
}

}  // extern "C"
