// Index arithmetic of the row-chunk permutation kernel (permute.hip): which
// written row and 1 KiB chunk a workgroup moves, and that row's rank, local row
// and global row under a closed-form row map.  Host- and device-callable, so a
// host build checks it over whole grids (tests/chunk_map_host.hip).
//
// Closed forms ("[PyTorch] Add experimental packed-contiguous THD all-gather
// CP", section "Why"; "Add stream-ordered CP gradient return primitive",
// author's reply): packed-contiguous gives rank r the rows [r n, (r+1) n),
// n = T / W; dual-chunk-swap with one document of T rows cuts it into 2W
// chunks of c = n / 2 rows and gives rank r chunk r, then chunk 2W-1-r.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpthd {

struct ChunkDiv {
  uint32_t chunks;   // 1 KiB chunks per row
  uint32_t chunk_m;  // ceil(2^32 / chunks), unused for chunks = 1
  uint64_t n_m;      // ceil(2^64 / n), 0 for n = 1
  uint64_t c_m;      // ceil(2^64 / (n / 2)), 0 for n / 2 = 1 (dual-chunk-swap only)
};

// floor(x / d) for m = ceil(2^64 / d), 2 <= d < 2^32, and for m = 0 (d = 1).
// Exact for every 32-bit x: x m / 2^64 exceeds x / d by x (m d - 2^64) / (d 2^64)
// < 2^-32, while the fraction of x / d is at most 1 - 1/d < 1 - 2^-32.  The
// high half of the 96-bit product comes from two 32 x 32 products without
// overflow.
__host__ __device__ inline uint32_t div_by_magic(uint32_t x, uint64_t m) {
  if (m == 0) return x;
  const uint64_t t = (uint64_t)x * (uint32_t)(m >> 32) + (((uint64_t)x * (uint32_t)m) >> 32);
  return (uint32_t)(t >> 32);
}

__host__ inline uint64_t magic_of(uint64_t d) {
  if (d <= 1) return 0;
  return (uint64_t)((((unsigned __int128)1 << 64) + d - 1) / d);
}

// Largest grid of row-chunk workgroups: HIP caps a grid's x extent at 2^32 - 1
// threads, 64 per workgroup here.
constexpr int64_t kChunkMaxGrid = (int64_t(1) << 26) - 1;

// The divisions for T rows of `upr` 16-byte units, n = T / W rows per rank;
// false when the row chunks do not apply: rows not a multiple of 1 KiB, odd n
// under dual-chunk-swap, a grid beyond kChunkMaxGrid, or a grid on which the
// row division by multiply-high would not be exact (workgroup b's row is
// b * chunk_m / 2^32, exact while b (chunk_m chunks - 2^32) < 2^32, which
// T chunks^2 < 2^32 guarantees).
__host__ inline bool chunk_div(int64_t T, int64_t n, bool dcs, int64_t upr, ChunkDiv* dv) {
  if (T <= 0 || n <= 0 || upr <= 0 || upr % 64 != 0 || (dcs && n % 2 != 0)) return false;
  const int64_t chunks = upr / 64;
  if (T > kChunkMaxGrid / chunks || T * chunks * chunks >= (int64_t(1) << 32)) return false;
  dv->chunks = (uint32_t)chunks;
  dv->chunk_m = chunks == 1 ? 0u : (uint32_t)(((uint64_t(1) << 32) + (uint64_t)chunks - 1) / (uint64_t)chunks);
  dv->n_m = magic_of((uint64_t)n);
  dv->c_m = dcs ? magic_of((uint64_t)(n / 2)) : 0;
  return true;
}

// Written row of workgroup b (its chunk is b - row * chunks).
__host__ __device__ inline uint32_t chunk_row(uint32_t b, const ChunkDiv& dv) {
  return dv.chunks == 1 ? b : (uint32_t)(((uint64_t)b * dv.chunk_m) >> 32);
}

struct ChunkRow {
  int32_t r;  // rank
  int64_t i;  // local row of rank r
  int64_t g;  // global row
};

// Row p of the written side under the closed form: a global row under GORDER
// (the gather), else a flat local row r n + i (partition, scatter).
template <bool GORDER>
__host__ __device__ inline ChunkRow chunk_map(uint32_t p, int32_t W, int64_t n, bool dcs, const ChunkDiv& dv) {
  ChunkRow m;
  m.g = p;
  if (GORDER && dcs) {
    const int64_t c = n >> 1;
    const int32_t k = (int32_t)div_by_magic(p, dv.c_m);  // chunk of the document
    const int64_t j = (int64_t)p - (int64_t)k * c;
    if (k < W) { m.r = k; m.i = j; }
    else { m.r = 2 * W - 1 - k; m.i = c + j; }
  } else {
    m.r = (int32_t)div_by_magic(p, dv.n_m);
    m.i = (int64_t)p - (int64_t)m.r * n;
    if (!GORDER && dcs) {
      const int64_t c = n >> 1;
      m.g = m.i < c ? (int64_t)m.r * c + m.i : (int64_t)(2 * W - 1 - m.r) * c + (m.i - c);
    }
  }
  return m;
}

}  // namespace cpthd
