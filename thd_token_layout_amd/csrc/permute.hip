// Row-permutation copy engine: THD partition, inverse gather and the
// gradient-return scatter.
//
// The row map (ownership rule and its formula) is in device_common.h: under
// dual-chunk-swap rank r holds chunk r then chunk 2W-1-r of every document;
// under packed-contiguous rank r holds tokens [r n, (r+1) n), n = T/W.
//
// Design (gfx950): pure data movement, HBM-bound.  Three tilings, all with a
// full grid (one tile per workgroup; measured on MI355X, concurrently running
// workgroups then stream one contiguous window of HBM, while a resident-
// capacity grid-stride loop, or several tiles per workgroup, streamed 5-20%
// slower):
//  - row chunks (permute_chunk_kernel): where the row map has a closed form
//    (packed-contiguous, one-document dual-chunk-swap), one wave moves 1 KiB
//    of one row, mapped by the formula in wave-uniform code (see there);
//  - unit tiles (permute_flat_kernel): a workgroup owns a fixed number of
//    16-byte units whatever the row length, with the touched rows looked up
//    into LDS; used where that lookup is cheap (see there);
//  - row tiles (permute_rows_kernel): a workgroup (4 waves) owns 8-20 KiB of
//    consecutive local rows; the row map is computed once per group in
//    wave-uniform code, a search of the per-rank document table and then an
//    incremental cursor, so each wave runs independently.
// Lanes move 16-byte units with non-temporal loads, fully coalesced (a wave
// touches 1 KiB contiguous per instruction); in the row chunks and unit tiles
// each lane has one load in flight at a time (see there).  Row tiles store
// with non-temporal global stores; row chunks and unit tiles store their
// contiguous units through a buffer resource with the nt and sc1 cache policy
// (measured on MI355X: 1.5-4% faster for unit tiles, slower for row tiles).
#include "chunk_map.h"
#include "device_common.h"


namespace cpthd {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Raw buffer resources: word 3 of the descriptor (32-bit data format, no
// swizzle) and the cache-policy operand of a store (2 = nt, 16 = sc1).
constexpr int kRawBufferWord3 = 0x00020000;
constexpr int kStoreNtSc1 = 2 | 16;

// A pointer every lane holds the same value of, as a wave-uniform value.
__device__ __forceinline__ char* uniform_ptr(char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return reinterpret_cast<char*>(((uint64_t)hi << 32) | lo);
}

template <typename U>
__device__ __forceinline__ U load_nt(const U* p) {
  return __builtin_nontemporal_load(p);
}
template <typename U>
__device__ __forceinline__ void store_nt(U* p, U v) {
  __builtin_nontemporal_store(v, p);
}

// Wave-uniform cursor over the flat local row index p = r*n + i.
struct Cursor {
  int32_t r;        // rank
  int64_t i;        // local row inside the rank
  int32_t b;        // document (dual-chunk-swap only)
  int64_t lstart;   // local_cu[b]
  int64_t lend;     // local_cu[b+1]
  int64_t gstart;   // cu[b]
  int64_t c;        // chunk length of document b
};

__device__ __forceinline__ void load_doc(Cursor& k, const int32_t* cu, const int32_t* lcu) {
  k.lstart = lcu[k.b];
  k.lend = lcu[k.b + 1];
  k.gstart = cu[k.b];
  k.c = (k.lend - k.lstart) >> 1;
}

// find_doc run by a whole wave at once (wave-uniform arguments, every lane
// active): each round the 64 lanes test 64 entries of `bound` at a stride that
// shrinks 63-fold from ceil((B+1)/63) to 1 and keep the last entry <= v, so
// the search costs ceil(log63(B+1)) dependent loads instead of log2(B).
// Measured on MI355X for the row tiles in local order: the 10 KiB-row gradient
// scatter 1-5% faster at 116-32768 documents, the layouts' partition
// unchanged; in global order (the gather) 1-2% slower, so the gather keeps
// find_doc.
__device__ __forceinline__ int32_t wave_find_doc(const int32_t* bound, int32_t B, int64_t v) {
  const int lane = threadIdx.x & 63;
  int32_t lo = 0;  // bound[lo] <= v throughout
  for (int32_t s = (int32_t)(((int64_t)B + 63) / 63);; s = (s + 62) / 63) {
    const int64_t idx = (int64_t)lo + (int64_t)lane * s;
    const bool le = idx < B && (int64_t)bound[idx] <= v;
    const int cnt = __popcll(__ballot(le));
    lo += (cnt > 1 ? cnt - 1 : 0) * s;
    if (s == 1) return lo;
  }
}

// WAVE: the caller is a whole wave with wave-uniform arguments.
template <bool WAVE>
__device__ __forceinline__ void seek(Cursor& k, int64_t p, int64_t n, int32_t B, bool dcs,
                                     const int32_t* cu, const int32_t* lcu) {
  k.r = (int32_t)(p / n);
  k.i = p - (int64_t)k.r * n;
  if (!dcs) return;
  k.b = WAVE ? wave_find_doc(lcu, B, k.i) : find_doc(lcu, B, k.i);
  load_doc(k, cu, lcu);
}

__device__ __forceinline__ void advance(Cursor& k, int64_t n, bool dcs, const int32_t* cu,
                                        const int32_t* lcu) {
  ++k.i;
  if (k.i == n) {
    ++k.r;
    k.i = 0;
    if (dcs) { k.b = 0; load_doc(k, cu, lcu); }
  }
  if (dcs) {
    while (k.i >= k.lend) { ++k.b; load_doc(k, cu, lcu); }
  }
}

__device__ __forceinline__ int64_t global_row(const Cursor& k, int32_t W, int64_t n, bool dcs) {
  if (!dcs) return (int64_t)k.r * n + k.i;
  const int64_t j = k.i - k.lstart;
  return j < k.c ? k.gstart + (int64_t)k.r * k.c + j
                 : k.gstart + (int64_t)(2 * W - 1 - k.r) * k.c + (j - k.c);
}

// Wave-uniform cursor in global order (used when the global side is the
// destination, so the writes are sequential): global row t lies in document b
// at offset off = t - cu[b], in chunk k = off / c_b at position j; chunk k
// belongs to rank k (k < W) or 2W-1-k, and sits at local row
// local_cu[b] + j (first chunk of the rank) or local_cu[b] + c_b + j.
struct GCursor {
  int64_t t;
  int32_t b;
  int64_t dstart;  // cu[b]
  int64_t lstart;  // local_cu[b]
  int64_t c;       // chunk length of document b
  int32_t k;       // chunk index in [0, 2W)
  int64_t j;       // position inside the chunk
};

__device__ __forceinline__ void gload_doc(GCursor& g, const int32_t* cu, const int32_t* lcu) {
  g.dstart = cu[g.b];
  g.lstart = lcu[g.b];
  g.c = (lcu[g.b + 1] - lcu[g.b]) >> 1;
}

__device__ __forceinline__ void gseek(GCursor& g, int64_t t, int32_t B, const int32_t* cu,
                                      const int32_t* lcu) {
  g.t = t;
  g.b = find_doc(cu, B, t);
  gload_doc(g, cu, lcu);
  const int64_t off = t - g.dstart;
  g.k = (int32_t)(off / g.c);
  g.j = off - (int64_t)g.k * g.c;
}

__device__ __forceinline__ void gadvance(GCursor& g, int32_t W, const int32_t* cu, const int32_t* lcu) {
  ++g.t;
  if (++g.j == g.c) {
    g.j = 0;
    if (++g.k == 2 * W) {
      g.k = 0;
      do { ++g.b; gload_doc(g, cu, lcu); } while (g.c == 0);
    }
  }
}

// Local position (rank, row) of the cursor's global row.
__device__ __forceinline__ void glocal(const GCursor& g, int32_t W, int32_t* r, int64_t* i) {
  if (g.k < W) { *r = g.k; *i = g.lstart + g.j; }
  else { *r = 2 * W - 1 - g.k; *i = g.lstart + g.c + g.j; }
}

// One workgroup = 4 waves = a tile of (4 / WPR) * G consecutive local rows.
// Waves are grouped WPR to a row: wave w takes rows [p_tile + (w / WPR) G, +G)
// and, inside each row, the column chunks c = w % WPR, c + WPR, ... of 64*VPL
// units each, so every lane has up to G*VPL loads in flight.
template <typename U, int VPL, int G, int WPR, bool GORDER>
__global__ void __launch_bounds__(kBlock) permute_rows_kernel(PermuteArgs a) {
  static_assert(kWavesPerBlock % WPR == 0, "WPR must divide the waves of a workgroup");
  constexpr int kRowsPerTile = (kWavesPerBlock / WPR) * G;
  cp_meta_header* h = a.meta;
  if (!meta_ok(h, a.total_tokens, a.expect_cp_size, a.expect_policy)) return;

  const int64_t T = a.total_tokens;
  const int32_t W = h->cp_size;
  const int32_t B = h->num_docs;
  const int64_t n = h->local_tokens;
  const bool dcs = h->policy == CP_POLICY_DUAL_CHUNK_SWAP;
  const int32_t* cu = meta_cu(h);
  const int32_t* lcu = meta_local_cu0(h, B);
  const int64_t upr = a.row_bytes / (int64_t)sizeof(U);  // units per row

  const int lane = threadIdx.x & 63;
  const int wave = wave_uniform(threadIdx.x >> 6);
  const int row_slot = wave / WPR;
  const int chunk = wave % WPR;
  const int64_t ntiles = (T + kRowsPerTile - 1) / kRowsPerTile;

  const int tsr = blockIdx.y;  // tensor of this workgroup's tiles
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t p0 = tile * kRowsPerTile + (int64_t)row_slot * G;
    if (p0 >= T) continue;
    char* const gbase = a.global[tsr];
    char* const lbase = a.local[tsr];
    const U* src[G];
    U* dst[G];
    bool ok[G];
    if constexpr (GORDER) {
      // p0 indexes global rows; rows are visited in global order.
      GCursor gc;
      int64_t pcr = 0, pci = 0;  // packed-contiguous: rank and local row
      if (dcs) gseek(gc, p0, B, cu, lcu);
      else { pcr = p0 / n; pci = p0 - pcr * n; }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        ok[g] = p0 + g < T;
        src[g] = nullptr;
        dst[g] = nullptr;
        if (ok[g]) {
          int32_t r;
          int64_t i;
          if (dcs) glocal(gc, W, &r, &i);
          else { r = (int32_t)pcr; i = pci; }
          char* gptr = gbase + (p0 + g) * a.row_bytes;
          char* lptr = a.local_table ? a.table.p[r] + i * a.row_bytes
                                     : lbase + ((int64_t)r * n + i) * a.row_bytes;
          src[g] = reinterpret_cast<const U*>(a.to_local ? gptr : lptr);
          dst[g] = reinterpret_cast<U*>(a.to_local ? lptr : gptr);
          if (g + 1 < G && p0 + g + 1 < T) {
            if (dcs) gadvance(gc, W, cu, lcu);
            else if (++pci == n) { pci = 0; ++pcr; }
          }
        }
      }
    } else {
      // p0 indexes local rows (flat r*n + i); rows are visited in local order.
      Cursor k;
      seek<true>(k, p0, n, B, dcs, cu, lcu);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        ok[g] = p0 + g < T;
        src[g] = nullptr;
        dst[g] = nullptr;
        if (ok[g]) {
          char* gptr = gbase + global_row(k, W, n, dcs) * a.row_bytes;
          char* lptr = a.local_table ? a.table.p[k.r] + k.i * a.row_bytes
                                     : lbase + ((int64_t)k.r * n + k.i) * a.row_bytes;
          src[g] = reinterpret_cast<const U*>(a.to_local ? gptr : lptr);
          dst[g] = reinterpret_cast<U*>(a.to_local ? lptr : gptr);
          if (g + 1 < G && p0 + g + 1 < T) advance(k, n, dcs, cu, lcu);
        }
      }
    }
    for (int64_t cb = (int64_t)chunk * 64 * VPL; cb < upr; cb += (int64_t)WPR * 64 * VPL) {
      U buf[G][VPL];
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int m = 0; m < VPL; ++m) {
          const int64_t col = cb + lane + 64 * m;
          if (ok[g] && col < upr) buf[g][m] = load_nt(src[g] + col);
        }
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int m = 0; m < VPL; ++m) {
          const int64_t col = cb + lane + 64 * m;
          if (ok[g] && col < upr) store_nt(dst[g] + col, buf[g][m]);
        }
    }
  }
}

// Unit-granular variant: the rows x units space of the side being written is
// cut into tiles of kBlock*NP consecutive 16-byte units (a tile may start and
// end inside a row), so the tile size no longer depends on the row length.  The
// first threads of the workgroup look up the source and destination of the
// <= kFlatMaxRows rows a tile touches and share them through LDS; the row of a
// unit is a multiply-high by `upr_magic` = ceil(2^32 / units_per_row), exact
// while (tile units + units_per_row) * units_per_row < 2^32.  The lookups sit
// on the workgroup's critical path (one barrier per tile), so under
// dual-chunk-swap the document tables (<= kFlatMaxDocs documents) are first
// staged in LDS with one coalesced load and searched there.  Measured on
// MI355X against the row tiles: +4..13% for packed-contiguous and
// single-document metadata, +3..5% at 32-64 documents, slower from ~128
// documents (the staging then costs more than it saves).
constexpr int kFlatMaxRows = 16;
constexpr int kFlatMaxDocs = kStagedMaxDocs;

// The metadata's shape as the unit-tile kernel uses it, and which dual-chunk-
// swap lookup follows from it: the row maps when the metadata has them (one
// load per row), else the document tables, staged in LDS when small enough
// (searched there), else searched in the metadata.
struct FlatShape {
  int32_t W, B, policy;
  int64_t n;  // T / W
  bool dcs, maps, staged;
};

template <bool MAPS>
__device__ __forceinline__ FlatShape flat_shape(int32_t W, int32_t B, int32_t policy, int64_t n, int32_t row_maps) {
  FlatShape s;
  s.W = W;
  s.B = B;
  s.policy = policy;
  s.n = n;
  s.dcs = policy == CP_POLICY_DUAL_CHUNK_SWAP;
  s.maps = MAPS && s.dcs && row_maps == 1;
  s.staged = s.dcs && !s.maps && B <= kFlatMaxDocs;
  return s;
}

// MAPS: the instantiation for metadata the host built with row maps (a
// separate kernel, so profiles tell the two lookups apart); it still checks the
// header and searches the tables when the maps are absent.
//
// When the host has a record of the metadata (its shape when the host built
// it at this address, in the hint_* arguments), the first tile's lookups start
// from that shape while the header is still in flight, and the header is
// checked before anything is loaded from the tensors: a header that fails the
// check stops the kernel, one whose shape differs from the record (the buffer
// rewritten since) has the lookups redone from the header.  Every load issued
// before the check stays inside the metadata extent the host checked for the
// record, or inside the tensors.  The header is read into LDS (no registers
// held while it is in flight, so occupancy stays at 8 waves per SIMD), and the
// gradient scatter's per-owner pointers are staged in LDS with it.  Measured
// on MI355X against the header read first and the pointers read per row: the
// gradient scatter 2-3% faster, the row-map layouts 1-1.5%.
// TABLE: the gradient scatter's instantiation (the local side is a per-owner
// pointer table); the layouts' instantiations carry no table code.
template <int NP, bool GORDER, bool MAPS, bool TABLE>
__global__ void __launch_bounds__(kBlock) permute_flat_kernel(PermuteArgs a, uint32_t upr_magic) {
  __shared__ const u32x4* s_src[kFlatMaxRows];
  __shared__ u32x4* s_dst[kFlatMaxRows];
  __shared__ int32_t s_rank[kFlatMaxRows];
  __shared__ int32_t s_cu[kFlatMaxDocs + 1];
  __shared__ int32_t s_lcu[kFlatMaxDocs + 1];
  __shared__ char* s_owner[kMaxRanks];
  __shared__ uint32_t s_header[kWavesPerBlock][16];
  cp_meta_header* h = a.meta;
  uint32_t* const my_header = s_header[wave_uniform(threadIdx.x >> 6)];
  const int64_t T = a.total_tokens;
  // The host launches this kernel only with a record; without one the lookups
  // start from a one-rank packed-contiguous shape (no table reads), which the
  // header then replaces.
  const bool hinted = a.hint_policy >= 0 && a.hint_cp_size > 0 && a.hint_docs >= 1 && a.hint_local_tokens > 0;
  FlatShape s = flat_shape<MAPS>(hinted ? a.hint_cp_size : 1, hinted ? a.hint_docs : 1,
                                 hinted ? a.hint_policy : (int32_t)CP_POLICY_PACKED_CONTIGUOUS,
                                 hinted ? a.hint_local_tokens : T, hinted && a.hint_row_maps ? 1 : 0);
  bool checked = false;
  // LDS copies of the per-owner pointers (gradient scatter) and of the
  // document tables (staged lookups): every load is issued before the first
  // LDS write waits for them.  The row-map instantiation stages nothing before
  // its first lookups (the host launches it for metadata recorded with maps),
  // so its header read stays in flight through them.
  static_assert(kBlock > kMaxRanks && kBlock > kFlatMaxDocs, "one element per thread");
  auto stage = [&](bool owners) {
    const int k = threadIdx.x;
    char* own = nullptr;
    int32_t c = 0, l = 0;
    if (owners && k < kMaxRanks) own = a.table.p[k];
    if (s.staged && k <= s.B) {
      c = meta_cu(h)[k];
      l = meta_local_cu0(h, s.B)[k];
    }
    if (owners && k < kMaxRanks) s_owner[k] = own;
    if (s.staged && k <= s.B) {
      s_cu[k] = c;
      s_lcu[k] = l;
    }
  };
  // A barrier waits for every load into LDS in flight: the instantiations
  // that stage tables issue the header read with them, the row-map one after
  // its first barrier, ahead of its first lookups.
  if constexpr (TABLE || !MAPS) {
    load_header_lds(h, my_header);
    stage(TABLE);
  }
  const int64_t upr = a.row_bytes / 16;
  const int64_t total = T * upr;
  constexpr int64_t kTileUnits = (int64_t)kBlock * NP;
  const int64_t ntiles = (total + kTileUnits - 1) / kTileUnits;
  const int tsr = blockIdx.y;
  char* const gbase = a.global[tsr];
  char* const lbase = a.local[tsr];

  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t u0 = tile * kTileUnits;
    const int64_t row0 = u0 / upr;
    const int64_t u_end = u0 + kTileUnits < total ? u0 + kTileUnits : total;
    const int nrows = (int)((u_end - 1) / upr - row0 + 1);
    for (;;) {
      __syncthreads();  // staged tables written; the previous tile's s_src / s_dst consumed
      if constexpr (MAPS && !TABLE) {
        if (!checked) load_header_lds(h, my_header);
      }
      if ((int)threadIdx.x < nrows) {
        const int32_t W = s.W, B = s.B;
        const int64_t n = s.n;
        const int32_t* cu = s.staged ? s_cu : meta_cu(h);
        const int32_t* lcu = s.staged ? s_lcu : meta_local_cu0(h, B);
        // row p of the written side: a global row (gather) or a flat local row r*n + i
        const int64_t p = row0 + threadIdx.x;
        int32_t r;
        int64_t i, g;
        if (s.maps) {
          // map entries are clamped to [0, T): rows stay inside the tensors
          // whatever the buffer holds
          const int32_t* row_of_local = reinterpret_cast<const int32_t*>(reinterpret_cast<const char*>(h) +
                                                                         meta_tables_bytes(B, W));
          const int32_t* local_of_row = row_of_local + T;
          const int64_t q = GORDER ? (int64_t)local_of_row[p] : p;
          const int64_t qc = q < 0 ? 0 : (q >= T ? T - 1 : q);
          r = (int32_t)(qc / n);
          i = qc - (int64_t)r * n;
          if constexpr (GORDER) {
            g = p;
          } else {
            const int64_t gm = row_of_local[p];
            g = gm < 0 ? 0 : (gm >= T ? T - 1 : gm);
          }
        } else if constexpr (GORDER) {
          g = p;
          if (s.dcs) {
            GCursor gc;
            gseek(gc, p, B, cu, lcu);
            glocal(gc, W, &r, &i);
          } else {
            r = (int32_t)(p / n);
            i = p - (int64_t)r * n;
          }
        } else {
          Cursor k;
          seek<false>(k, p, n, B, s.dcs, cu, lcu);
          r = k.r;
          i = k.i;
          g = global_row(k, W, n, s.dcs);
        }
        r = r < 0 ? 0 : (r >= W ? W - 1 : r);  // only a shape the header has not confirmed yet strays
        char* gptr = gbase + g * a.row_bytes;
        char* lptr = TABLE ? s_owner[r] + i * a.row_bytes : lbase + ((int64_t)r * n + i) * a.row_bytes;
        s_src[threadIdx.x] = reinterpret_cast<const u32x4*>(a.to_local ? gptr : lptr);
        s_dst[threadIdx.x] = reinterpret_cast<u32x4*>(a.to_local ? lptr : gptr);
        s_rank[threadIdx.x] = r;
      }
      if (checked) break;
      // the record's shape, checked against the header (uniform: every
      // workgroup takes the same branch)
      checked = true;
      const cp_meta_header hv = header_from_lds(my_header);
      if (!meta_ok(h, hv, T, a.expect_cp_size, a.expect_policy)) return;
      const FlatShape hs = flat_shape<MAPS>(hv.cp_size, hv.num_docs, hv.policy, hv.local_tokens, hv.row_maps);
      if (hs.W == s.W && hs.B == s.B && hs.policy == s.policy && hs.n == s.n && hs.maps == s.maps) break;
      s = hs;
      __syncthreads();  // every lookup above done before the tables are restaged
      stage(false);
    }
    __syncthreads();
    const int64_t base = u0 - row0 * upr;  // offset of the tile's first unit inside row0
    u32x4 v[NP];
    int row[NP];
    int64_t col[NP];
    bool ok[NP];
    // One load in flight per lane: each is waited for before the next is
    // issued.  Measured on MI355X: 3-7% faster than the tile's loads all in
    // flight (the same trend as plain streams, which run fastest with one
    // 16-byte load in flight per lane: HBM saturates with ~8 MiB in flight, and
    // more only queues).
#pragma unroll
    for (int m = 0; m < NP; ++m) {
      const uint32_t f = (uint32_t)(base + (int64_t)m * kBlock + threadIdx.x);
      ok[m] = u0 + (int64_t)m * kBlock + threadIdx.x < u_end;
      row[m] = ok[m] ? (int)__umulhi(f, upr_magic) : 0;
      col[m] = (int64_t)f - (int64_t)row[m] * upr;
      if (ok[m]) v[m] = load_nt(s_src[row[m]] + col[m]);
      __builtin_amdgcn_s_waitcnt(0);
    }
    // The tile's written units are contiguous in memory (the parts buffer in
    // local order, the global tensor in global order, one owner's slot of the
    // scatter unless the tile straddles two owners): stores through one buffer
    // resource over them, with the nt and sc1 cache policy.
    const bool contiguous = GORDER || !TABLE || wave_uniform(s_rank[0] == s_rank[nrows - 1]);
    if (contiguous) {
      char* const wtile = uniform_ptr(reinterpret_cast<char*>(s_dst[0])) + (u0 - row0 * upr) * 16;
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(wtile, 0, (int)((u_end - u0) * 16), kRawBufferWord3);
#pragma unroll
      for (int m = 0; m < NP; ++m)
        if (ok[m]) __builtin_amdgcn_raw_buffer_store_b128(v[m], rs, (m * kBlock + (int)threadIdx.x) * 16, 0, kStoreNtSc1);
    } else {
#pragma unroll
      for (int m = 0; m < NP; ++m)
        if (ok[m]) store_nt(s_dst[row[m]] + col[m], v[m]);
    }
  }
}

// Row chunks: for metadata whose row map has a closed form (packed-contiguous,
// where rank r holds rows [r n, (r+1) n); dual-chunk-swap with one document,
// where rank r holds global chunks r and 2W-1-r of c = n/2 rows), with rows a
// multiple of 1 KiB.  A workgroup is one wave moving 1 KiB (64 lanes x 16
// bytes) of one written row; the row is blockIdx.x / chunks-per-row, and its
// source and destination follow from the formula in wave-uniform code: no
// table read, no LDS lookup, no barrier.  The shape comes from the host's
// record of the metadata; the 64-byte header is read in flight with the data
// load and checked before the store (a header that fails the check
// stops the workgroup; one whose shape differs from the record, the buffer
// rewritten since, has the row redone from the header's tables).  Measured on
// MI355X against the unit tiles, S=262144, interleaved: the one-document
// gradient scatter of 10 KiB rows 837 -> 809 us, the packed-contiguous
// partition and gather of 5 KiB rows 410 -> 400 and 409 -> 403 us, the
// one-document dual-chunk-swap ones -0.3..-0.7%.  (With the row maps the same
// shape is 5-8% slower than the unit tiles at S=262144, the map read then
// sitting on each workgroup's path before its only data load, and no faster
// at T=32768: 28.1-28.4 against 27.9 us per 67 MB tensor.)
// GORDER: the gather (rows written in global order); else partition or, with
// TABLE, the gradient scatter (rows written in local order, into the owners'
// slots of the pointer table).
template <bool GORDER, bool TABLE>
__global__ void __launch_bounds__(64) permute_chunk_kernel(PermuteArgs a, ChunkDiv dv) {
  cp_meta_header* h = a.meta;
  const int lane = threadIdx.x;
  const uint32_t p = (uint32_t)wave_uniform((int)chunk_row(blockIdx.x, dv));  // written row
  const uint32_t ch = blockIdx.x - p * dv.chunks;
  const int64_t col = (int64_t)ch * 64 + lane;
  const int64_t rb = a.row_bytes;
  char* const gbase = a.global[blockIdx.y];
  char* const lbase = a.local[blockIdx.y];
  // Row p's rank r, local row i and global row g under the recorded shape; all
  // in range for any p < T, since the host records W n = T.
  const int32_t W = a.hint_cp_size;
  const int64_t n = a.hint_local_tokens;
  const bool dcs = a.hint_policy == CP_POLICY_DUAL_CHUNK_SWAP;
  const ChunkRow m = chunk_map<GORDER>(p, W, n, dcs, dv);
  int32_t r = m.r;
  int64_t i = m.i, g = m.g;
  auto source = [&](int32_t r_, int64_t i_, int64_t g_, int64_t n_) {
    return reinterpret_cast<const u32x4*>(GORDER ? lbase + ((int64_t)r_ * n_ + i_) * rb : gbase + g_ * rb) + col;
  };
  auto written = [&](int32_t r_, int64_t i_) {
    return TABLE ? a.table.p[r_] + i_ * rb : (GORDER ? gbase : lbase) + (int64_t)p * rb;
  };
  u32x4 v = load_nt(source(r, i, g, n));
  char* wrow = written(r, i);
  // The written row's address (the scatter's owner pointer), the header (one
  // 64-byte scalar load; the kernel touches no LDS, so nothing else waits on
  // it) and the argument fields the check compares are read while the data
  // load is in flight: left to the compiler, those scalar loads sat between
  // the data's arrival and the store, one wait each.  Measured on MI355X: the
  // scatter 0.3-0.8% faster with the argument reads in flight, and 0.3-0.65%
  // faster again with the header read this way rather than into LDS (the whole
  // check costs about 1%).
  __builtin_amdgcn_sched_barrier(0);
  const cp_meta_header hv = read_header(h);
  __asm__ volatile("" : : "s"(wrow), "s"(a.hint_policy), "s"(a.hint_docs), "s"(a.expect_cp_size),
                   "s"(a.expect_policy), "s"(a.total_tokens), "s"(hv.magic), "s"(hv.flags), "s"(hv.policy),
                   "s"(hv.cp_size), "s"(hv.num_docs), "s"(hv.total_tokens), "s"(hv.local_tokens));
  __builtin_amdgcn_s_waitcnt(0);  // the data load
  if (!meta_ok(h, hv, a.total_tokens, a.expect_cp_size, a.expect_policy)) return;
  if (hv.policy != a.hint_policy || hv.cp_size != W || hv.local_tokens != n || (dcs && hv.num_docs != 1)) {
    // The buffer was rewritten since the host's record: the row from the
    // header's own shape and tables (which the check above has accepted).
    const int32_t Wh = hv.cp_size, Bh = hv.num_docs;
    const int64_t nh = hv.local_tokens;
    const int32_t* cu = meta_cu(h);
    const int32_t* lcu = meta_local_cu0(h, Bh);
    if (GORDER && hv.policy == CP_POLICY_DUAL_CHUNK_SWAP) {
      GCursor gc;
      gseek(gc, p, Bh, cu, lcu);
      glocal(gc, Wh, &r, &i);
    } else {
      r = (int32_t)((int64_t)p / nh);
      i = (int64_t)p - (int64_t)r * nh;
      if (!GORDER) g = owner_global_row(hv.policy, r, i, nh, Wh, Bh, cu, lcu);
    }
    wrow = written(r, i);
    v = load_nt(source(r, i, g, nh));
  }
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(wrow) + (int64_t)ch * 1024, 0, 1024, kRawBufferWord3);
  __builtin_amdgcn_raw_buffer_store_b128(v, rs, lane * 16, 0, kStoreNtSc1);
}

// Whether the row-chunk kernel serves this call (a record of a closed-form
// shape, 16-byte units, rows a multiple of 1 KiB, a grid within HIP's limit
// and the row division exact), and its magic numbers.
bool chunk_fits(const PermuteArgs& a, int64_t upr, ChunkDiv* dv) {
  const int64_t T = a.total_tokens, n = a.hint_local_tokens;
  if (a.hint_cp_size <= 0 || n <= 0 || a.hint_docs < 1 || (int64_t)a.hint_cp_size * n != T) return false;
  if (a.local_table && !a.to_local) return false;
  const bool pc = a.hint_policy == CP_POLICY_PACKED_CONTIGUOUS;
  const bool dcs1 = a.hint_policy == CP_POLICY_DUAL_CHUNK_SWAP && a.hint_docs == 1;
  return (pc || dcs1) && chunk_div(T, n, dcs1, upr, dv);
}

typedef void (*PermuteKernel)(PermuteArgs);

struct Variant {
  PermuteKernel fn[2];  // [0]: local order (partition, scatter); [1]: global order (gather)
  int rows_per_tile;
  const char* name[2];
};

#define CP_VARIANT(U, UNAME, VPL, G, WPR)                                                  \
  Variant{{permute_rows_kernel<U, VPL, G, WPR, false>, permute_rows_kernel<U, VPL, G, WPR, true>}, \
          (kWavesPerBlock / WPR) * G,                                                        \
          {"permute_rows<" UNAME "," #VPL "x" #G "/" #WPR ">",                               \
           "permute_rows<" UNAME "," #VPL "x" #G "/" #WPR ",g>"}}

// Shapes by units per row (upr), from a sweep of tile shapes on MI355X
// (partition, gather and scatter of 2, 5, 8 and 10 KiB rows): a workgroup
// tile of 8-20 KiB with 4-8 loads in flight per lane streamed best; longer
// tiles or more loads per lane lost 5-10%.
#define CP_VARIANTS_FOR(U, UNAME)                                                           \
  {CP_VARIANT(U, UNAME, 1, 4, 1),  /* upr <=   64: 4 rows per wave            */           \
   CP_VARIANT(U, UNAME, 2, 4, 1),  /* upr <=  128: 4 rows per wave            */           \
   CP_VARIANT(U, UNAME, 4, 1, 1),  /* upr <=  256: 1 row per wave             */           \
   CP_VARIANT(U, UNAME, 5, 1, 1),  /* upr <=  320: 1 row per wave, 5 loads    */           \
   CP_VARIANT(U, UNAME, 4, 1, 2),  /* upr <=  512: 2 waves per row            */           \
   CP_VARIANT(U, UNAME, 4, 1, 2),  /* upr <=  640: 2 waves per row, 2 passes  */           \
   CP_VARIANT(U, UNAME, 4, 1, 4)}  /* longer rows: 1 row per tile, 16 KiB passes */
constexpr int64_t kUprLimit[7] = {64, 128, 256, 320, 512, 640, INT64_MAX};

Variant g_variants[4][7] = {
    CP_VARIANTS_FOR(u32x4, "16B"),
    CP_VARIANTS_FOR(u32x2, "8B"),
    CP_VARIANTS_FOR(unsigned int, "4B"),
    CP_VARIANTS_FOR(unsigned short, "2B"),
};

// Flat tiles (see permute_flat_kernel) of kFlatUnits units per thread, for
// metadata the host recorded when it built it: packed-contiguous, and
// dual-chunk-swap with <= kFlatMaxDocs documents or with the row maps.
// Swept on MI355X over 2, 5, 8 and 10 KiB rows with one load in flight per
// lane: 3 units per thread (12 KiB tiles) streamed best under both policies
// (packed-contiguous 1-1.5% ahead of 2 units, dual-chunk-swap 2-4% ahead of
// 4).  0: keep the row tiles.
constexpr int kFlatUnits = 3;

int flat_units_per_thread(const PermuteArgs& a, int64_t upr) {
  if (a.hint_cp_size <= 0 || a.hint_local_tokens <= 0 || a.hint_docs < 1) return 0;  // no record
  if (a.local_table && !a.to_local) return 0;  // owner tables are only written in local order
  const bool flat = a.hint_policy == CP_POLICY_PACKED_CONTIGUOUS ||
                    (a.hint_policy == CP_POLICY_DUAL_CHUNK_SWAP && (a.hint_docs <= kFlatMaxDocs || a.hint_row_maps));
  if (!flat || upr <= 0) return 0;
  const int64_t tile_units = (int64_t)kBlock * kFlatUnits;
  if (tile_units / upr + 2 > kFlatMaxRows) return 0;            // short rows: row tiles
  if ((tile_units + upr) * upr >= (int64_t(1) << 32)) return 0;  // row split would not be exact
  return kFlatUnits;
}

// [kind: local order, global order, owner table][row maps]
const char* const kFlatNames[3][2] = {{"permute_flat<16B,3>", "permute_flat<16B,3,maps>"},
                                      {"permute_flat<16B,3,g>", "permute_flat<16B,3,maps,g>"},
                                      {"permute_flat<16B,3,owners>", "permute_flat<16B,3,maps,owners>"}};
static_assert(kFlatUnits == 3, "kFlatNames spell the unit count");

}  // namespace

hipError_t launch_permute(const PermuteArgs& a, hipStream_t stream) {
  if (a.total_tokens == 0 || a.row_bytes == 0 || a.n_tensors < 1) return hipSuccess;
  if (a.n_tensors > kMaxLayoutTensors || (a.local_table && a.n_tensors != 1)) return hipErrorInvalidValue;
  // Widest unit that divides the row size and every base address.
  uintptr_t align_bits = (uintptr_t)a.row_bytes;
  for (int t = 0; t < a.n_tensors; ++t) align_bits |= (uintptr_t)a.global[t] | (uintptr_t)a.local[t];
  if (a.local_table)
    for (int k = 0; k < kMaxRanks; ++k) align_bits |= (uintptr_t)a.table.p[k];
  int ui;
  int usize;
  if ((align_bits & 15) == 0) { ui = 0; usize = 16; }
  else if ((align_bits & 7) == 0) { ui = 1; usize = 8; }
  else if ((align_bits & 3) == 0) { ui = 2; usize = 4; }
  else if ((align_bits & 1) == 0) { ui = 3; usize = 2; }
  else return hipErrorInvalidValue;  // rows of 2- or 4-byte elements are always even
  const int64_t upr = a.row_bytes / usize;
  int vi = 6;
  for (int k = 0; k < 7; ++k)
    if (upr <= kUprLimit[k]) { vi = k; break; }
  const Variant& v = g_variants[ui][vi];
  // Visit rows in the order of the side being written: a gather writes the
  // global layout, partition and scatter write the per-rank layout.
  const int order = a.to_local ? 0 : 1;
  ChunkDiv dv{};
  const bool chunk = ui == 0 && chunk_fits(a, upr, &dv);
  const int np = ui == 0 && !chunk ? flat_units_per_thread(a, upr) : 0;
  PermuteKernel row_fn = v.fn[order];
  void (*flat_fn)(PermuteArgs, uint32_t) = nullptr;
  const char* name = v.name[order];
  int64_t tiles = (a.total_tokens + v.rows_per_tile - 1) / v.rows_per_tile;
  uint32_t magic = 0;
  if (np != 0) {
    // [kind][row maps]
    static void (*const kFlat[3][2])(PermuteArgs, uint32_t) = {
        {permute_flat_kernel<kFlatUnits, false, false, false>, permute_flat_kernel<kFlatUnits, false, true, false>},
        {permute_flat_kernel<kFlatUnits, true, false, false>, permute_flat_kernel<kFlatUnits, true, true, false>},
        {permute_flat_kernel<kFlatUnits, false, false, true>, permute_flat_kernel<kFlatUnits, false, true, true>}};
    const int kind = a.local_table ? 2 : order;
    // The row maps when the metadata has them, except for the gradient scatter
    // (a per-owner pointer table) with few documents: measured on MI355X the
    // maps speed up the layouts at any document count (one document: -2.7%)
    // and the scatter from 65 documents on, but slow the few-document scatter
    // (one document: +1.8%) against the tables staged in LDS.
    const bool staged_scatter = a.local_table && a.hint_docs <= kFlatMaxDocs;
    const int m = a.hint_row_maps && a.hint_policy == CP_POLICY_DUAL_CHUNK_SWAP && !staged_scatter ? 1 : 0;
    flat_fn = kFlat[kind][m];
    name = kFlatNames[kind][m];
    tiles = (a.total_tokens * upr + (int64_t)kBlock * np - 1) / ((int64_t)kBlock * np);
    magic = (uint32_t)(((uint64_t(1) << 32) + (uint64_t)upr - 1) / (uint64_t)upr);
  }
  void (*chunk_fn)(PermuteArgs, ChunkDiv) = nullptr;
  if (chunk) {
    static void (*const kChunk[3])(PermuteArgs, ChunkDiv) = {
        permute_chunk_kernel<false, false>, permute_chunk_kernel<true, false>, permute_chunk_kernel<false, true>};
    static const char* const kChunkNames[3] = {"permute_chunk<1KiB>", "permute_chunk<1KiB,g>",
                                               "permute_chunk<1KiB,owners>"};
    const int kind = a.local_table ? 2 : order;
    chunk_fn = kChunk[kind];
    name = kChunkNames[kind];
    tiles = a.total_tokens * (int64_t)dv.chunks;  // < 2^26: one chunk per workgroup, no grid-stride
  }
  const int blocks = (int)(tiles < kMaxGrid || chunk ? tiles : kMaxGrid);  // grid-stride beyond kMaxGrid
  auto launch = [&](const PermuteArgs& b) {
    profile_before(name, stream);
    if (chunk_fn) hipLaunchKernelGGL(chunk_fn, dim3(blocks, b.n_tensors), dim3(64), 0, stream, b, dv);
    else if (flat_fn) hipLaunchKernelGGL(flat_fn, dim3(blocks, b.n_tensors), dim3(kBlock), 0, stream, b, magic);
    else hipLaunchKernelGGL(row_fn, dim3(blocks, b.n_tensors), dim3(kBlock), 0, stream, b);
    hipError_t e = hipGetLastError();
    profile_after(stream);
    return e;
  };
  // Several tensors: one launch (a tensor per grid row) when each tensor is
  // small, one launch per tensor when each moves >= 1 GiB.  Measured on
  // MI355X: Q,K,V of 32768 x 8 x 128 bf16 run 19% faster in one launch, of
  // 262144 x 20 x 128 bf16 4% slower.
  const bool per_tensor = a.n_tensors > 1 && 2 * a.total_tokens * a.row_bytes >= (int64_t(1) << 30);
  if (per_tensor) {
    for (int t = 0; t < a.n_tensors; ++t) {
      PermuteArgs b = a;
      b.n_tensors = 1;
      b.global[0] = a.global[t];
      b.local[0] = a.local[t];
      const hipError_t e = launch(b);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  return launch(a);
}

}  // namespace cpthd
