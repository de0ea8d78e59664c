// Host-side check of the row-chunk kernel's index arithmetic (chunk_map.h)
// over whole grids: every workgroup's written row and chunk against plain
// division, every row's rank, local row and global row against the ownership
// formula written with plain division, all of them in range, and the local
// order a permutation of the global rows (each global row written once).  Also
// the magic-number division against plain division at edge and random
// arguments.  Built host-only by tests/test_c_abi.py; no GPU is touched.
#include <stdint.h>
#include <stdio.h>

#include <vector>

#include "chunk_map.h"

static int failures = 0;

#define EXPECT(cond, ...)                  \
  do {                                     \
    if (!(cond)) {                         \
      if (failures < 20) {                 \
        printf("FAIL " __VA_ARGS__);       \
        printf("\n");                      \
      }                                    \
      ++failures;                          \
    }                                      \
  } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64() {  // splitmix64
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static void check_div(uint32_t x, uint64_t d) {
  const uint32_t got = cpthd::div_by_magic(x, cpthd::magic_of(d));
  EXPECT(got == x / d, "div_by_magic x=%u d=%llu got %u", x, (unsigned long long)d, got);
}

// One closed-form shape: T rows, W ranks, upr units per row.
static void check_shape(int64_t T, int32_t W, bool dcs, int64_t upr, bool full) {
  const int64_t n = T / W;
  cpthd::ChunkDiv dv;
  if (!cpthd::chunk_div(T, n, dcs, upr, &dv)) {
    printf("FAIL shape T=%lld W=%d upr=%lld not accepted\n", (long long)T, W, (long long)upr);
    ++failures;
    return;
  }
  const int64_t chunks = upr / 64, c = n / 2;
  // every workgroup (or a stride through the grid and its last rows)
  const int64_t blocks = T * chunks;
  const int64_t step = full ? 1 : 7919;
  for (int64_t b = 0; b < blocks; b += (b + step < blocks - 4 * chunks ? step : 1)) {
    const uint32_t p = cpthd::chunk_row((uint32_t)b, dv);
    EXPECT(p == b / chunks && (int64_t)(b - (int64_t)p * chunks) == b % chunks, "chunk_row b=%lld chunks=%lld got %u",
           (long long)b, (long long)chunks, p);
  }
  std::vector<uint8_t> seen(full ? (size_t)T : 0, 0);
  const int64_t rstep = full ? 1 : 101;
  for (int64_t p = 0; p < T; p += (p + rstep < T - 8 ? rstep : 1)) {
    // local order: p = r n + i
    const cpthd::ChunkRow lo = cpthd::chunk_map<false>((uint32_t)p, W, n, dcs, dv);
    const int64_t r = p / n, i = p % n;
    const int64_t g = !dcs ? p : (i < c ? r * c + i : (2 * W - 1 - r) * c + (i - c));
    EXPECT(lo.r == r && lo.i == i && lo.g == g, "local T=%lld W=%d dcs=%d p=%lld got (%d,%lld,%lld) want (%lld,%lld,%lld)",
           (long long)T, W, dcs, (long long)p, lo.r, (long long)lo.i, (long long)lo.g, (long long)r, (long long)i,
           (long long)g);
    EXPECT(lo.r >= 0 && lo.r < W && lo.i >= 0 && lo.i < n && lo.g >= 0 && lo.g < T, "local range p=%lld", (long long)p);
    if (full && lo.g >= 0 && lo.g < T) {
      EXPECT(!seen[lo.g], "global row %lld written twice", (long long)lo.g);
      seen[lo.g] = 1;
    }
    // global order: p is a global row; its rank and local row invert the local map
    const cpthd::ChunkRow go = cpthd::chunk_map<true>((uint32_t)p, W, n, dcs, dv);
    int64_t gr = p / n, gi = p % n;
    if (dcs) {
      const int64_t k = p / c, j = p % c;
      gr = k < W ? k : 2 * W - 1 - k;
      gi = k < W ? j : c + j;
    }
    EXPECT(go.r == gr && go.i == gi && go.g == p, "global T=%lld W=%d dcs=%d p=%lld got (%d,%lld) want (%lld,%lld)",
           (long long)T, W, dcs, (long long)p, go.r, (long long)go.i, (long long)gr, (long long)gi);
    EXPECT(go.r >= 0 && go.r < W && go.i >= 0 && go.i < n, "global range p=%lld", (long long)p);
    if (go.r >= 0 && go.r < W && go.i >= 0 && go.i < n) {
      const cpthd::ChunkRow back = cpthd::chunk_map<false>((uint32_t)(go.r * n + go.i), W, n, dcs, dv);
      EXPECT(back.g == p, "global row %lld does not round-trip (got %lld)", (long long)p, (long long)back.g);
    }
  }
  if (full)
    for (int64_t g = 0; g < T; ++g) EXPECT(seen[g], "global row %lld never written", (long long)g);
}

int main() {
  // magic division: edge divisors and dividends, then random pairs
  const uint64_t ds[] = {1, 2, 3, 5, 7, 10, 63, 64, 65, 513, 1026, 65536, 65537, 1000003, (1u << 31) - 1,
                         1u << 31, (1ull << 32) - 1};
  const uint32_t xs[] = {0, 1, 2, 62, 63, 64, 1025, 65535, 65536, 0x7FFFFFFFu, 0x80000000u, 0xFFFFFFFEu, 0xFFFFFFFFu};
  for (uint64_t d : ds)
    for (uint32_t x : xs) {
      check_div(x, d);
      const uint32_t m = x - (uint32_t)(x % d);  // the multiple of d at or below x, and the value below it
      check_div(m, d);
      if (m > 0) check_div(m - 1, d);
    }
  for (int k = 0; k < 2000000; ++k) {
    const uint64_t d = 1 + (next_u64() >> (32 + (k % 32)));
    check_div((uint32_t)next_u64(), d);
    const uint32_t q = (uint32_t)(next_u64() % (0xFFFFFFFFull / d + 1));
    check_div((uint32_t)(q * d), d);  // exact multiples and the value just below
    if (q * d > 0) check_div((uint32_t)(q * d - 1), d);
  }
  // shapes of the tests and benchmarks, every workgroup and row
  const struct { int64_t T; int32_t W; int64_t upr; } shapes[] = {
      {4104, 4, 64}, {4104, 4, 128}, {6000, 3, 320}, {6000, 3, 640}, {4096, 8, 64}, {1000, 1, 128},
      {8, 4, 64},    {4, 4, 64},     {16, 8, 64},    {2048, 2, 128}, {8192, 4, 64}, {262144, 4, 640},
      {262144, 4, 320}, {131072, 8, 512}, {32768, 4, 128}, {65536, 4, 128}};
  for (const auto& s : shapes)
    for (int dcs = 0; dcs < 2; ++dcs)
      if (!dcs || s.T % (2 * s.W) == 0) check_shape(s.T, s.W, dcs != 0, s.upr, true);
  check_shape(999, 1, false, 64, true);
  // the largest grids the row chunks take: T chunks near 2^26 (one chunk per row)
  // and T chunks^2 just under 2^32 (63 chunks per row), strided
  check_shape((int64_t(1) << 26) - 4, 2, true, 64, false);
  check_shape(1065216, 8, true, 63 * 64, false);
  check_shape(1065216, 3, false, 63 * 64, false);
  check_shape(4000, 4, false, 1000 * 64, false);
  // shapes the row chunks refuse
  cpthd::ChunkDiv dv;
  EXPECT(!cpthd::chunk_div(4096, 1024, false, 96, &dv), "rows of 1.5 KiB accepted");
  EXPECT(!cpthd::chunk_div(4100, 1025, true, 64, &dv), "odd n under dual-chunk-swap accepted");
  EXPECT(!cpthd::chunk_div(int64_t(1) << 26, int64_t(1) << 25, true, 64, &dv), "grid of 2^26 accepted");
  EXPECT(!cpthd::chunk_div(5000, 1250, false, 1000 * 64, &dv), "inexact row division accepted");
  if (failures) {
    printf("%d failures\n", failures);
    return 1;
  }
  printf("chunk_map ok\n");
  return 0;
}
