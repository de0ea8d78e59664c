/* Host-validation fuzz of the C ABI: every entry point called many times with
 * seeded random scalar arguments (edge values of every integer type included)
 * and fake or NULL pointers.  Every call must return a known status code and
 * neither crash nor hit undefined behaviour; the test that runs this program
 * builds the library's host layer with AddressSanitizer and UBSan.  No call
 * here can reach a kernel: no pointer below is device memory. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "cpthd.h"

static uint64_t state = 0x9E3779B97F4A7C15ull;

static uint64_t next(void) {
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return state;
}

static int64_t pick64(void) {
  static const int64_t edge[] = {0, 1, -1, 2, 3, 4, 7, 8, 48, 64, 65, 1000, INT32_MAX, INT32_MIN,
                                 (int64_t)INT32_MAX + 1, INT64_MAX, INT64_MIN, (int64_t)1 << 40,
                                 ((int64_t)1 << 31) - 8, -((int64_t)1 << 62)};
  const uint64_t r = next();
  if (r % 3 == 0) return (int64_t)(next() >> (r % 63));
  return edge[(r >> 8) % (sizeof(edge) / sizeof(edge[0]))];
}

static int32_t pick32(void) {
  static const int32_t edge[] = {0, 1, -1, 2, 3, 4, 5, 8, 16, 63, 64, 65, 128, INT32_MAX, INT32_MIN};
  const uint64_t r = next();
  if (r % 4 == 0) return (int32_t)(next() >> 33);
  return edge[(r >> 8) % (sizeof(edge) / sizeof(edge[0]))];
}

static int32_t pick_small(int32_t lo, int32_t hi) { return lo + (int32_t)(next() % (uint64_t)(hi - lo + 1)); }

#define TABLE (8 * 64 * 64)
static void* table[TABLE];
static const void* ctable[TABLE];

static void* fake(void) {
  static void* const choices[] = {NULL, (void*)(uintptr_t)0x10000, (void*)(uintptr_t)0x20000,
                                  (void*)(uintptr_t)0x10008};
  return choices[next() % 4];
}

static int known(int st) { return st >= CP_OK && st <= CP_ERR_TOO_LARGE; }

int main(int argc, char** argv) {
  int bad = 0;
  const long iters = argc > 2 ? atol(argv[2]) : 20000;
  if (argc > 1) state ^= (uint64_t)strtoull(argv[1], NULL, 10) * 0xD1B54A32D192ED03ull;
  for (long i = 0; i < iters && bad < 10; ++i) {
    for (int k = 0; k < 64; ++k) {
      table[next() % TABLE] = fake();
      ctable[next() % TABLE] = fake();
    }
    int st[16];
    int n = 0;
    char names[128 * 4];
    int64_t counts[4];
    double ms[4];
    int32_t flags = 0;
    uint64_t timeouts = 0;
    (void)cp_meta_bytes(pick32(), pick32());
    (void)cp_meta_bytes_row_maps(pick32(), pick32(), pick64());
    (void)cp_attn_meta_bytes(pick32(), pick32());
    (void)cp_allreduce_signal_bytes(pick32());
    (void)cp_status_string(pick32());
    st[n++] = cp_build_meta((const int32_t*)fake(), pick32(), pick64(), pick32(), pick32(), fake(),
                            (size_t)pick64(), NULL);
    st[n++] = cp_meta_status(fake(), NULL, &flags, &timeouts);
    st[n++] = cp_build_attn_meta(fake(), pick32(), pick32(), fake(), (size_t)pick64(), NULL);
    st[n++] = cp_partition_thd(fake(), fake(), pick64(), pick32(), pick32(), pick32(), fake(), NULL);
    st[n++] = cp_gather_thd(fake(), fake(), pick64(), pick32(), pick32(), pick32(), fake(), NULL);
    st[n++] = cp_partition_thd_multi(pick_small(-2, 9), ctable, table, pick64(), pick32(), pick32(),
                                     pick32(), fake(), NULL);
    st[n++] = cp_gather_thd_multi(pick_small(-2, 9), ctable, table, pick64(), pick32(), pick32(), pick32(),
                                  fake(), NULL);
    st[n++] = cp_grad_return(pick32(), pick32(), pick_small(-1, 8), ctable, table, table, pick64(), pick32(),
                             pick32(), pick32(), pick32(), fake(), (uint32_t*)fake(), (uint32_t)next(),
                             pick64(), pick32(), NULL);
    st[n++] = cp_grad_return_fused(pick32(), pick32(), pick_small(-1, 8), ctable, table, pick64(), pick32(),
                                   pick32(), pick32(), pick32(), fake(), pick32(), NULL);
    st[n++] = cp_grad_return_noalloc(pick32(), pick_small(-1, 8), ctable, table, pick64(), pick32(), pick32(),
                                     pick32(), pick32(), fake(), pick32(), NULL);
    st[n++] = cp_slot_sum(pick32(), ctable, fake(), pick64(), pick32(), pick32(), pick32(), NULL);
    st[n++] = cp_allreduce(pick32(), pick32(), ctable, table, pick64(), pick32(), NULL);
    st[n++] = cp_allreduce_signal(pick32(), ctable, table, pick64(), pick32(), fake(), (size_t)pick64(),
                                  (uint64_t)pick64(), pick64(), NULL);
    st[n++] = cp_allreduce_signal_status(fake(), pick32(), (uint64_t)pick64(), NULL);
    {
      char sel[160];
      const int len = pick_small(0, 159);
      for (int j = 0; j < len; ++j) sel[j] = (char)('a' + (next() % 26));
      sel[len] = '\0';
      const int use = (int)(next() & 1);
      const int want = use && len > 127 ? CP_ERR_ARG : CP_OK;
      const int got = cp_profile_select(use ? sel : NULL);
      if (got != want) {
        printf("iteration %ld: cp_profile_select returned %d\n", i, got);
        ++bad;
      }
      (void)cp_profile_select(NULL);
    }
    const int cap = pick_small(-2, 4);
    const int k = cp_profile_read(names, counts, ms, cap);
    if (k > 4 || k < -CP_ERR_META) {
      printf("iteration %ld: cp_profile_read returned %d\n", i, k);
      ++bad;
    }
    for (int j = 0; j < n; ++j)
      if (!known(st[j])) {
        printf("iteration %ld, call %d: unknown status %d\n", i, j, st[j]);
        ++bad;
      }
  }
  if (bad == 0) printf("fuzz ok: %ld iterations\n", iters);
  return bad == 0 ? 0 : 1;
}
