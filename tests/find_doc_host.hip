// Host-side check of the document search used by the permutation and metadata
// kernels (device_common.h find_doc) at document counts near 2^31, with the
// cu_seqlens table computed on the fly instead of stored (8 GiB otherwise).
// Built host-only by tests/test_c_abi.py; no GPU is touched.
#include <stdint.h>
#include <stdio.h>

#include "device_common.h"

// cu[k] = max(0, k - empties): `empties` empty documents, then documents of
// one token each; total tokens = B - empties.
struct Ramp {
  int64_t empties;
  int32_t operator[](int64_t k) const { return (int32_t)(k > empties ? k - empties : 0); }
};

static int failures = 0;

static void expect(int32_t got, int64_t want, const char* what, int64_t v) {
  if (got != want) {
    printf("FAIL %s: v=%lld got %d want %lld\n", what, (long long)v, got, (long long)want);
    ++failures;
  }
}

int main() {
  const int32_t sizes[] = {1, 2, 3, 1000, (1 << 30) + 1, INT32_MAX - 2, INT32_MAX - 1, INT32_MAX};
  for (int32_t B : sizes) {
    // one-token documents: position v lies in document v
    const Ramp ones{0};
    const int64_t vs[] = {0, 1, B / 2, (int64_t)B - 2, (int64_t)B - 1};
    for (int64_t v : vs)
      if (v >= 0 && v < B) expect(cpthd::find_doc(ones, B, v), v, "one-token documents", v);
    // all but the last 1000 documents empty: the search must skip every empty one
    if (B > 1000) {
      const Ramp tail{(int64_t)B - 1000};
      const int64_t ws[] = {0, 1, 500, 999};
      for (int64_t v : ws) expect(cpthd::find_doc(tail, B, v), (int64_t)B - 1000 + v, "empty prefix", v);
    }
  }
  if (failures) return 1;
  printf("find_doc ok\n");
  return 0;
}
