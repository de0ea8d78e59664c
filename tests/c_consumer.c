/* A plain C11 consumer of the library's C ABI: includes only cpthd.h and links
 * libcpthd.so, with no HIP header and no Python.  It exercises the calls that
 * need no GPU (sizes, strings, version) and the host-side validation that
 * rejects a call before any device work. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "cpthd.h"

static int failures = 0;

static void expect(int cond, const char* what) {
  if (!cond) {
    printf("FAILED: %s\n", what);
    ++failures;
  }
}

int main(void) {
  void* fake = (void*)(uintptr_t)0x10000; /* never dereferenced: every call fails host-side */
  const void* table[8] = {fake, fake, fake, fake, fake, fake, fake, fake};
  void* otable[8] = {fake, fake, fake, fake, fake, fake, fake, fake};

  expect(cp_version() >= 100, "version");
  expect(strcmp(cp_status_string(CP_OK), "ok") == 0, "status string of CP_OK");
  expect(strcmp(cp_status_string(12345), "unknown status") == 0, "unknown status string");
  expect(cp_meta_bytes(3, 2) % 256 == 0 && cp_meta_bytes(3, 2) >= 64 + 4 * 4 * 3 + 8, "meta bytes");
  expect(cp_meta_bytes(3, 0) == 0, "meta bytes for W = 0");
  expect(cp_attn_meta_bytes(3, 2) == 512, "attention table bytes");

  expect(cp_build_meta(NULL, 3, 48, 2, CP_POLICY_DUAL_CHUNK_SWAP, fake, 4096, NULL) == CP_ERR_ARG,
         "build_meta NULL cu_seqlens");
  expect(cp_build_meta((const int32_t*)fake, 3, 50, 4, CP_POLICY_PACKED_CONTIGUOUS, fake, 4096, NULL) ==
             CP_ERR_SHAPE,
         "build_meta packed-contiguous T % W");
  expect(cp_partition_thd(fake, fake, 48, 2, 8, CP_FP8_E4M3, fake, NULL) == CP_ERR_UNSUPPORTED,
         "partition rejects FP8");
  expect(cp_gather_thd_multi(0, table, otable, 48, 2, 8, CP_BF16, fake, NULL) == CP_ERR_ARG,
         "gather_multi with no tensor");
  expect(cp_grad_return(CP_ALL_RANKS, 2, 2, table, otable, otable, 48, 2, 8, CP_F32, CP_F32, fake, NULL,
                        0, 0, CP_SUM_ACCUMULATE, NULL) == CP_ERR_ARG,
         "grad_return with no phase");
  expect(cp_grad_return_fused(CP_ALL_RANKS, 2, 2, table, otable, 48, 2, 8, CP_F16, CP_F16, fake, 0,
                              NULL) == CP_ERR_UNSUPPORTED,
         "fused rejects an unsupported dtype pair");
  expect(cp_slot_sum(4, NULL, NULL, 0, CP_F32, CP_F32, 0, NULL) == CP_OK, "empty slot sum");
  expect(cp_build_attn_meta(fake, 3, 2, fake, 16, NULL) == CP_ERR_SHAPE, "attention buffer too small");
  expect(cp_allreduce(CP_ALLREDUCE_RING, 8, table, otable, 256, CP_F16, NULL) == CP_ERR_UNSUPPORTED,
         "all-reduce rejects fp16");
  expect(cp_allreduce(CP_ALLREDUCE_ONE_SHOT, 8, NULL, NULL, 0, CP_F32, NULL) == CP_OK, "empty all-reduce");

  if (failures == 0) printf("c consumer ok\n");
  return failures == 0 ? 0 : 1;
}
