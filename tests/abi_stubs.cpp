// Stand-ins for the library's launch functions, for building the host layer
// (abi.cpp) alone with sanitizers in tests/test_c_abi.py.  Every function
// reports an error, so no call through this build reaches a kernel; the host
// validation in abi.cpp runs unchanged.
#include "cpthd_internal.h"

namespace cpthd {

hipError_t launch_build_meta(const int32_t*, int32_t, int64_t, int32_t, int32_t, bool, void*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_build_attn_meta(cp_meta_header*, int32_t, int32_t, void*, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_permute(const PermuteArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_slot_sum(const SlotSumArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_fused(const FusedArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_allreduce_one_shot(const AllreduceArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_allreduce_two_shot(const AllreduceArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_ring_reduce_step(const AllreduceArgs&, int32_t, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_ring_gather_step(const AllreduceArgs&, int32_t, bool, hipStream_t) { return hipErrorNotSupported; }
int ring_signal_tiles(const AllreduceArgs&, int64_t*) { return 0; }
hipError_t launch_ring_signal(const AllreduceArgs&, const RingSignalArgs&, int, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t noalloc_scratch(void** p) {
  *p = nullptr;
  return hipErrorNotSupported;
}
hipError_t launch_epoch_publish(uint32_t*, int32_t, int32_t, uint32_t, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_epoch_wait(const uint32_t*, int32_t, int32_t, uint32_t, int64_t, cp_meta_header*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace cpthd
