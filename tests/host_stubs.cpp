// host_stubs.cpp -- stand-ins for the device-side launch functions, so the
// host half of libra.so (argument checks, workspace sizing, the ring
// drivers' bookkeeping) can be built with g++ alone, under AddressSanitizer
// and UndefinedBehaviorSanitizer, and driven by the ABI tests on a machine
// without a GPU.  Every launch reports that no device is present.
#include "ra_internal.h"

namespace ra {

hipError_t launch_pack_v(const void *, void *, int, int64_t, int64_t, int64_t, int64_t, int64_t,
                         int64_t, int64_t, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_block_fwd_packed(const BatchParams &, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_block_fwd(const BatchParams &, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode(const DecodeParams &, int, void *, float *, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t decode_scratch(void **) { return hipErrorNoDevice; }
hipError_t launch_merge(float *, float *, float *, const float *, const float *, const float *,
                        int64_t, int32_t, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_finalize(const float *, const float *, const float *, void *, float *, int,
                           int64_t, int32_t, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_layout_permute(int, int64_t, int32_t, int32_t *, int32_t *, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_copy(void *, const void *, size_t, hipStream_t, int) { return hipErrorNoDevice; }
hipError_t launch_delay(int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_handoff_copy(void *, const void *, size_t, hipStream_t, bool) {
  return hipErrorNoDevice;
}
hipError_t launch_layout_move(bool, const void *, void *, const int32_t *, int32_t, int64_t,
                              int64_t, int64_t, int64_t, int32_t, int32_t, int32_t, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_bwd_prep(const void *, const void *, const float *, float *, float *, int,
                           int64_t, int32_t, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_bwd(const BwdParams &, int, hipStream_t, int) { return hipErrorNoDevice; }
hipError_t launch_zero(float *, int64_t, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_cast(const float *, void *, int, int64_t, hipStream_t) { return hipErrorNoDevice; }

}  // namespace ra
