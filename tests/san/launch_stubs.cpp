// Test-only stand-ins for libsscan's kernel launchers, linked with a host-sanitized build
// of sscan_api.cpp so that its argument validation can run under AddressSanitizer and
// UndefinedBehaviorSanitizer without the GPU kernels.  Every stand-in fails, so a call
// that passed validation by mistake shows up as SSCAN_ERR_HIP in the test.
#include "sscan_internal.h"

namespace sscan {

hipError_t launch_fwd(int, int, int, bool, bool, const FwdParams&, unsigned, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_bc_pack(int, int, const FwdParams&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_fwd_sg(int, int, int, bool, bool, const FwdParams&, unsigned, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_bwd(int, int, int, bool, bool, const BwdParams&, unsigned, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_bwd_hf(int, int, int, bool, const BwdParams&, unsigned, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_reduce(const ReduceParams&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_decode(int, int, const DecodeParams&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_fill(float*, int64_t, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_copy_or_zero(float*, const float*, int64_t, hipStream_t) { return hipErrorNotSupported; }

}  // namespace sscan
