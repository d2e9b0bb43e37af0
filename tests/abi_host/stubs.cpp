// Stand-ins for the device launchers, for a host-only build of the C ABI
// (argument checking, workspace bookkeeping, status mapping) under the
// address and undefined-behaviour sanitizers: every launcher reports a failed
// launch without enqueuing anything.
#include "fa_internal.h"
#include "fa_scratch.h"

namespace fa {
hipError_t launch_bs_plan(const uint8_t*, long long, int, int, bool, uint32_t*, int*, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_fwd(const FwdArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_merge(const float*, const float*, int, void*, float*, int, int, int, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_transpose_v(const void*, void*, int, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_bwd(const BwdArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_quant_v_pow2(const void*, uint8_t*, uint8_t*, int, int, int, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_quant_fp8(const void*, uint8_t*, float*, int, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t scratch_address(void** out) {
    *out = nullptr;
    return hipErrorNoDevice;
}
}  // namespace fa
