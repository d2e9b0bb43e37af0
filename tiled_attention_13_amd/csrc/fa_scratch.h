// Interface of the static scratch buffer behind fa_fwd_splitkv_noalloc.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

// Device address of the static scratch buffer (FA_NOALLOC_SCRATCH_BYTES bytes)
// on the current device; looked up once per device and kept.
hipError_t scratch_address(void** out);

}  // namespace fa
