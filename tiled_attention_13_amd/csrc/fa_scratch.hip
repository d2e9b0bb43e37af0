// The static device buffer behind fa_fwd_splitkv_noalloc (see include/fa.h):
// the split-KV kernels' partial O and lse for callers that cannot allocate.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "fa.h"
#include "fa_scratch.h"

// One copy per GPU the library runs on, held from the library's load on that
// device until the process ends.  In host code this name is only a stand-in
// for the device object: kernels get the address hipGetSymbolAddress returns.
static __device__ __align__(256) uint8_t scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace fa {
namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_mutex;
void* g_addr[kMaxScratchDevices];     // device address per device, guarded by g_mutex
}  // namespace

hipError_t scratch_address(void** out) {
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_addr[dev] == nullptr) {
        // first use on this device, which is current: look the address up once
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_addr[dev] = p;
    }
    *out = g_addr[dev];
    return hipSuccess;
}
}  // namespace fa
