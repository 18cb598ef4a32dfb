// noalloc.hip -- the device memory behind the allocation-free backward
// (maxsim_bwd_noalloc): a file-scope device array that stands in for the
// caller's workspace, for callers that cannot allocate.
//
// In host code `scratch` names a host-side stand-in, not a device address:
// its device address is read once per device with hipGetSymbolAddress (with
// that device current) and every launch takes that address.  Each GPU holds
// its own copy of the array for the life of the process.  Every call on a
// device shares that device's copy, so calls that overlap on one device
// race; the kernels write every word they later read, so no clearing is
// needed between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace maxsim {
namespace {

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_addr[dev] = p;
    }
    *out = g_addr[dev];
    return hipSuccess;
}

}  // namespace maxsim
