// dn_noalloc.hip -- the scratch memory of dn_chunk_fwd_noalloc: a device array of
// the library (one copy per GPU, held until the process ends) in place of the
// caller's workspace, for callers that cannot allocate.
//
// Host code never passes `scratch` itself to a kernel or a copy: in host code the
// name is a host-side stand-in, not a device address.  The device address comes
// from hipGetSymbolAddress, taken once per device with that device current, and
// is kept per device.
#include <hip/hip_runtime.h>

#include <mutex>

#include "dn.h"
#include "dn_internal.h"

namespace dn {

namespace {

static __device__ __align__(256) unsigned char scratch[DN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

// Device address of the current device's scratch array (looked up on the first
// call on each device).  hipSuccess or the runtime's error; *ptr untouched on error.
hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    *bytes = DN_NOALLOC_SCRATCH_BYTES;
    return hipSuccess;
}

}  // namespace dn
