// hh_noalloc.hip -- the library-owned scratch buffer of hh_linattn_fwd_noalloc.
//
// The forward's segment slots normally come from a caller workspace.  For callers that cannot
// allocate device memory at all, the same kernels take their slots from a file-scope device
// array instead, of a fixed maximum size, one copy per device (each GPU the library runs on
// holds it until the process ends).  Host code never uses the array's name as a device address:
// the address comes from hipGetSymbolAddress, taken once per device with that device current,
// and is cached per device.
#include <hip/hip_runtime.h>
#include <stddef.h>

#include <mutex>

#include "hh_kernels.h"

namespace hh {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices];  // device address of `scratch` per device, once resolved
}  // namespace

hipError_t noalloc_scratch(void **ptr) {
    *ptr = nullptr;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    return hipSuccess;
}

}  // namespace hh
