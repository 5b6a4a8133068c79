// The library-owned scratch array behind the allocation-free entry point
// (gdn_chunk_prefill_noalloc in gdn_api.hip). It stands in for the caller-provided
// workspace of gdn_chunk_prefill: one array per GPU, held from the first call on that GPU
// until the process ends. Nothing in it has to start at zero (every workspace byte the
// prefill kernels read was written earlier in the same call), and calls that overlap in time
// on one GPU share it and race.
//
// In host code `scratch` names a host-side stand-in, not the device array: its device address
// comes from hipGetSymbolAddress, once per device with that device current, and only that
// address is ever handed to a kernel.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/gdn.h"
#include "gdn_launch.h"

namespace {

static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

namespace gdn {

hipError_t noalloc_scratch(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    return hipSuccess;
}

}  // namespace gdn
