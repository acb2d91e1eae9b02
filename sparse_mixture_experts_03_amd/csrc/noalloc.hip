// noalloc.hip -- the static device scratch behind moe_forward_noalloc.
//
// moe_forward_noalloc serves callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): instead of a caller workspace it carves moe_forward's
// workspace out of one file-scope device array of MOE_NOALLOC_SCRATCH_BYTES.
// The code object gives every device that loads it its own copy of the
// array, at its own device address; that copy lives until the process ends.
//
// In host code the array's name is only a host-side stand-in, not a device
// address, so it is never handed to a kernel or a copy: the device address
// is looked up once per device with hipGetSymbolAddress (with that device
// current) and kept; every later use goes through the kept pointer.
#include <mutex>

#include "moe.h"
#include "moe_internal.h"

namespace moe {

namespace {

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

}  // namespace

hipError_t noalloc_scratch(void **ptr) {
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

}  // namespace moe
