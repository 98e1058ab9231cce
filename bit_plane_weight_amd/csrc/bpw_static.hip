// bpw_static.hip - the library's one fixed device scratch array, for callers that cannot allocate
// device memory (code under graph capture, serving loops, harnesses that forbid hipMalloc).
//
// `scratch` is a file-scope device array: every GPU the library runs on holds its own copy, at its
// own address, from the first use until the process ends. In host code the name `scratch` is only a
// host-side stand-in for the symbol, not a device address, so host code never passes it to a kernel
// or a copy: static_scratch() looks the device address up once per device (with that device
// current) and every later use goes through the address it returns.
#include <hip/hip_runtime.h>

#include <mutex>

#include "bpw_internal.h"

namespace bpw {

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

int static_scratch(void **ptr, size_t *len) {
    static std::mutex mu;
    static void *addr[kStaticMaxDevices] = {};
    *ptr = nullptr;
    *len = 0;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kStaticMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    *len = kStaticScratchBytes;
    return hipSuccess;
}

}  // namespace bpw
