// kvarn_scratch.hip -- the library's static device scratch buffer, for the
// entry point that allocates nothing (callers that cannot allocate device
// memory: code under graph capture, tight serving loops).
//
// `scratch` is a file-scope device array: the runtime gives every GPU the
// library runs on its own copy when the code object is loaded there, and it
// lives until the process ends.  In host code the array's name is only a
// host-side stand-in, never a device address: the device address is taken
// once per device with hipGetSymbolAddress (that device current) and kept
// here; host code passes only that pointer to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kvarn_internal.hpp"

namespace kvarn {

namespace {

__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> guard(g_lock);
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

}  // namespace kvarn
