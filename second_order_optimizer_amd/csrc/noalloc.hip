// The device-resident scratch of the root pass that allocates nothing
// (shampoo_compute_inverse_roots_noalloc): the batched coupled-Newton
// iterates live in this file-scope array instead of the caller's state
// buffer.  Every GPU the library runs on holds its own copy, at its own
// address, until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.hpp"

namespace shampoo {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};
}  // namespace

// The device address of this device's copy of `scratch`.  In host code the
// array's name only stands in for the symbol, so its address is asked of the
// runtime, once per device with that device current, and kept.
hipError_t noalloc_scratch_ptr(void** out) {
    *out = nullptr;
    int dev = -1;
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
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace shampoo
