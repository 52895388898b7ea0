// Device scratch of the allocation-free entry points: a fixed array in the library's code
// object. Each GPU the library runs on holds its own copy, from the first launch on that GPU
// until the process ends; its device address is looked up once per device and kept.
//
// Every call on one GPU shares that GPU's copy and leaves its contents behind, so calls that
// overlap in time on one GPU (two streams, two host threads) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdr_kernels.hpp"

namespace {

static __device__ __align__(256) char scratch[gdr::kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch_ptr[kMaxDevices];

}  // namespace

namespace gdr {

// The current device's scratch address. In host code `scratch` names a host-side stand-in,
// never the device memory, so only the address returned here is handed to kernels.
hipError_t scratch_region(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace gdr
