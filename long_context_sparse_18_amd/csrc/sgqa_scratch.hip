// sgqa_scratch.hip -- a fixed device scratch area for entry points that allocate nothing.
//
// Some callers cannot allocate device memory at all (code under stream capture, tight
// serving loops, harnesses that forbid it).  For them the library keeps one file-scope
// device array, `scratch`, of kScratchBytes.  Every GPU the library runs on holds its own
// copy until the process ends.  In host code the array's name is only a host-side stand-in,
// so its device address is looked up once per device with hipGetSymbolAddress, and only
// that address is ever handed to kernels.
//
// Every call on one GPU shares that GPU's array and leaves the last call's contents in it:
// calls that overlap on one GPU (different streams, different host threads) race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "sgqa_launch.hpp"

namespace sgqa {
namespace {

constexpr int kMaxDevices = 64;

}  // namespace
}  // namespace sgqa

static __device__ __align__(256) float scratch[sgqa::kScratchBytes / sizeof(float)];

namespace sgqa {
namespace {

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once looked up

}  // namespace

hipError_t scratch_region(void **ptr, size_t *bytes)
{
    *ptr = nullptr;
    *bytes = 0;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        // the current device is `dev`: the address returned is that device's copy
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    *bytes = kScratchBytes;
    return hipSuccess;
}

}  // namespace sgqa
