// Workspace of jfa_bwd_noalloc: a scratch area in the library's own device
// memory, so that the call allocates nothing. Each GPU holds its own copy of
// the array (made when the code object is loaded there) until the process
// ends. In host code `scratch` is only a host-side stand-in for the device
// array: kernels get the address that hipGetSymbolAddress gives on the
// current device, looked up once per device and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

static __device__ __align__(256) char scratch[JFA_NOALLOC_SCRATCH_BYTES];

namespace jfa {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

int32_t noalloc_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int32_t)e;
    if (dev < 0 || dev >= kMaxDevices) return (int32_t)hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return (int32_t)e;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return (int32_t)hipSuccess;
}

}  // namespace jfa
