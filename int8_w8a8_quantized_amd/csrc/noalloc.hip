// Device scratch of the allocation-free fused Linear (for callers that
// cannot allocate: HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  The activation codes and scales that the fused Linear
// keeps in a caller workspace live here instead, in a file-scope device
// array: each GPU the library runs on holds its own copy until the process
// ends, found once per device with hipGetSymbolAddress.  In host code the
// array's name only stands for the symbol; kernels get the device address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "tfq_internal.h"

namespace tfq {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** out)
{
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        // with device `dev` current: the address of its copy of the array
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace tfq
