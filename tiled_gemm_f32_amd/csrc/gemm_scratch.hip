// The library's own device scratch memory, for callers that cannot allocate
// (gemm_general_noalloc).
//
// The K-split paths keep their partial products in a workspace (the split-K
// variant of "Tiled matrix multiplication", "Variants and alternatives").
// Normally the caller passes one; gemm_general_noalloc uses this file-scope
// device array instead.  Every GPU the library runs on holds its own copy of
// it, from the first call on that device until the process ends.
//
// In host code the array's name denotes a host-side stand-in, not device
// memory: its device address is looked up once per device, with that device
// current, and only that address is ever handed to a kernel.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "gemm_kernels.hpp"

namespace gemm {
namespace {

static __device__ __align__(256) char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

hipError_t static_scratch(void **out) {
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (err != hipSuccess || p == nullptr) return err != hipSuccess ? err : hipErrorInvalidSymbol;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

}  // namespace gemm
