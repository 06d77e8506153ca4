// Library-owned split-K scratch for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc). The FP32 partial planes of gemm_bf16_splitk_noalloc live
// in a file-scope device array; each device the library runs on holds its own
// copy until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: the
// device address is taken once per device with hipGetSymbolAddress (with that
// device current) and only that address is ever handed to kernels.
#include <atomic>
#include <mutex>

#include "bg_internal.hpp"

namespace bg {
namespace {

static __device__ __align__(256) float scratch[kNoallocScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || p == nullptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace bg
