// Library-owned split-K workspace for dgp_gemm_preshuffle_splitk_noalloc
// (include/dgp.h): callers that cannot allocate device memory (code under
// graph capture, serving loops that forbid allocation) get the fp32 partials
// of pass 1 in this fixed array instead of a workspace of their own.
//
// The array is a file-scope device variable: every GPU the library runs on
// holds its own copy, from the first use on that device until the process
// ends.  Its name in host code is only a host-side handle, never a device
// address: the device address is taken once per device with
// hipGetSymbolAddress, with that device current, and kept per device.
//
// Nothing here needs clearing: pass 1 writes every partial it later reads
// (ws[s][m][n] for s < split_k, m < M, n < N) before the reduce reads it.
// All calls on one GPU share the array, so calls that overlap on one GPU
// (different streams, or host threads) race on it.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "launch.h"

namespace dgp {

static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

hipError_t noalloc_scratch(float **out)
{
    static std::atomic<float *> ptr[kMaxDevices];
    static std::mutex init;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    float *p = ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> g(init);
        p = ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            void *addr = nullptr;
            e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
            if (e != hipSuccess)
                return e;
            p = static_cast<float *>(addr);
            ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

}  // namespace dgp
