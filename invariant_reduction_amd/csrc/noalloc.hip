// Device-side scratch of det_splitk_gemm_noalloc: the split-K partials and
// arrival counters of a product for callers that cannot allocate (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// allocation).  One file-scope array per device, held until the process
// ends; its device address is looked up once per device and kept, since
// the array's name in host code is only a host-side stand-in for it.
#include <hip/hip_runtime.h>
#include <stddef.h>

#include <mutex>

#include "kernels.h"

namespace detred {

namespace {

// [0, kNoallocCounterBytes): arrival counters of the last-arriver combine,
// zero at rest (every call that uses them leaves them at zero);
// [kNoallocCounterBytes, kNoallocScratchBytes): the slice partials.
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
std::mutex g_mutex;

}  // namespace

hipError_t noalloc_scratch(hipStream_t s, void** ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch[dev]) {
        // first call on this device, with it current: its own copy of the
        // array, at its own address
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        // the counters start at zero: a fill kernel on the caller's stream
        // (no memset node, should the caller be capturing a graph)
        e = launch_fill_zero(static_cast<float*>(p), 0, 1,
                             (int)(kNoallocCounterBytes / sizeof(float)), s);
        if (e != hipSuccess)
            return e;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    return hipSuccess;
}

}  // namespace detred
