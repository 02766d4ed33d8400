// kda_noalloc.hip -- the library's own device scratch for kda_chunk_fwd_noalloc.
//
// Callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation) run the chunked
// forward with its workspace in this file-scope device array instead of a
// caller-provided one.  Each GPU that loads the library holds its own copy of
// the array until the process ends.  In host code the array's name is only a
// host-side stand-in: its device address is looked up per device with
// hipGetSymbolAddress, once, and only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kda_launch.hpp"

namespace kda {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_workspace(void** ptr) {
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
    *ptr = g_ptr[dev];
    return hipSuccess;
}

}  // namespace kda
