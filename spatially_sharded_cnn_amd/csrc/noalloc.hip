// noalloc.hip -- the device scratch behind sscnn_conv_bwd_noalloc, for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// The scratch is a file-scope device array: every GPU the library runs on
// holds its own copy, at its own address, from module load until the process
// ends.  Host code never passes the array's name to a kernel (on the host it
// is only a stand-in for the symbol); it asks the runtime for the array's
// device address once per device, with that device current, and hands that
// address to the kernels as their workspace.
#include <mutex>

#include "internal.h"

namespace sscnn {
namespace {

static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];    // device address of `scratch` on each device, once looked up

}  // namespace

hipError_t noalloc_scratch(void** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace sscnn
