// stream.hip -- a plain streaming copy, one read and one write of every
// element: the rate it reaches is the practical HBM ceiling that the
// library's bandwidth-bound kernels (the depthwise layers, the halo gathers,
// the reductions) are measured against, next to the 8 TB/s published peak.
//
// One float4 per thread over a grid that covers the whole array in one
// pass: the workgroups run in dispatch order, so the ones resident at any
// moment read and write one contiguous window of memory.  On the MI355X this
// measured 6.2 TB/s for 1 GiB each way, against 4.2-4.6 TB/s for grid-stride
// loops of 4 or 8 float4 per thread (each thread's loads a grid apart) and
// 5.2-5.6 TB/s for workgroup-contiguous chunks of 4-8 KB per trip.
#include "internal.h"

namespace sscnn {
namespace {

__global__ void __launch_bounds__(256)
stream_copy_kernel(const float4* __restrict__ src, float4* __restrict__ dst, int64_t n4)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x)
        dst[i] = src[i];
}

__global__ void __launch_bounds__(64)
stream_copy_tail_kernel(const float* __restrict__ src, float* __restrict__ dst, int64_t from, int64_t count)
{
    const int64_t i = from + threadIdx.x;
    if (i < count) dst[i] = src[i];
}

}  // namespace

hipError_t launch_stream_copy(const float* src, float* dst, int64_t count, hipStream_t st)
{
    const int64_t n4 = count / 4;
    if (n4 > 0) {
        const int64_t want = (n4 + 255) / 256;
        const int64_t cap = (int64_t)1 << 30;              // more than any array here needs
        hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)(want < cap ? want : cap)), dim3(256), 0, st,
                           reinterpret_cast<const float4*>(src), reinterpret_cast<float4*>(dst), n4);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (count > n4 * 4) {
        hipLaunchKernelGGL(stream_copy_tail_kernel, dim3(1), dim3(64), 0, st, src, dst, n4 * 4, count);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace sscnn
