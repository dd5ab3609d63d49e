// gelu.h -- GELU, x * Phi(x) with Phi the standard normal CDF, and its
// derivative Phi(x) + x * phi(x), written with the device library's erff and
// expf.  Shared by the elementwise kernels and the pointwise convolution's
// fused epilogues, so both give the same values.
#pragma once

#include <hip/hip_runtime.h>

namespace sscnn {

__device__ __forceinline__ float gelu(float v)
{
    return 0.5f * v * (1.f + erff(v * 0.70710678118654752f));
}

__device__ __forceinline__ float gelu_grad(float v)
{
    const float cdf = 0.5f * (1.f + erff(v * 0.70710678118654752f));
    const float pdf = 0.39894228040143268f * expf(-0.5f * v * v);
    return __builtin_fmaf(v, pdf, cdf);
}

}  // namespace sscnn
