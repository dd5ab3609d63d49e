// blockops.h -- launchers of the ConvNeXt block's non-convolution steps
// (blockops.hip).  Arguments are validated by the callers in api.cpp.
#pragma once

#include "internal.h"

namespace sscnn {

hipError_t launch_layernorm_fwd(int n, int c, int64_t hw, float eps, const float* x, const float* gamma,
                                const float* beta, float* y, float* mean, float* rstd, hipStream_t st);
// dx, dgamma, dbeta each nullable (skipped)
hipError_t launch_layernorm_bwd(int n, int c, int64_t hw, const float* x, const float* dy, const float* gamma,
                                const float* mean, const float* rstd, float* dx, float* dgamma, float* dbeta,
                                hipStream_t st);
hipError_t launch_gelu_fwd(int64_t count, const float* x, float* y, hipStream_t st);
hipError_t launch_gelu_bwd(int64_t count, const float* x, const float* dy, float* dx, hipStream_t st);
// thr = floor(keep * 2^32) capped at 2^32 - 1, inv_keep = 1 / keep; draw false gives all ones
hipError_t launch_droppath_scales(int n, uint64_t seed, uint64_t offset, uint32_t thr, float inv_keep, bool draw,
                                  float* scales, hipStream_t st);
// hw % 4 == 0; scales nullable (ones)
hipError_t launch_scale_residual_fwd(int n, int c, int64_t hw, const float* x, const float* h, const float* gamma,
                                     const float* scales, float* out, hipStream_t st);
// dh, dgamma each nullable (skipped)
hipError_t launch_scale_residual_bwd(int n, int c, int64_t hw, const float* h, const float* dout, const float* gamma,
                                     const float* scales, float* dh, float* dgamma, hipStream_t st);

}  // namespace sscnn
