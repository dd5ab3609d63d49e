// mfma_conv.h -- dense stride-1 convolution on the FP32 matrix cores.
#pragma once

#include "internal.h"

namespace sscnn {

// groups == 1, stride 1, k in {3, 5}, pad k/2, c_in and c_out multiples of 4
// (at least 16), w_local % 4 == 0.
bool mfma_conv_supported(const Geom& g);
hipError_t launch_mfma_fwd(const Geom& g, const float* x, const float* xh, const float* w,
                           const float* b, float* y, hipStream_t st);
hipError_t launch_mfma_bwd_input(const Geom& g, const float* gy, const float* gyh, const float* w,
                                 float* gx, hipStream_t st);

// mfma_wgrad.hip: split-K grad_weight / grad_bias partials (same layers).
size_t mfma_wgrad_workspace_bytes(const Geom& g);
hipError_t launch_mfma_bwd_weight(const Geom& g, const float* x, const float* xh, const float* gy,
                                  float* gw, float* gb, void* ws, hipStream_t st);

}  // namespace sscnn
