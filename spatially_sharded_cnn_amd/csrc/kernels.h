// kernels.h -- per-operation dispatch to the kernel family that fits a layer.
// Arguments are already validated by the ABI layer.
#pragma once

#include "internal.h"

namespace sscnn {

hipError_t kernels_conv_fwd(const Geom& g, const float* x, const float* xh, const float* w,
                            const float* b, float* y, hipStream_t st);
hipError_t kernels_conv_bwd_input(const Geom& g, const float* gy, const float* gyh,
                                  const float* w, float* gx, hipStream_t st);
size_t kernels_bwd_weight_workspace_bytes(const Geom& g);
hipError_t kernels_conv_bwd_weight(const Geom& g, const float* x, const float* xh,
                                   const float* gy, float* gw, float* gb, void* ws,
                                   hipStream_t st);
hipError_t kernels_conv_bwd(const Geom& g, const float* x, const float* xh, const float* gy,
                            const float* gyh, const float* w, float* gx, float* gw, float* gb,
                            void* ws, hipStream_t st);

}  // namespace sscnn
