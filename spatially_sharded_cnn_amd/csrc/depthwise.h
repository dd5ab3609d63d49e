// depthwise.h -- the depthwise (groups == channels) stride-1 kernel family.
#pragma once

#include "internal.h"

namespace sscnn {

// k in {3, 5, 7}, pad k/2, stride 1, groups == c_in == c_out, w_local % 16 == 0.
bool dw_supported(const Geom& g);
size_t dw_wgrad_workspace_bytes(const Geom& g);
hipError_t launch_dw_fwd(const Geom& g, const float* x, const float* xh, const float* w,
                         const float* b, float* y, hipStream_t st);
hipError_t launch_dw_bwd_input(const Geom& g, const float* gy, const float* gyh, const float* w,
                               float* gx, hipStream_t st);
hipError_t launch_dw_bwd_weight(const Geom& g, const float* x, const float* xh, const float* gy,
                                float* gw, float* gb, void* ws, hipStream_t st);
// grad_input and the grad_weight / grad_bias partials in one pass over grad_output
// (workspace as for launch_dw_bwd_weight).
hipError_t launch_dw_bwd(const Geom& g, const float* x, const float* xh, const float* gy, const float* gyh,
                         const float* w, float* gx, float* gw, float* gb, void* ws, hipStream_t st);

}  // namespace sscnn
