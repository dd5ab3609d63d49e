// mfma_conv.h -- dense stride-1 convolution on the FP32 matrix cores.
#pragma once

#include "internal.h"

namespace sscnn {

// Rows beyond a slice's top and bottom, for a slice split along H (and W):
// up holds the rh rows above row 0 and down the rh rows below row H-1 of
// every plane, rplane floats from one plane to the next (the row-halo layout
// (planes, rh + rh, W): up rows then down rows).  Rows beyond those, and all
// rows outside [0, H) when up / down are null, read as zeros.  crh: the
// column halo, if any, covers rows -crh .. H + crh - 1 (0: rows 0 .. H-1).
struct RowHalo {
    const float* up = nullptr;
    const float* down = nullptr;
    int64_t rplane = 0;
    int rh = 0;
    int crh = 0;
};

// groups == 1, stride 1, k in {3, 5}, pad k/2, c_in and c_out multiples of 4
// (at least 16), w_local % 4 == 0.
bool mfma_conv_supported(const Geom& g);
hipError_t launch_mfma_fwd(const Geom& g, const float* x, const float* xh, const float* w,
                           const float* b, float* y, hipStream_t st);
hipError_t launch_mfma_bwd_input(const Geom& g, const float* gy, const float* gyh, const float* w,
                                 float* gx, hipStream_t st);
// The same with row halos (height and 2-D sharding): rows are read through rows.
hipError_t launch_mfma_fwd_rows(const Geom& g, const float* x, const float* xh, const RowHalo& rows,
                                const float* w, const float* b, float* y, hipStream_t st);
hipError_t launch_mfma_bwd_input_rows(const Geom& g, const float* gy, const float* gyh, const RowHalo& rows,
                                      const float* w, float* gx, hipStream_t st);

// mfma_wgrad.hip: split-K grad_weight / grad_bias partials (same layers).
size_t mfma_wgrad_workspace_bytes(const Geom& g);
hipError_t launch_mfma_bwd_weight(const Geom& g, const float* x, const float* xh, const float* gy,
                                  float* gw, float* gb, void* ws, hipStream_t st);
hipError_t launch_mfma_bwd_weight_rows(const Geom& g, const float* x, const float* xh, const RowHalo& rows,
                                       const float* gy, float* gw, float* gb, void* ws, hipStream_t st);

}  // namespace sscnn
