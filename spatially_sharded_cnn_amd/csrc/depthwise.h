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

// Height sharding: the same kernels with the rows beyond the slice's top and
// bottom read from row halos (N*C, up + down, W), up rows first (the layout
// of sscnn_row_halo_gather); no column halo.  Same workspace as above.
hipError_t launch_dw_fwd_rows(const Geom& g, const float* x, const float* x_rh, int up, int down,
                              const float* w, const float* b, float* y, hipStream_t st);
hipError_t launch_dw_bwd_input_rows(const Geom& g, const float* gy, const float* gy_rh, int up, int down,
                                    const float* w, float* gx, hipStream_t st);
hipError_t launch_dw_bwd_weight_rows(const Geom& g, const float* x, const float* x_rh, int up, int down,
                                     const float* gy, float* gw, float* gb, void* ws, hipStream_t st);
hipError_t launch_dw_bwd_rows(const Geom& g, const float* x, const float* x_rh, int x_up, int x_down,
                              const float* gy, const float* gy_rh, int g_up, int g_down, const float* w, float* gx,
                              float* gw, float* gb, void* ws, hipStream_t st);

// 2-D shards: rows beyond the block from the row halo (N*C, up + down, W),
// columns beside it from the column halo over the extended rows
// (N*C, up + H + down, 2P), corners included.  Same workspace as above.
hipError_t launch_dw_fwd_grid(const Geom& g, const float* x, const float* x_rh, const float* x_ch, int up, int down,
                              const float* w, const float* b, float* y, hipStream_t st);
hipError_t launch_dw_bwd_input_grid(const Geom& g, const float* gy, const float* gy_rh, const float* gy_ch, int up,
                                    int down, const float* w, float* gx, hipStream_t st);
hipError_t launch_dw_bwd_weight_grid(const Geom& g, const float* x, const float* x_rh, const float* x_ch, int up,
                                     int down, const float* gy, float* gw, float* gb, void* ws, hipStream_t st);
hipError_t launch_dw_bwd_grid(const Geom& g, const float* x, const float* x_rh, const float* x_ch, int x_up,
                              int x_down, const float* gy, const float* gy_rh, const float* gy_ch, int g_up,
                              int g_down, const float* w, float* gx, float* gw, float* gb, void* ws, hipStream_t st);

}  // namespace sscnn
