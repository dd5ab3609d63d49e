// dispatch.cpp -- choose the kernel family for a layer.
//
//   depthwise  groups == channels, stride 1, k in {3,5,7}, pad k/2, w_local % 16 == 0
//   patchify   groups == 1, k == stride in {2,4}, pad 0 (stem, downsamples): a
//              matrix product after a reshape, on the FP32 matrix cores
//   mfma       groups == 1, stride 1, k in {3,5}, pad k/2, channels multiples of 4
//              (forward, grad_input and grad_weight on the FP32 matrix cores)
//   direct     any other layer (one thread per output element)
#include "kernels.h"

#include "depthwise.h"
#include "mfma_conv.h"
#include "patchify.h"

namespace sscnn {

hipError_t kernels_conv_fwd(const Geom& g, const float* x, const float* xh, const float* w,
                            const float* b, float* y, hipStream_t st)
{
    if (dw_supported(g)) return launch_dw_fwd(g, x, xh, w, b, y, st);
    if (patch_supported(g)) return launch_patch_fwd(g, x, w, b, y, st);
    if (mfma_conv_supported(g)) return launch_mfma_fwd(g, x, xh, w, b, y, st);
    return launch_direct_fwd(g, x, xh, w, b, y, st);
}

hipError_t kernels_conv_bwd_input(const Geom& g, const float* gy, const float* gyh,
                                  const float* w, float* gx, hipStream_t st)
{
    if (dw_supported(g)) return launch_dw_bwd_input(g, gy, gyh, w, gx, st);
    if (patch_supported(g)) return launch_patch_bwd_input(g, gy, w, gx, st);
    if (mfma_conv_supported(g)) return launch_mfma_bwd_input(g, gy, gyh, w, gx, st);
    return launch_direct_bwd_input(g, gy, gyh, w, gx, st);
}

size_t kernels_bwd_weight_workspace_bytes(const Geom& g)
{
    if (dw_supported(g)) return dw_wgrad_workspace_bytes(g);
    if (patch_supported(g)) return patch_wgrad_workspace_bytes(g);
    if (mfma_conv_supported(g)) return mfma_wgrad_workspace_bytes(g);
    return 0;
}

hipError_t kernels_conv_bwd_weight(const Geom& g, const float* x, const float* xh,
                                   const float* gy, float* gw, float* gb, void* ws,
                                   hipStream_t st)
{
    if (dw_supported(g)) return launch_dw_bwd_weight(g, x, xh, gy, gw, gb, ws, st);
    if (patch_supported(g)) return launch_patch_bwd_weight(g, x, gy, gw, gb, ws, st);
    if (mfma_conv_supported(g)) return launch_mfma_bwd_weight(g, x, xh, gy, gw, gb, ws, st);
    return launch_direct_bwd_weight(g, x, xh, gy, gw, gb, st);
}

hipError_t kernels_conv_bwd(const Geom& g, const float* x, const float* xh, const float* gy,
                            const float* gyh, const float* w, float* gx, float* gw, float* gb,
                            void* ws, hipStream_t st)
{
    if (dw_supported(g)) return launch_dw_bwd(g, x, xh, gy, gyh, w, gx, gw, gb, ws, st);
    const hipError_t e = kernels_conv_bwd_input(g, gy, gyh, w, gx, st);
    if (e != hipSuccess) return e;
    return kernels_conv_bwd_weight(g, x, xh, gy, gw, gb, ws, st);
}

}  // namespace sscnn
