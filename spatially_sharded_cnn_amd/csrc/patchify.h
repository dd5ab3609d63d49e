// patchify.h -- convolutions whose kernel equals their stride (stem, downsamples)
// on the FP32 matrix cores.
#pragma once

#include "internal.h"

namespace sscnn {

// Push form of the halo exchange (see sscnn_push_t): besides its own slice,
// a forward (or grad_input) writes its first hr and last hl output columns
// into the next layer's halo buffers of the neighbouring shards, and zeros
// the part of its own halo that has no neighbour.
struct Push {
    float* to_left = nullptr;
    float* to_right = nullptr;
    float* own = nullptr;
    int hl = 0, hr = 0;
};

// groups == 1, k == stride in {2, 4}, pad 0, c_in*k*k and c_out multiples of 16,
// output width a multiple of 16.
bool patch_supported(const Geom& g);
size_t patch_wgrad_workspace_bytes(const Geom& g);
// act (pointwise layers only): also write GELU(y) there.
hipError_t launch_patch_fwd(const Geom& g, const float* x, const float* w, const float* b, float* y,
                            hipStream_t st, float* act = nullptr, const Push* push = nullptr);
// pre (pointwise layers only): write dX * GELU'(pre) instead of dX.
hipError_t launch_patch_bwd_input(const Geom& g, const float* gy, const float* w, float* gx, hipStream_t st,
                                  const float* pre = nullptr, const Push* push = nullptr);
hipError_t launch_patch_bwd_weight(const Geom& g, const float* x, const float* gy, float* gw, float* gb,
                                   void* ws, hipStream_t st);

}  // namespace sscnn
