// edge.h -- the edge half of a split convolution (edge.hip): the terms that
// read a halo column, added to the output of an interior call (the same
// layer computed with its halos read as zeros).  Any layer shape; a no-op
// when the halo in question has zero width.
#pragma once

#include "internal.h"

namespace sscnn {

// y += the forward's input-halo terms (y holds the interior forward).
hipError_t launch_edge_fwd(const Geom& g, const float* xh, const float* w, float* y, hipStream_t st);
// gx += grad_input's grad_output-halo terms (gx holds the interior grad_input).
hipError_t launch_edge_bwd_input(const Geom& g, const float* gyh, const float* w, float* gx,
                                 hipStream_t st);
// gw += grad_weight's input-halo terms over the shard's own output columns.
hipError_t launch_edge_bwd_weight(const Geom& g, const float* xh, const float* gy, float* gw,
                                  hipStream_t st);

}  // namespace sscnn
