// rowedge.h -- height sharding (rowedge.hip): the row halo exchange and the
// kernels that add the row halos' terms to an interior result (the slice
// convolved as its own image).  g describes the local slice: g.h input rows,
// g.ho output rows, full width; hu / hd are the halo rows above / below.
#pragma once

#include "internal.h"

namespace sscnn {

// halo[p, e, :]: the last hu rows of up[p], then the first hd rows of down[p]
// (rows of `width` floats; zeros for a null neighbour).
hipError_t launch_row_halo_gather(const float* up, const float* down, int64_t planes, int rows, int width, int hu,
                                  int hd, float* halo, hipStream_t st);
// 2-D shards, second phase: out[p, e, :] = the last hl columns of the left
// neighbour's extended row e, then the first hr columns of the right
// neighbour's (extended rows: up rows of its row halo, its rows, down rows of
// its row halo; (planes, up + rows + down, hl + hr); zeros for a null
// neighbour or row halo).
hipError_t launch_grid_col_halo(const float* left, const float* left_rh, const float* right, const float* right_rh,
                                int64_t planes, int rows, int width, int up, int down, int hl, int hr, float* out,
                                hipStream_t st);
// y += the forward's terms that read an input halo row (rh: (n, ci, hu + hd, wl)).
hipError_t launch_row_edge_fwd(const Geom& g, int hu, int hd, const float* rh, const float* w, float* y,
                               hipStream_t st);
// gx += grad_input's terms that read a grad_output halo row (grh: (n, co, ghu + ghd, wol)).
hipError_t launch_row_edge_bwd_input(const Geom& g, int ghu, int ghd, const float* grh, const float* w, float* gx,
                                     hipStream_t st);
// Scratch the row-edge grad_weight needs (depthwise layers: one partial per
// channel, image and halo tap); it may share the interior call's workspace,
// which is free by then.
size_t row_edge_workspace_bytes(const Geom& g);
// gw += grad_weight's terms over the shard's own output rows that read an input halo row.
hipError_t launch_row_edge_bwd_weight(const Geom& g, int hu, int hd, const float* rh, const float* gy, float* gw,
                                      void* ws, hipStream_t st);

}  // namespace sscnn
