// halo.hip -- the single-GPU halo exchange and the fixed-order reductions.
//
// Halo exchange (NVIDIA blog "Perception Model Training for Autonomous
// Vehicles with Tensor Parallelism", Figure 1 and Figure 2 text; kwkr.cn
// retelling, section 2.2): a shard receives the last hl columns of its left
// neighbour's slice and the first hr columns of its right neighbour's slice,
// zeros where there is no neighbour.  Here the neighbours' slices are buffers
// in the same HBM, so the "receive" is a gather into a compact
// (planes, rows, hl + hr) buffer that the convolution kernels read as the two
// side regions of the extended row.
//
// Partial reduction (blog, DTensor section: _Partial gradients reduced to
// Replicate): a fixed left-to-right float32 sum, so results are reproducible.
#include "internal.h"

namespace sscnn {
namespace {

// One thread per halo element; consecutive threads write consecutive halo
// floats (fully coalesced writes).  For the common widths hl + hr is a
// template constant (HW), so the row / column split is a multiply-shift;
// HW == 0 takes the width at run time.  Reads touch hl (or hr) contiguous
// floats per row of the neighbour.
template <int HW>
__global__ void __launch_bounds__(256)
halo_gather_kernel(const float* __restrict__ left, const float* __restrict__ right,
                   int64_t total_rows, int width, int hl, int hw_rt, float* __restrict__ halo)
{
    const int hw = HW ? HW : hw_rt;
    const int64_t total = total_rows * hw;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = t / hw;
        const int e = (int)(t - row * hw);
        float v = 0.0f;
        if (e < hl) {
            if (left) v = left[row * width + (width - hl + e)];
        } else {
            if (right) v = right[row * width + (e - hl)];
        }
        halo[t] = v;
    }
}

// The same gather with one thread per (row, side) for halos of at most 4
// columns a side on rows of a multiple of 4 floats (16-byte aligned slices):
// the side's columns sit in one aligned 16-byte piece of the neighbour's row
// (its last 4 floats, or its first 4), read with one load instead of one per
// column.  Each row piece still costs the 128-byte line it sits in.
template <int HL, int HR>
__global__ void __launch_bounds__(256)
halo_gather_vec_kernel(const float* __restrict__ left, const float* __restrict__ right, int64_t total_rows,
                       int width, float* __restrict__ halo)
{
    constexpr int HW = HL + HR;
    const int64_t total = total_rows * 2;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = t >> 1;
        const int side = (int)(t & 1);
        float* h = halo + row * HW;
        if (side == 0) {
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (left) v = *reinterpret_cast<const float4*>(left + row * width + width - 4);
            const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < HL; ++i) h[i] = e[4 - HL + i];
        } else {
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (right) v = *reinterpret_cast<const float4*>(right + row * width);
            const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < HR; ++i) h[HL + i] = e[i];
        }
    }
}

// Push form of the exchange for layers whose kernels do not push from their
// epilogue: after the layer wrote its slice t, one thread per (row, halo
// column) copies the slice's last hl columns into the right neighbour's halo
// (its columns [0, hl)) and its first hr columns into the left neighbour's
// (columns [hl, hl + hr)), and zeros the own halo's sides without a
// neighbour.  Reads hit one 128-byte line per few-byte row piece, like the
// gather it replaces.
__global__ void __launch_bounds__(256)
push_edges_kernel(const float* __restrict__ t, int64_t total_rows, int width, int hl, int hr,
                  float* __restrict__ to_left, float* __restrict__ to_right, float* __restrict__ own)
{
    const int hw = hl + hr;
    const int64_t total = total_rows * hw;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = i / hw;
        const int e = (int)(i - row * hw);
        if (e < hl) {                    // the slice's column width - hl + e
            if (to_right) to_right[row * hw + e] = t[row * width + (width - hl + e)];
            if (!to_left) own[row * hw + e] = 0.f;
        } else {                         // the slice's column e - hl
            if (to_left) to_left[row * hw + e] = t[row * width + (e - hl)];
            if (!to_right) own[row * hw + e] = 0.f;
        }
    }
}

struct PartPtrs {
    const float* p[kMaxParts];
};

// Each thread owns 4 consecutive outputs (float4 when the whole range is
// 16-byte aligned, which the host checks) and adds the parts in order.
template <bool kVec4>
__global__ void __launch_bounds__(256)
partial_reduce_kernel(PartPtrs parts, int nparts, int64_t count, float* __restrict__ out)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x * 4;
    for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < count; i += stride) {
        if (kVec4 && i + 4 <= count) {
            float4 acc = *reinterpret_cast<const float4*>(parts.p[0] + i);
            for (int s = 1; s < nparts; ++s) {
                const float4 v = *reinterpret_cast<const float4*>(parts.p[s] + i);
                acc.x += v.x;
                acc.y += v.y;
                acc.z += v.z;
                acc.w += v.w;
            }
            *reinterpret_cast<float4*>(out + i) = acc;
        } else {
            for (int64_t j = i; j < i + 4 && j < count; ++j) {
                float acc = parts.p[0][j];
                for (int s = 1; s < nparts; ++s) acc += parts.p[s][j];
                out[j] = acc;
            }
        }
    }
}

__global__ void __launch_bounds__(256)
split_reduce_kernel(const float* __restrict__ ws, int nsplit, int64_t count, float* __restrict__ out)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (int64_t)gridDim.x * blockDim.x) {
        float acc = ws[i];
        for (int s = 1; s < nsplit; ++s) acc += ws[(int64_t)s * count + i];
        out[i] = acc;
    }
}

int grid_for(int64_t work, int per_block)
{
    int64_t blocks = (work + per_block - 1) / per_block;
    if (blocks < 1) blocks = 1;
    if (blocks > 65536) blocks = 65536;   // grid-stride loops cover the rest
    return (int)blocks;
}

}  // namespace

hipError_t launch_halo_gather(const float* left, const float* right, int64_t planes, int rows,
                              int width, int hl, int hr, float* halo, hipStream_t st)
{
    const int64_t total_rows = planes * rows;
    if (total_rows == 0 || hl + hr == 0) return hipSuccess;
    const int hw = hl + hr;
    const bool vec = width % 4 == 0 && width >= 4 && (reinterpret_cast<uintptr_t>(left) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(right) & 15) == 0;
    if (vec && hl == hr && (hl == 2 || hl == 3)) {
        const int grid2 = grid_for(total_rows * 2, 256);
        if (hl == 3)
            hipLaunchKernelGGL((halo_gather_vec_kernel<3, 3>), dim3(grid2), dim3(256), 0, st, left, right, total_rows,
                               width, halo);
        else
            hipLaunchKernelGGL((halo_gather_vec_kernel<2, 2>), dim3(grid2), dim3(256), 0, st, left, right, total_rows,
                               width, halo);
        return hipGetLastError();
    }
    const int grid = grid_for(total_rows * hw, 256);
    switch (hw) {
#define SSCNN_HALO_CASE(HW)                                                                  \
    case HW:                                                                                 \
        hipLaunchKernelGGL(halo_gather_kernel<HW>, dim3(grid), dim3(256), 0, st, left, right, \
                           total_rows, width, hl, hw, halo);                                 \
        break;
        SSCNN_HALO_CASE(2) SSCNN_HALO_CASE(4) SSCNN_HALO_CASE(6)
#undef SSCNN_HALO_CASE
        default:
            hipLaunchKernelGGL(halo_gather_kernel<0>, dim3(grid), dim3(256), 0, st, left, right,
                               total_rows, width, hl, hw, halo);
    }
    return hipGetLastError();
}

hipError_t launch_push_edges(const float* t, int64_t planes, int rows, int width, int hl, int hr, float* to_left,
                             float* to_right, float* own, hipStream_t st)
{
    const int64_t total_rows = planes * rows;
    if (total_rows == 0 || hl + hr == 0) return hipSuccess;
    hipLaunchKernelGGL(push_edges_kernel, dim3(grid_for(total_rows * (hl + hr), 256)), dim3(256), 0, st, t,
                       total_rows, width, hl, hr, to_left, to_right, own);
    return hipGetLastError();
}

hipError_t launch_partial_reduce(const float* const* parts, int nparts, int64_t count, float* out,
                                 hipStream_t st)
{
    PartPtrs pp{};
    bool vec = (reinterpret_cast<uintptr_t>(out) & 15) == 0;
    for (int s = 0; s < nparts; ++s) {
        pp.p[s] = parts[s];
        vec = vec && (reinterpret_cast<uintptr_t>(parts[s]) & 15) == 0;
    }
    if (count == 0) return hipSuccess;
    const int grid = grid_for((count + 3) / 4, 256);
    if (vec)
        hipLaunchKernelGGL(partial_reduce_kernel<true>, dim3(grid), dim3(256), 0, st, pp, nparts,
                           count, out);
    else
        hipLaunchKernelGGL(partial_reduce_kernel<false>, dim3(grid), dim3(256), 0, st, pp, nparts,
                           count, out);
    return hipGetLastError();
}

hipError_t launch_split_reduce(const float* ws, int nsplit, int64_t count, float* out,
                               hipStream_t st)
{
    if (count == 0) return hipSuccess;
    hipLaunchKernelGGL(split_reduce_kernel, dim3(grid_for(count, 256)), dim3(256), 0, st, ws,
                       nsplit, count, out);
    return hipGetLastError();
}

}  // namespace sscnn
