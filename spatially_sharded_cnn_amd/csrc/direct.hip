// direct.hip -- one-thread-per-output direct convolution kernels for any
// shape the ABI accepts (any square k, stride, pad, groups).  They serve the
// small layers where launch latency dominates (the 3->8 5x5 case) and every
// layer the specialised kernels do not cover.
//
// Each kernel reads the shard's EXTENDED row -- [left halo | local slice |
// right halo] -- through ext_load(), which picks the region from the column
// index, so the concatenated tensor of the pages (kwkr.cn retelling,
// section 2.2) is never materialised, and only the shard's own output columns
// are computed, so nothing has to be cropped.
//
// Sums run in float32 with fused multiply-add, in a fixed order.
#include "internal.h"

namespace sscnn {
namespace {

// Extended-row load: column e of the row (plane, r) of [halo_l | local | halo_r];
// a null halo reads as zeros (the interior half of a split convolution).
__device__ __forceinline__ float ext_load(const float* __restrict__ loc, const float* __restrict__ halo,
                                          int64_t plane_row, int wl, int hl, int hw, int e)
{
    if (e >= hl && e < hl + wl) return loc[plane_row * wl + (e - hl)];
    if (!halo) return 0.0f;
    return e < hl ? halo[plane_row * hw + e] : halo[plane_row * hw + (e - wl)];
}

// y[b, o, i, j] for j < wol (shard-local):  input column of tap kw is global
// j_g*stride + kw - pad = s*wl + j*stride + kw - pad, i.e. extended column
// j*stride + kw since the extended row starts at global column s*wl - hl and
// hl == pad.
__global__ void __launch_bounds__(256)
direct_fwd_kernel(Geom g, const float* __restrict__ x, const float* __restrict__ xh,
                  const float* __restrict__ w, const float* __restrict__ bias, float* __restrict__ y)
{
    const int64_t total = (int64_t)g.n * g.co * g.ho * g.wol;
    const int hw = g.hl + g.hr;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        int64_t q = t;
        const int j = (int)(q % g.wol); q /= g.wol;
        const int i = (int)(q % g.ho); q /= g.ho;
        const int o = (int)(q % g.co);
        const int b = (int)(q / g.co);
        const int grp = o / g.cog;
        float acc = bias ? bias[o] : 0.0f;
        for (int c = 0; c < g.cig; ++c) {
            const int64_t plane = (int64_t)b * g.ci + grp * g.cig + c;
            const float* wp = w + ((int64_t)o * g.cig + c) * g.k * g.k;
            for (int kh = 0; kh < g.k; ++kh) {
                const int r = i * g.stride + kh - g.pad;
                if (r < 0 || r >= g.h) continue;
                const int64_t pr = plane * g.h + r;
                for (int kw = 0; kw < g.k; ++kw)
                    acc = fmaf(wp[kh * g.k + kw], ext_load(x, xh, pr, g.wl, g.hl, hw, j * g.stride + kw), acc);
            }
        }
        y[t] = acc;
    }
}

// grad_x[b, c, yy, xx] (xx shard-local) = sum over o in c's group, kh, kw with
// yy + pad - kh = i*stride, xx + pad - kw = jl*stride (exact), 0 <= i < ho, of
// w[o, c mod cig, kh, kw] * G[b, o, i, jl], where jl is the shard-local output
// column (jl < 0 or jl >= wol reads the grad_output halo; s*wl is a multiple of
// the stride, so exactness only depends on the local column).
__global__ void __launch_bounds__(256)
direct_bwd_input_kernel(Geom g, const float* __restrict__ gy, const float* __restrict__ gyh,
                        const float* __restrict__ w, float* __restrict__ gx)
{
    const int64_t total = (int64_t)g.n * g.ci * g.h * g.wl;
    const int ghw = g.ghl + g.ghr;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        int64_t q = t;
        const int xx = (int)(q % g.wl); q /= g.wl;
        const int yy = (int)(q % g.h); q /= g.h;
        const int c = (int)(q % g.ci);
        const int b = (int)(q / g.ci);
        const int grp = c / g.cig, cl = c - grp * g.cig;
        float acc = 0.0f;
        for (int oo = 0; oo < g.cog; ++oo) {
            const int o = grp * g.cog + oo;
            const int64_t plane = (int64_t)b * g.co + o;
            const float* wp = w + ((int64_t)o * g.cig + cl) * g.k * g.k;
            for (int kh = 0; kh < g.k; ++kh) {
                const int tr = yy + g.pad - kh;
                if (tr < 0 || tr % g.stride != 0) continue;
                const int i = tr / g.stride;
                if (i >= g.ho) continue;
                const int64_t pr = plane * g.ho + i;
                for (int kw = 0; kw < g.k; ++kw) {
                    const int tc = xx + g.pad - kw;
                    // floor-safe exact division of a possibly negative column offset
                    const int tq = tc + g.stride * (g.ghl + 1);
                    if (tq % g.stride != 0) continue;
                    const int e = tq / g.stride - 1;   // = jl + ghl, extended column
                    if (e < 0 || e >= g.wol + ghw) continue;
                    acc = fmaf(wp[kh * g.k + kw], ext_load(gy, gyh, pr, g.wol, g.ghl, ghw, e), acc);
                }
            }
        }
        gx[t] = acc;
    }
}

// grad_w[o, c, kh, kw] = sum over b, i, j < wol (the shard's own output
// columns) of G[b, o, i, j] * Xext[b, grp*cig + c, i*stride + kh - pad, j*stride + kw].
// One thread per weight element, sequential sum in (b, i, j) order.
__global__ void __launch_bounds__(256)
direct_bwd_weight_kernel(Geom g, const float* __restrict__ x, const float* __restrict__ xh,
                         const float* __restrict__ gy, float* __restrict__ gw)
{
    const int64_t total = (int64_t)g.co * g.cig * g.k * g.k;
    const int hw = g.hl + g.hr;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        int64_t q = t;
        const int kw = (int)(q % g.k); q /= g.k;
        const int kh = (int)(q % g.k); q /= g.k;
        const int c = (int)(q % g.cig);
        const int o = (int)(q / g.cig);
        const int cin = (o / g.cog) * g.cig + c;
        float acc = 0.0f;
        for (int b = 0; b < g.n; ++b) {
            const int64_t xplane = (int64_t)b * g.ci + cin;
            const int64_t gplane = (int64_t)b * g.co + o;
            for (int i = 0; i < g.ho; ++i) {
                const int r = i * g.stride + kh - g.pad;
                if (r < 0 || r >= g.h) continue;
                const float* grow = gy + (gplane * g.ho + i) * g.wol;
                const int64_t pr = xplane * g.h + r;
                for (int j = 0; j < g.wol; ++j)
                    acc = fmaf(grow[j], ext_load(x, xh, pr, g.wl, g.hl, hw, j * g.stride + kw), acc);
            }
        }
        gw[t] = acc;
    }
}

// grad_b[o] = sum over b, i, j < wol of G[b, o, i, j]; one 256-thread block per
// channel: per-thread strided partial sums, then a fixed-shape tree in LDS.
__global__ void __launch_bounds__(256)
direct_bwd_bias_kernel(Geom g, const float* __restrict__ gy, float* __restrict__ gb)
{
    __shared__ float red[256];
    const int o = blockIdx.x;
    const int64_t per_img = (int64_t)g.ho * g.wol;
    float acc = 0.0f;
    for (int b = 0; b < g.n; ++b) {
        const float* p = gy + ((int64_t)b * g.co + o) * per_img;
        for (int64_t e = threadIdx.x; e < per_img; e += blockDim.x) acc += p[e];
    }
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0) gb[o] = red[0];
}

int grid_for(int64_t work)
{
    int64_t blocks = (work + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 1 << 20) blocks = 1 << 20;
    return (int)blocks;
}

}  // namespace

hipError_t launch_direct_fwd(const Geom& g, const float* x, const float* xh, const float* w,
                             const float* b, float* y, hipStream_t st)
{
    const int64_t total = (int64_t)g.n * g.co * g.ho * g.wol;
    hipLaunchKernelGGL(direct_fwd_kernel, dim3(grid_for(total)), dim3(256), 0, st, g, x, xh, w, b, y);
    return hipGetLastError();
}

hipError_t launch_direct_bwd_input(const Geom& g, const float* gy, const float* gyh,
                                   const float* w, float* gx, hipStream_t st)
{
    const int64_t total = (int64_t)g.n * g.ci * g.h * g.wl;
    hipLaunchKernelGGL(direct_bwd_input_kernel, dim3(grid_for(total)), dim3(256), 0, st, g, gy, gyh,
                       w, gx);
    return hipGetLastError();
}

hipError_t launch_direct_bwd_weight(const Geom& g, const float* x, const float* xh,
                                    const float* gy, float* gw, float* gb, hipStream_t st)
{
    const int64_t total = (int64_t)g.co * g.cig * g.k * g.k;
    hipLaunchKernelGGL(direct_bwd_weight_kernel, dim3(grid_for(total)), dim3(256), 0, st, g, x, xh,
                       gy, gw);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || gb == nullptr) return e;
    hipLaunchKernelGGL(direct_bwd_bias_kernel, dim3(g.co), dim3(256), 0, st, g, gy, gb);
    return hipGetLastError();
}

}  // namespace sscnn
