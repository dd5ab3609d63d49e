// blockops.hip -- the ConvNeXt block's steps other than its convolutions, on
// one shard's NCHW activations: LayerNorm over channels, GELU, layer scale
// with DropPath and the residual add, and the DropPath factors themselves.
// None of them looks across pixels, so a W- (or H-) shard runs them on its
// own slice with no halo; their weight gradients are per-shard partial sums,
// reduced like the convolutions' (kwkr.cn retelling, section 3.1: the
// DropPath layer is distributed with its random state kept consistent).
//
//  * LayerNorm: a workgroup takes 64 consecutive pixels and its waves split
//    the C values of each (so every load is a 256-byte run of one channel
//    row).  Up to C = 1024 (512 in the backward) each thread keeps its
//    values in registers and reads them once; wider maps take them from
//    memory again for each pass.  The backward recomputes x-hat from the
//    saved mean and rstd.  The per-channel
//    weight and bias gradients are a second kernel, one workgroup per
//    channel, reduced in a fixed order (bitwise reproducible).
//  * GELU: elementwise, 4 values per thread, with the device library's erff
//    and expf.
//  * DropPath factors: Philox4x32-10 (Salmon et al., SC'11) of the counter
//    (sample, offset low, offset high, 0) under the key (seed low, seed high),
//    kept when the first word is below a threshold the host computes; every
//    shard gets the same factors because they depend on the sample index
//    only (NVIDIA blog "Perception Model Training for Autonomous Vehicles with
//    Tensor Parallelism": DropPath's Bernoulli draws must agree across GPUs).
#include "internal.h"
#include "blockops.h"
#include "gelu.h"

namespace sscnn {
namespace {

constexpr int kThreads = 256;

// ---- LayerNorm over channels ------------------------------------------------
//
// A workgroup takes 64 consecutive pixels; its 4 waves split the channels
// (wave g takes channels g, g + 4, ...), so every load is one 256-byte run of
// a channel row and there are 4 times as many waves in flight as pixels / 64.
// The per-pixel sums of the 4 waves meet in LDS and are added in wave order.

constexpr int kPix = 64, kGroups = 4;

// sum over the G waves of v for this lane's pixel, in wave order
template <int G = kGroups>
__device__ __forceinline__ float pixel_sum(float v, float (*red)[kPix], int g, int lane)
{
    red[g][lane] = v;
    __syncthreads();
    float r = red[0][lane];
#pragma unroll
    for (int i = 1; i < G; ++i) r += red[i][lane];
    __syncthreads();
    return r;
}

__global__ void __launch_bounds__(kPix * kGroups)
ln_fwd_kernel(const float* __restrict__ x, const float* __restrict__ gamma, const float* __restrict__ beta,
              float* __restrict__ y, float* __restrict__ mean_out, float* __restrict__ rstd_out, int C, int64_t HW,
              int64_t npix, float eps)
{
    __shared__ float red[kGroups][kPix];
    const int lane = threadIdx.x % kPix, g = threadIdx.x / kPix;
    const int64_t t = (int64_t)blockIdx.x * kPix + lane;
    const bool live = t < npix;
    const int64_t tt = live ? t : 0;
    const int64_t n = tt / HW, p = tt - n * HW;
    const float* xp = x + n * C * HW + p;
    float s = 0.f;
    if (live) {
#pragma unroll 8
        for (int c = g; c < C; c += kGroups) s += xp[c * HW];
    }
    const float mean = pixel_sum(s, red, g, lane) / (float)C;
    float v = 0.f;
    if (live) {
#pragma unroll 8
        for (int c = g; c < C; c += kGroups) {
            const float d = xp[c * HW] - mean;
            v = __builtin_fmaf(d, d, v);
        }
    }
    const float rstd = 1.f / sqrtf(pixel_sum(v, red, g, lane) / (float)C + eps);
    if (!live) return;
    float* yp = y + n * C * HW + p;
#pragma unroll 8
    for (int c = g; c < C; c += kGroups) yp[c * HW] = __builtin_fmaf((xp[c * HW] - mean) * rstd, gamma[c], beta[c]);
    if (g == 0) {
        mean_out[t] = mean;
        rstd_out[t] = rstd;
    }
}

// dx = rstd * (dxhat - mean_c(dxhat) - xhat * mean_c(dxhat * xhat)), dxhat = dy * gamma.
// No implicit FMA contraction here: dxhat is then the same rounded product in
// both passes (with one channel dx is exactly 0); the explicit FMAs stay.
__global__ void __launch_bounds__(kPix * kGroups)
ln_bwd_kernel(const float* __restrict__ x, const float* __restrict__ dy, const float* __restrict__ gamma,
              const float* __restrict__ mean_in, const float* __restrict__ rstd_in, float* __restrict__ dx, int C,
              int64_t HW, int64_t npix)
{
#pragma clang fp contract(off)
    __shared__ float red[kGroups][kPix];
    const int lane = threadIdx.x % kPix, g = threadIdx.x / kPix;
    const int64_t t = (int64_t)blockIdx.x * kPix + lane;
    const bool live = t < npix;
    const int64_t tt = live ? t : 0;
    const int64_t n = tt / HW, p = tt - n * HW;
    const int64_t base = n * C * HW + p;
    const float mean = mean_in[tt], rstd = rstd_in[tt];
    float a = 0.f, b = 0.f;
    if (live) {
#pragma unroll 8
        for (int c = g; c < C; c += kGroups) {
            const float gg = dy[base + c * HW] * gamma[c];
            a += gg;
            b = __builtin_fmaf(gg, (x[base + c * HW] - mean) * rstd, b);
        }
    }
    a = pixel_sum(a, red, g, lane) / (float)C;
    b = pixel_sum(b, red, g, lane) / (float)C;
    if (!live) return;
#pragma unroll 8
    for (int c = g; c < C; c += kGroups) {
        const float gg = dy[base + c * HW] * gamma[c];
        const float xh = (x[base + c * HW] - mean) * rstd;
        dx[base + c * HW] = rstd * (gg - a - xh * b);
    }
}

// The same two passes with the pixel's values held in registers, for C up to
// G * V: G waves per 64 pixels, thread (g, lane) keeps channels g, g + G, ...
// (at most V of them), so x -- and dy in the backward -- is read from memory
// once.  The per-thread sums run in channel order and the per-pixel sums in
// wave order, as above: with G = 4 the results equal the loop kernels' bit
// for bit.  Pixels past the end read pixel 0 (in bounds) and store nothing.
template <int G, int V>
__global__ void __launch_bounds__(kPix * G)
ln_fwd_reg_kernel(const float* __restrict__ x, const float* __restrict__ gamma, const float* __restrict__ beta,
                  float* __restrict__ y, float* __restrict__ mean_out, float* __restrict__ rstd_out, int C,
                  int64_t HW, int64_t npix, float eps)
{
    __shared__ float red[G][kPix];
    const int lane = threadIdx.x % kPix;
    const int g = __builtin_amdgcn_readfirstlane(threadIdx.x / kPix);
    const int64_t t = (int64_t)blockIdx.x * kPix + lane;
    const bool live = t < npix;
    const int64_t tt = live ? t : 0;
    const int64_t n = tt / HW, p = tt - n * HW;
    const float* xp = x + n * C * HW + p;
    float v[V];
#pragma unroll
    for (int k = 0; k < V; ++k)
        if (g + k * G < C) v[k] = xp[(int64_t)(g + k * G) * HW];
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < V; ++k)
        if (g + k * G < C) s += v[k];
    const float mean = pixel_sum<G>(s, red, g, lane) / (float)C;
    float q = 0.f;
#pragma unroll
    for (int k = 0; k < V; ++k)
        if (g + k * G < C) {
            const float d = v[k] - mean;
            q = __builtin_fmaf(d, d, q);
        }
    const float rstd = 1.f / sqrtf(pixel_sum<G>(q, red, g, lane) / (float)C + eps);
    if (!live) return;
    float* yp = y + n * C * HW + p;
#pragma unroll
    for (int k = 0; k < V; ++k) {
        const int c = g + k * G;
        if (c < C) yp[(int64_t)c * HW] = __builtin_fmaf((v[k] - mean) * rstd, gamma[c], beta[c]);
    }
    if (g == 0) {
        mean_out[t] = mean;
        rstd_out[t] = rstd;
    }
}

template <int G, int V>
__global__ void __launch_bounds__(kPix * G)
ln_bwd_reg_kernel(const float* __restrict__ x, const float* __restrict__ dy, const float* __restrict__ gamma,
                  const float* __restrict__ mean_in, const float* __restrict__ rstd_in, float* __restrict__ dx,
                  int C, int64_t HW, int64_t npix)
{
#pragma clang fp contract(off)
    __shared__ float red[G][kPix];
    const int lane = threadIdx.x % kPix;
    const int g = __builtin_amdgcn_readfirstlane(threadIdx.x / kPix);
    const int64_t t = (int64_t)blockIdx.x * kPix + lane;
    const bool live = t < npix;
    const int64_t tt = live ? t : 0;
    const int64_t n = tt / HW, p = tt - n * HW;
    const int64_t base = n * C * HW + p;
    const float mean = mean_in[tt], rstd = rstd_in[tt];
    float xv[V], gv[V];
#pragma unroll
    for (int k = 0; k < V; ++k) {
        const int c = g + k * G;
        if (c < C) {
            xv[k] = x[base + (int64_t)c * HW];
            gv[k] = dy[base + (int64_t)c * HW] * gamma[c];
        }
    }
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int k = 0; k < V; ++k)
        if (g + k * G < C) {
            a += gv[k];
            b = __builtin_fmaf(gv[k], (xv[k] - mean) * rstd, b);
        }
    a = pixel_sum<G>(a, red, g, lane) / (float)C;
    b = pixel_sum<G>(b, red, g, lane) / (float)C;
    if (!live) return;
#pragma unroll
    for (int k = 0; k < V; ++k) {
        const int c = g + k * G;
        if (c < C) {
            const float xh = (xv[k] - mean) * rstd;
            dx[base + (int64_t)c * HW] = rstd * (gv[k] - a - xh * b);
        }
    }
}

// Per-channel sums over every pixel: one 1024-thread workgroup per channel,
// 4 loads in flight per thread, reduced in a fixed order (LDS tree).
constexpr int kRedThreads = 1024;

__device__ __forceinline__ float block_sum(float v, float* red)
{
    red[threadIdx.x] = v;
    __syncthreads();
#pragma unroll
    for (int s = kRedThreads / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
        __syncthreads();
    }
    const float r = red[0];
    __syncthreads();
    return r;
}

// dgamma[c] = sum over the pixels of dy * xhat, dbeta[c] = sum of dy.
__global__ void __launch_bounds__(kRedThreads)
ln_params_kernel(const float* __restrict__ x, const float* __restrict__ dy, const float* __restrict__ mean_in,
                 const float* __restrict__ rstd_in, float* __restrict__ dgamma, float* __restrict__ dbeta, int N,
                 int C, int64_t HW)
{
    __shared__ float red[kRedThreads];
    const int c = blockIdx.x;
    float sg = 0.f, sb = 0.f;
    for (int n = 0; n < N; ++n) {
        const int64_t base = ((int64_t)n * C + c) * HW;
#pragma unroll 4
        for (int64_t p = threadIdx.x; p < HW; p += kRedThreads) {
            const float d = dy[base + p];
            sg = __builtin_fmaf(d, (x[base + p] - mean_in[n * HW + p]) * rstd_in[n * HW + p], sg);
            sb += d;
        }
    }
    sg = block_sum(sg, red);
    sb = block_sum(sb, red);
    if (threadIdx.x == 0) {
        if (dgamma) dgamma[c] = sg;
        if (dbeta) dbeta[c] = sb;
    }
}

// ---- GELU ---------------------------------------------------------------------

__global__ void __launch_bounds__(kThreads)
gelu_fwd_kernel(const float* __restrict__ x, float* __restrict__ y, int64_t count)
{
    const int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x;   // group of 4 values
    const int64_t i = q * 4;
    if (i + 4 <= count) {
        const float4 v = *reinterpret_cast<const float4*>(x + i);
        *reinterpret_cast<float4*>(y + i) = make_float4(gelu(v.x), gelu(v.y), gelu(v.z), gelu(v.w));
    } else {
        for (int64_t k = i; k < count; ++k) y[k] = gelu(x[k]);
    }
}

__global__ void __launch_bounds__(kThreads)
gelu_bwd_kernel(const float* __restrict__ x, const float* __restrict__ dy, float* __restrict__ dx, int64_t count)
{
    const int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t i = q * 4;
    if (i + 4 <= count) {
        const float4 v = *reinterpret_cast<const float4*>(x + i);
        const float4 d = *reinterpret_cast<const float4*>(dy + i);
        *reinterpret_cast<float4*>(dx + i) = make_float4(d.x * gelu_grad(v.x), d.y * gelu_grad(v.y),
                                                         d.z * gelu_grad(v.z), d.w * gelu_grad(v.w));
    } else {
        for (int64_t k = i; k < count; ++k) dx[k] = dy[k] * gelu_grad(x[k]);
    }
}

// ---- DropPath factors (Philox4x32-10) -----------------------------------------------

__device__ __forceinline__ uint32_t philox_first_word(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                      uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    }
    return c0;
}

__global__ void __launch_bounds__(kThreads)
droppath_kernel(int n, uint32_t seed_lo, uint32_t seed_hi, uint32_t off_lo, uint32_t off_hi, uint32_t thr,
                float inv_keep, int draw, float* __restrict__ scales)
{
    const int i = blockIdx.x * kThreads + threadIdx.x;
    if (i >= n) return;
    if (!draw) {
        scales[i] = 1.f;
        return;
    }
    const uint32_t w = philox_first_word((uint32_t)i, off_lo, off_hi, 0u, seed_lo, seed_hi);
    scales[i] = w < thr ? inv_keep : 0.f;
}

// ---- layer scale, DropPath and the residual --------------------------------------------

// out = x + s[n] * (gamma[c] * h), 4 values per thread (HW a multiple of 4).
__global__ void __launch_bounds__(kThreads)
scale_residual_fwd_kernel(const float* __restrict__ x, const float* __restrict__ h, const float* __restrict__ gamma,
                          const float* __restrict__ scales, float* __restrict__ out, int C, int64_t HW,
                          int64_t count)
{
    const int64_t i = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 4;
    if (i >= count) return;
    const int64_t nc = i / HW;
    const int c = (int)(nc % C);
    const float s = scales ? scales[nc / C] : 1.f, g = gamma[c];
    const float4 xv = *reinterpret_cast<const float4*>(x + i);
    const float4 hv = *reinterpret_cast<const float4*>(h + i);
    *reinterpret_cast<float4*>(out + i) = make_float4(__builtin_fmaf(s, g * hv.x, xv.x), __builtin_fmaf(s, g * hv.y, xv.y),
                                                      __builtin_fmaf(s, g * hv.z, xv.z), __builtin_fmaf(s, g * hv.w, xv.w));
}

// dh = (s[n] * dout) * gamma[c]
__global__ void __launch_bounds__(kThreads)
scale_residual_bwd_kernel(const float* __restrict__ dout, const float* __restrict__ gamma,
                          const float* __restrict__ scales, float* __restrict__ dh, int C, int64_t HW, int64_t count)
{
    const int64_t i = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 4;
    if (i >= count) return;
    const int64_t nc = i / HW;
    const int c = (int)(nc % C);
    const float s = scales ? scales[nc / C] : 1.f, g = gamma[c];
    const float4 d = *reinterpret_cast<const float4*>(dout + i);
    *reinterpret_cast<float4*>(dh + i) = make_float4(s * d.x * g, s * d.y * g, s * d.z * g, s * d.w * g);
}

// dgamma[c] = sum over n and pixels of (s[n] * dout) * h; one workgroup per channel.
__global__ void __launch_bounds__(kRedThreads)
scale_params_kernel(const float* __restrict__ h, const float* __restrict__ dout, const float* __restrict__ scales,
                    float* __restrict__ dgamma, int N, int C, int64_t HW)
{
    __shared__ float red[kRedThreads];
    const int c = blockIdx.x;
    float sg = 0.f;
    for (int n = 0; n < N; ++n) {
        const float s = scales ? scales[n] : 1.f;
        const int64_t base = ((int64_t)n * C + c) * HW;
#pragma unroll 4
        for (int64_t p = threadIdx.x; p < HW; p += kRedThreads)
            sg = __builtin_fmaf(s * dout[base + p], h[base + p], sg);
    }
    sg = block_sum(sg, red);
    if (threadIdx.x == 0) dgamma[c] = sg;
}

int blocks(int64_t work)
{
    return (int)((work + kThreads - 1) / kThreads);
}

}  // namespace

hipError_t launch_layernorm_fwd(int n, int c, int64_t hw, float eps, const float* x, const float* gamma,
                                const float* beta, float* y, float* mean, float* rstd, hipStream_t st)
{
    const int64_t npix = (int64_t)n * hw;
    const dim3 grid((unsigned)((npix + kPix - 1) / kPix));
#define SSCNN_LN_FWD(G, V)                                                                                  \
    hipLaunchKernelGGL((ln_fwd_reg_kernel<G, V>), grid, dim3(kPix * G), 0, st, x, gamma, beta, y, mean, rstd, c, \
                       hw, npix, eps)
    if (c <= 64)
        SSCNN_LN_FWD(4, 16);
    else if (c <= 256)
        SSCNN_LN_FWD(4, 64);
    else if (c <= 512)
        SSCNN_LN_FWD(8, 64);
    else if (c <= 1024)
        SSCNN_LN_FWD(16, 64);
    else
        hipLaunchKernelGGL(ln_fwd_kernel, grid, dim3(kPix * kGroups), 0, st, x, gamma, beta, y, mean, rstd, c, hw,
                           npix, eps);
#undef SSCNN_LN_FWD
    return hipGetLastError();
}

hipError_t launch_layernorm_bwd(int n, int c, int64_t hw, const float* x, const float* dy, const float* gamma,
                                const float* mean, const float* rstd, float* dx, float* dgamma, float* dbeta,
                                hipStream_t st)
{
    const int64_t npix = (int64_t)n * hw;
    if (dx) {
        const dim3 grid((unsigned)((npix + kPix - 1) / kPix));
#define SSCNN_LN_BWD(G, V)                                                                                      \
    hipLaunchKernelGGL((ln_bwd_reg_kernel<G, V>), grid, dim3(kPix * G), 0, st, x, dy, gamma, mean, rstd, dx, c, hw, \
                       npix)
        if (c <= 64)
            SSCNN_LN_BWD(4, 16);
        else if (c <= 256)
            SSCNN_LN_BWD(8, 32);
        else if (c <= 512)
            SSCNN_LN_BWD(16, 32);
        else
            hipLaunchKernelGGL(ln_bwd_kernel, grid, dim3(kPix * kGroups), 0, st, x, dy, gamma, mean, rstd, dx, c,
                               hw, npix);
#undef SSCNN_LN_BWD
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (dgamma || dbeta)
        hipLaunchKernelGGL(ln_params_kernel, dim3(c), dim3(kRedThreads), 0, st, x, dy, mean, rstd, dgamma, dbeta, n,
                           c, hw);
    return hipGetLastError();
}

hipError_t launch_gelu_fwd(int64_t count, const float* x, float* y, hipStream_t st)
{
    hipLaunchKernelGGL(gelu_fwd_kernel, dim3(blocks((count + 3) / 4)), dim3(kThreads), 0, st, x, y, count);
    return hipGetLastError();
}

hipError_t launch_gelu_bwd(int64_t count, const float* x, const float* dy, float* dx, hipStream_t st)
{
    hipLaunchKernelGGL(gelu_bwd_kernel, dim3(blocks((count + 3) / 4)), dim3(kThreads), 0, st, x, dy, dx, count);
    return hipGetLastError();
}

hipError_t launch_droppath_scales(int n, uint64_t seed, uint64_t offset, uint32_t thr, float inv_keep, bool draw,
                                  float* scales, hipStream_t st)
{
    hipLaunchKernelGGL(droppath_kernel, dim3(blocks(n)), dim3(kThreads), 0, st, n, (uint32_t)seed,
                       (uint32_t)(seed >> 32), (uint32_t)offset, (uint32_t)(offset >> 32), thr, inv_keep, draw ? 1 : 0,
                       scales);
    return hipGetLastError();
}

hipError_t launch_scale_residual_fwd(int n, int c, int64_t hw, const float* x, const float* h, const float* gamma,
                                     const float* scales, float* out, hipStream_t st)
{
    const int64_t count = (int64_t)n * c * hw;
    hipLaunchKernelGGL(scale_residual_fwd_kernel, dim3(blocks(count / 4)), dim3(kThreads), 0, st, x, h, gamma, scales,
                       out, c, hw, count);
    return hipGetLastError();
}

hipError_t launch_scale_residual_bwd(int n, int c, int64_t hw, const float* h, const float* dout, const float* gamma,
                                     const float* scales, float* dh, float* dgamma, hipStream_t st)
{
    const int64_t count = (int64_t)n * c * hw;
    if (dh) {
        hipLaunchKernelGGL(scale_residual_bwd_kernel, dim3(blocks(count / 4)), dim3(kThreads), 0, st, dout, gamma,
                           scales, dh, c, hw, count);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (dgamma)
        hipLaunchKernelGGL(scale_params_kernel, dim3(c), dim3(kRedThreads), 0, st, h, dout, scales, dgamma, n, c,
                           hw);
    return hipGetLastError();
}

}  // namespace sscnn
