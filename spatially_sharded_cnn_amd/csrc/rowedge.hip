// rowedge.hip -- height sharding (Shard(2)): the row halo exchange and the
// row-edge kernels.
//
// The pages switch the sharded dimension to H for very high resolutions
// (kwkr.cn retelling, section 5.2: choose the Shard dimension from the input
// resolution, Shard(2) to split the height).  A shard then holds rows
// [s*h, (s+1)*h) of every plane at full width, and a stride-1 k x k layer
// needs k/2 rows from the shard above and below: the row halo.  Rows are
// contiguous in memory, so the exchange copies whole rows.
//
// The convolution of an H-shard is composed of two steps:
//   1. the interior: the ordinary kernels applied to the local slice as if
//      it were a whole image (rows beyond it read as zero);
//   2. the row edge: the kernels here add the terms whose input row (forward,
//      grad_weight) or grad_output row (grad_input) lies in a row halo, for
//      the few output rows next to the top and bottom of the slice.
// Each output is owned by one thread (or, for the depthwise grad_weight, one
// block reduces in thread order): results are reproducible.
#include "internal.h"
#include "rowedge.h"
#include "wavesum.h"

namespace sscnn {
namespace {

// halo[p, e, :] = up[p, rows - hu + e, :] for e < hu, down[p, e - hu, :] for
// hu <= e < hu + hd; zeros where the neighbour is absent.  Each thread copies
// V consecutive floats (V = 4 when rows are whole float4s) of one halo row
// (pe = p * (hu + hd) + e), grid-stride over the halo: every access is a
// contiguous run of a row.
template <int V>
__global__ void __launch_bounds__(256)
row_halo_kernel(const float* __restrict__ up, const float* __restrict__ down, int rows, int width, int hu,
                int hd, int64_t hrows_total, float* __restrict__ halo)
{
    typedef float vec __attribute__((ext_vector_type(V)));
    const int hrows = hu + hd, wv = width / V;
    const int64_t total = hrows_total * wv;
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total; t += (int64_t)gridDim.x * 256) {
        const int64_t pe = t / wv;
        const int cv = (int)(t - pe * wv);
        const int64_t p = pe / hrows;
        const int e = (int)(pe - p * hrows);
        const float* src = e < hu ? (up ? up + (p * rows + rows - hu + e) * width : nullptr)
                                  : (down ? down + (p * rows + e - hu) * width : nullptr);
        vec v = (vec)0.0f;
        if (src) v = reinterpret_cast<const vec*>(src)[cv];
        reinterpret_cast<vec*>(halo + pe * width)[cv] = v;
    }
}

// Output rows with a tap in a row halo: [0, lo) and [hi, count).
struct Strips {
    int lo, hi, count;
    __host__ __device__ int n() const { return lo + (count - hi); }
    __host__ __device__ int row(int e) const { return e < lo ? e : hi + (e - lo); }
};

Strips strips(int lo, int hi, int count)
{
    if (lo > count) lo = count;
    if (hi < 0) hi = 0;
    if (hi > count) hi = count;
    if (hi <= lo) lo = hi = count;    // the strips meet: every row
    return Strips{lo, hi, count};
}

// ---- any layer: one thread per output (forward, grad_input) or weight -------
//
// The local slice has g.h input rows, with hu halo rows above it and hd below;
// the forward reads input row i*stride + kh - pad.

__global__ void __launch_bounds__(256)
row_edge_fwd_kernel(Geom g, Strips sp, int hu, int hd, const float* __restrict__ rh,
                    const float* __restrict__ w, float* __restrict__ y)
{
    const int ne = sp.n(), hrows = hu + hd;
    const int64_t total = (int64_t)g.n * g.co * ne * g.wol;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        int64_t q = t;
        const int j = (int)(q % g.wol); q /= g.wol;
        const int e = (int)(q % ne); q /= ne;
        const int o = (int)(q % g.co);
        const int b = (int)(q / g.co);
        const int i = sp.row(e);
        const int grp = o / g.cog;
        float acc = 0.0f;
        for (int c = 0; c < g.cig; ++c) {
            const int64_t plane = (int64_t)b * g.ci + grp * g.cig + c;
            const float* wp = w + ((int64_t)o * g.cig + c) * g.k * g.k;
            for (int kh = 0; kh < g.k; ++kh) {
                const int r = i * g.stride + kh - g.pad;
                if (r >= 0 && r < g.h) continue;                    // an interior row
                const int ri = r < 0 ? r + hu : hu + (r - g.h);
                if (ri < 0 || ri >= hrows) continue;                // beyond the halo: zero
                const float* hp = rh + (plane * hrows + ri) * g.wl;
                for (int kw = 0; kw < g.k; ++kw) {
                    const int col = j * g.stride + kw - g.pad;
                    if (col < 0 || col >= g.wl) continue;           // the image's zero padding
                    acc = fmaf(wp[kh * g.k + kw], hp[col], acc);
                }
            }
        }
        y[(((int64_t)b * g.co + o) * g.ho + i) * g.wol + j] += acc;
    }
}

__global__ void __launch_bounds__(256)
row_edge_bwd_input_kernel(Geom g, Strips sp, int ghu, int ghd, const float* __restrict__ grh,
                          const float* __restrict__ w, float* __restrict__ gx)
{
    const int ne = sp.n(), ghrows = ghu + ghd;
    const int64_t total = (int64_t)g.n * g.ci * ne * g.wl;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        int64_t q = t;
        const int xx = (int)(q % g.wl); q /= g.wl;
        const int e = (int)(q % ne); q /= ne;
        const int c = (int)(q % g.ci);
        const int b = (int)(q / g.ci);
        const int yy = sp.row(e);
        const int grp = c / g.cig, cl = c - grp * g.cig;
        float acc = 0.0f;
        bool any = false;
        for (int oo = 0; oo < g.cog; ++oo) {
            const int o = grp * g.cog + oo;
            const int64_t plane = (int64_t)b * g.co + o;
            const float* wp = w + ((int64_t)o * g.cig + cl) * g.k * g.k;
            for (int kh = 0; kh < g.k; ++kh) {
                const int tq = yy + g.pad - kh + g.stride * (ghu + 1);   // > 0: floor-safe
                if (tq % g.stride != 0) continue;
                const int ri = tq / g.stride - 1;                     // row in [halo_u | slice | halo_d]
                if (ri < 0 || ri >= g.ho + ghrows) continue;          // beyond the halo: zero
                if (ri >= ghu && ri < ghu + g.ho) continue;           // an interior row
                const float* hp = grh + (plane * ghrows + (ri < ghu ? ri : ri - g.ho)) * g.wol;
                for (int kw = 0; kw < g.k; ++kw) {
                    const int tc = xx + g.pad - kw;
                    if (tc < 0 || tc % g.stride != 0) continue;
                    const int jj = tc / g.stride;
                    if (jj >= g.wol) continue;
                    acc = fmaf(wp[kh * g.k + kw], hp[jj], acc);
                    any = true;
                }
            }
        }
        if (any) gx[(((int64_t)b * g.ci + c) * g.h + yy) * g.wl + xx] += acc;
    }
}

__global__ void __launch_bounds__(256)
row_edge_bwd_weight_kernel(Geom g, int hu, int hd, const float* __restrict__ rh, const float* __restrict__ gy,
                           float* __restrict__ gw)
{
    const int hrows = hu + hd;
    const int64_t total = (int64_t)g.co * g.cig * g.k * g.k;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        int64_t q = t;
        const int kw = (int)(q % g.k); q /= g.k;
        const int kh = (int)(q % g.k); q /= g.k;
        const int c = (int)(q % g.cig);
        const int o = (int)(q / g.cig);
        const int cin = (o / g.cog) * g.cig + c;
        // own output rows i whose tap kh reads a halo row: i*stride + kh - pad < 0 or >= h
        int il = g.pad > kh ? (g.pad - kh + g.stride - 1) / g.stride : 0;
        if (il > g.ho) il = g.ho;
        const int num = g.h + g.pad - kh;
        int ir = num <= 0 ? 0 : (num + g.stride - 1) / g.stride;
        if (ir > g.ho) ir = g.ho;
        if (ir < il) ir = il;
        if (il == 0 && ir == g.ho) continue;                     // this tap never reads a halo row
        float acc = 0.0f;
        for (int b = 0; b < g.n; ++b) {
            const int64_t xplane = (int64_t)b * g.ci + cin;
            const int64_t gplane = (int64_t)b * g.co + o;
            for (int pass = 0; pass < 2; ++pass) {
                const int i0 = pass ? ir : 0, i1 = pass ? g.ho : il;
                for (int i = i0; i < i1; ++i) {
                    const int r = i * g.stride + kh - g.pad;
                    const int ri = r < 0 ? r + hu : hu + (r - g.h);
                    if (ri < 0 || ri >= hrows) continue;
                    const float* hp = rh + (xplane * hrows + ri) * g.wl;
                    const float* grow = gy + (gplane * g.ho + i) * g.wol;
                    for (int j = 0; j < g.wol; ++j) {
                        const int col = j * g.stride + kw - g.pad;
                        if (col < 0 || col >= g.wl) continue;
                        acc = fmaf(grow[j], hp[col], acc);
                    }
                }
            }
        }
        gw[t] += acc;
    }
}

// ---- depthwise, stride 1, odd k, pad k/2 (row halos of P rows each side) ----
//
// Output row i < P of the top strip reads halo row i + kh for the taps
// kh < P - i; output row h - P + m of the bottom strip reads halo row
// m + kh - P (in [P, 2P)) for the taps kh >= 2P - m.  Columns beyond the
// image are its zero padding.

bool dw_rows(const Geom& g)
{
    return g.groups == g.ci && g.ci == g.co && g.stride == 1 && (g.k == 3 || g.k == 5 || g.k == 7) &&
           g.pad == g.k / 2 && g.h >= 2 * g.pad;
}

// One thread per (plane, column): the column's 2P strip outputs (top P rows,
// bottom P rows).  A block is 256 columns of one plane, so the plane's taps
// are block-uniform; every halo value and strip output the thread needs is
// loaded before the first multiply.
template <int K, bool FLIP>
__global__ void __launch_bounds__(256)
dw_row_edge_kernel(const float* __restrict__ rh, const float* __restrict__ w, float* __restrict__ out, int C,
                   int H, int W, int col_blocks)
{
    constexpr int P = K / 2;
    const int plane = blockIdx.x / col_blocks;
    const int j = (blockIdx.x - plane * col_blocks) * 256 + threadIdx.x;
    const auto wp = as_const(w) + (int64_t)(plane % C) * K * K;
    float wr[K * K];
#pragma unroll
    for (int k = 0; k < K * K; ++k) wr[k] = wp[FLIP ? K * K - 1 - k : k];
    if (j >= W) return;
    const float* hp = rh + (int64_t)plane * (2 * P) * W;
    float* op = out + (int64_t)plane * H * W + j;
    float h[2 * P][K];                          // halo rows x columns j - P .. j + P
#pragma unroll
    for (int q = 0; q < 2 * P; ++q)
#pragma unroll
        for (int kw = 0; kw < K; ++kw) {
            const int col = j + kw - P;
            h[q][kw] = (col >= 0 && col < W) ? hp[(int64_t)q * W + col] : 0.0f;
        }
    float o[2 * P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        o[i] = op[(int64_t)i * W];
        o[P + i] = op[(int64_t)(H - P + i) * W];
    }
#pragma unroll
    for (int i = 0; i < P; ++i) {               // top row i: halo rows i + kh for kh < P - i
        float acc = 0.0f;
#pragma unroll
        for (int kh = 0; kh < P - i; ++kh)
#pragma unroll
            for (int kw = 0; kw < K; ++kw) acc = fmaf(wr[kh * K + kw], h[i + kh][kw], acc);
        op[(int64_t)i * W] = o[i] + acc;
    }
#pragma unroll
    for (int m = 0; m < P; ++m) {               // bottom row H - P + m: halo rows m + kh - P for kh >= 2P - m
        float acc = 0.0f;
#pragma unroll
        for (int kh = 2 * P - m; kh < K; ++kh)
#pragma unroll
            for (int kw = 0; kw < K; ++kw) acc = fmaf(wr[kh * K + kw], h[m + kh - P][kw], acc);
        op[(int64_t)(H - P + m) * W] = o[P + m] + acc;
    }
}

// Depthwise grad_weight, in two passes.  First one 256-thread block per
// (channel, image), threads over the columns: each thread sums the taps that
// read a halo row (kh < P: top, kh > P: bottom) over its columns; each wave
// adds its lanes' sums (a fixed-order cross-lane reduce-scatter), and the
// block adds the four waves' totals in order and writes one partial per tap.
// Then one thread per (channel, tap) adds the images' partials in order.
template <int K>
__global__ void __launch_bounds__(256)
dw_row_edge_wgrad_kernel(const float* __restrict__ rh, const float* __restrict__ gy, float* __restrict__ part,
                         int N, int C, int H, int W)
{
    constexpr int P = K / 2, NA = 2 * P * K;      // acc[q * K + kw]: kh = q (q < P) or q + 1 (q >= P)
    __shared__ float red[4][NA];
    const int c = blockIdx.x / N, n = blockIdx.x - c * N, tid = threadIdx.x;
    float acc[NA];
#pragma unroll
    for (int a = 0; a < NA; ++a) acc[a] = 0.0f;
    const int64_t plane = (int64_t)n * C + c;
    const float* hp = rh + plane * (2 * P) * W;
    for (int j = tid; j < W; j += 256) {
        const float* gp = gy + plane * H * W + j;
        float g[2 * P];                           // grad_output at the strip rows: top P, bottom P
#pragma unroll
        for (int q = 0; q < P; ++q) {
            g[q] = gp[(int64_t)q * W];
            g[P + q] = gp[(int64_t)(H - P + q) * W];
        }
        float h[2 * P][K];
#pragma unroll
        for (int q = 0; q < 2 * P; ++q)
#pragma unroll
            for (int kw = 0; kw < K; ++kw) {
                const int col = j + kw - P;
                h[q][kw] = (col >= 0 && col < W) ? hp[(int64_t)q * W + col] : 0.0f;
            }
#pragma unroll
        for (int kw = 0; kw < K; ++kw) {
#pragma unroll
            for (int kh = 0; kh < P; ++kh)        // top: rows i < P - kh read halo row i + kh
#pragma unroll
                for (int i = 0; i < P - kh; ++i) acc[kh * K + kw] = fmaf(g[i], h[i + kh][kw], acc[kh * K + kw]);
#pragma unroll
            for (int kh = P + 1; kh < K; ++kh)    // bottom: rows H - P + m, m >= 2P - kh, read halo row m + kh - P
#pragma unroll
                for (int m = 2 * P - kh; m < P; ++m)
                    acc[(kh - 1) * K + kw] = fmaf(g[P + m], h[m + kh - P][kw], acc[(kh - 1) * K + kw]);
        }
    }
    {
        const int lane = tid & 63, wave = tid >> 6;
        const float s = wave_sum_scatter<NA>(acc, lane);
        const int idx = wave_sum_index<NA>(lane);
        if (idx >= 0) red[wave][idx] = s;
    }
    __syncthreads();
    if (tid < NA)
        part[((int64_t)c * N + n) * NA + tid] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
}

template <int K>
__global__ void __launch_bounds__(256)
dw_row_edge_wgrad_sum_kernel(const float* __restrict__ part, float* __restrict__ gw, int N, int C)
{
    constexpr int P = K / 2, NA = 2 * P * K;
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= C * NA) return;
    const int c = t / NA, a = t - c * NA;
    float sum = 0.0f;
    for (int n = 0; n < N; ++n) sum += part[((int64_t)c * N + n) * NA + a];
    const int q = a / K, kw = a - q * K;
    const int kh = q < P ? q : q + 1;
    gw[((int64_t)c * K + kh) * K + kw] += sum;
}

int grid_for(int64_t work)
{
    int64_t blocks = (work + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 1 << 20) blocks = 1 << 20;
    return (int)blocks;
}

template <int K, bool FLIP>
void dw_row_launch(const Geom& g, const float* rh, const float* w, float* out, hipStream_t st)
{
    const int col_blocks = (g.wl + 255) / 256;
    const int64_t blocks = (int64_t)g.n * g.ci * col_blocks;
    hipLaunchKernelGGL((dw_row_edge_kernel<K, FLIP>), dim3((unsigned)blocks), dim3(256), 0, st, rh, w, out, g.ci,
                       g.h, g.wl, col_blocks);
}

}  // namespace

namespace {

// 2-D shards, second phase of the exchange: the columns beside a block over
// its extended rows (the up rows above it, its own rows, the down rows below).
// Extended row e (row r = e - up of the block) of the left neighbour is its
// row r for 0 <= r < rows, else a row of its row halo, which its first phase
// filled from the blocks above and below it: so the corners travel with the
// columns.  out[p, e, :] = left columns hl, then right columns hr.
__global__ void __launch_bounds__(256)
grid_col_halo_kernel(const float* __restrict__ left, const float* __restrict__ left_rh,
                     const float* __restrict__ right, const float* __restrict__ right_rh, int64_t planes, int rows,
                     int width, int up, int down, int hl, int hr, float* __restrict__ out)
{
    const int ext = up + rows + down, wh = hl + hr;
    const int64_t total = planes * ext * wh;
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total; t += (int64_t)gridDim.x * 256) {
        const int col = (int)(t % wh);
        const int64_t pe = t / wh;
        const int e = (int)(pe % ext);
        const int64_t p = pe / ext;
        const int r = e - up;
        const bool lft = col < hl;
        const float* slice = lft ? left : right;
        const float* rh = lft ? left_rh : right_rh;
        const int x = lft ? width - hl + col : col - hl;
        float v = 0.f;
        if (r >= 0 && r < rows) {
            if (slice) v = slice[(p * rows + r) * width + x];
        } else if (rh) {
            const int hrow = r < 0 ? up + r : up + (r - rows);
            v = rh[(p * (up + down) + hrow) * width + x];
        }
        out[t] = v;
    }
}

}  // namespace

hipError_t launch_grid_col_halo(const float* left, const float* left_rh, const float* right, const float* right_rh,
                                int64_t planes, int rows, int width, int up, int down, int hl, int hr, float* out,
                                hipStream_t st)
{
    const int64_t total = planes * (up + rows + down) * (hl + hr);
    if (total == 0) return hipSuccess;
    const int grid = (int)((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
    hipLaunchKernelGGL(grid_col_halo_kernel, dim3(grid), dim3(256), 0, st, left, left_rh, right, right_rh, planes,
                       rows, width, up, down, hl, hr, out);
    return hipGetLastError();
}

hipError_t launch_row_halo_gather(const float* up, const float* down, int64_t planes, int rows, int width, int hu,
                                  int hd, float* halo, hipStream_t st)
{
    const int64_t hrows = planes * (hu + hd);
    if (hrows == 0 || width == 0) return hipSuccess;
    // whole float4s per row (the ABI's 16-byte aligned bases keep them aligned)
    const bool v4 = width % 4 == 0;
    const int64_t work = hrows * (v4 ? width / 4 : width);
    const int grid = (int)((work + 255) / 256 < 4096 ? (work + 255) / 256 : 4096);
    if (v4)
        hipLaunchKernelGGL(row_halo_kernel<4>, dim3(grid), dim3(256), 0, st, up, down, rows, width, hu, hd, hrows,
                           halo);
    else
        hipLaunchKernelGGL(row_halo_kernel<1>, dim3(grid), dim3(256), 0, st, up, down, rows, width, hu, hd, hrows,
                           halo);
    return hipGetLastError();
}

hipError_t launch_row_edge_fwd(const Geom& g, int hu, int hd, const float* rh, const float* w, float* y,
                               hipStream_t st)
{
    if (hu + hd == 0) return hipSuccess;
    if (dw_rows(g) && hu == g.pad && hd == g.pad) {
        switch (g.k) {
            case 3: dw_row_launch<3, false>(g, rh, w, y, st); break;
            case 5: dw_row_launch<5, false>(g, rh, w, y, st); break;
            default: dw_row_launch<7, false>(g, rh, w, y, st); break;
        }
        return hipGetLastError();
    }
    // rows with a tap in a halo row: i*stride < hu (top) and i*stride + k - 1 - pad >= h (bottom)
    const int lo = (hu + g.stride - 1) / g.stride;
    const int num = g.h + g.pad - g.k + 1;
    const int hi = hd == 0 ? g.ho : (num <= 0 ? 0 : (num + g.stride - 1) / g.stride);
    const Strips sp = strips(lo, hi, g.ho);
    const int64_t total = (int64_t)g.n * g.co * sp.n() * g.wol;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(row_edge_fwd_kernel, dim3(grid_for(total)), dim3(256), 0, st, g, sp, hu, hd, rh, w, y);
    return hipGetLastError();
}

hipError_t launch_row_edge_bwd_input(const Geom& g, int ghu, int ghd, const float* grh, const float* w, float* gx,
                                     hipStream_t st)
{
    if (ghu + ghd == 0) return hipSuccess;
    if (dw_rows(g) && ghu == g.pad && ghd == g.pad) {
        switch (g.k) {
            case 3: dw_row_launch<3, true>(g, grh, w, gx, st); break;
            case 5: dw_row_launch<5, true>(g, grh, w, gx, st); break;
            default: dw_row_launch<7, true>(g, grh, w, gx, st); break;
        }
        return hipGetLastError();
    }
    // input rows reading a grad_output row above the slice: yy + pad - (k - 1) < 0;
    // below it: yy + pad >= ho * stride = h
    const int lo = ghu == 0 ? 0 : (g.k - 1 - g.pad > 0 ? g.k - 1 - g.pad : 0);
    const int hi = ghd == 0 ? g.h : g.h - g.pad;
    const Strips sp = strips(lo, hi, g.h);
    const int64_t total = (int64_t)g.n * g.ci * sp.n() * g.wl;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(row_edge_bwd_input_kernel, dim3(grid_for(total)), dim3(256), 0, st, g, sp, ghu, ghd, grh, w,
                       gx);
    return hipGetLastError();
}

size_t row_edge_workspace_bytes(const Geom& g)
{
    if (!dw_rows(g)) return 0;
    return (size_t)g.n * g.ci * (2 * (g.k / 2) * g.k) * sizeof(float);
}

hipError_t launch_row_edge_bwd_weight(const Geom& g, int hu, int hd, const float* rh, const float* gy, float* gw,
                                      void* ws, hipStream_t st)
{
    if (hu + hd == 0) return hipSuccess;
    if (dw_rows(g) && hu == g.pad && hd == g.pad) {
        float* part = static_cast<float*>(ws);
        const int na = 2 * (g.k / 2) * g.k;
        const int sum_blocks = (g.ci * na + 255) / 256;
        switch (g.k) {
#define SSCNN_DW_RW(K)                                                                                              \
    case K:                                                                                                         \
        hipLaunchKernelGGL((dw_row_edge_wgrad_kernel<K>), dim3((unsigned)(g.ci * g.n)), dim3(256), 0, st, rh, gy,   \
                           part, g.n, g.ci, g.h, g.wl);                                                             \
        hipLaunchKernelGGL((dw_row_edge_wgrad_sum_kernel<K>), dim3(sum_blocks), dim3(256), 0, st, part, gw, g.n,    \
                           g.ci);                                                                                   \
        break;
            SSCNN_DW_RW(3)
            SSCNN_DW_RW(5)
            SSCNN_DW_RW(7)
#undef SSCNN_DW_RW
        }
        return hipGetLastError();
    }
    const int64_t total = (int64_t)g.co * g.cig * g.k * g.k;
    hipLaunchKernelGGL(row_edge_bwd_weight_kernel, dim3(grid_for(total)), dim3(256), 0, st, g, hu, hd, rh, gy, gw);
    return hipGetLastError();
}

}  // namespace sscnn
