// edge.hip -- the edge half of a split convolution.
//
// Splitting a layer into a part that needs no halo and a part that does lets
// the halo exchange run while the bulk of the layer is computed (kwkr.cn
// retelling, section 5.2: overlap communication with the computation that
// does not depend on it).  The interior calls run the ordinary kernels with
// the halo read as zeros; every output that a halo column feeds then lacks
// exactly the terms that involve that column, and the kernels here add them:
//
//   forward      y[n, o, i, j]      += sum over the halo taps of w * x_halo
//   grad_input   gx[n, c, yy, xx]   += sum over the halo taps of w * g_halo
//   grad_weight  gw[o, c, kh, kw]   += sum over the shard's own output columns
//                                      j whose tap (kh, kw) reads the input
//                                      halo, of g * x_halo
//
// A halo tap is one whose column of the extended row [halo_l | slice |
// halo_r] lies outside the slice.  Only the few output columns next to a
// shard edge have any (a strip of about k/2 columns on each side); the
// grad_weight terms are the products along those strips.  Each output is
// owned by one thread, which sums its terms in a fixed order and adds the sum
// once: results are reproducible, and equal the monolithic call's up to the
// rounding of that addition.
//
// Index conventions are those of the direct kernels (direct.hip): the forward
// reads extended column j*stride + kw, grad_input reads extended grad_output
// column (xx + pad - kw)/stride + ghalo_l where the division is exact.
#include "internal.h"
#include "edge.h"
#include "wavesum.h"

namespace sscnn {
namespace {

// Output columns of the forward with a halo tap: [0, jl) and [jr, wol).
struct Strips {
    int lo, hi;   // [0, lo) and [hi, count)
    int count;    // columns in the row
    __host__ __device__ int n() const { return lo + (count - hi); }
    __host__ __device__ int col(int e) const { return e < lo ? e : hi + (e - lo); }
};

Strips strips(int lo, int hi, int count)
{
    if (lo > count) lo = count;
    if (hi < 0) hi = 0;
    if (hi > count) hi = count;
    if (hi <= lo) {   // the two strips meet: every column
        lo = count;
        hi = count;
    }
    return Strips{lo, hi, count};
}

// Forward: column j has a left halo tap when j*stride < hl (tap kw = 0) and a
// right one when j*stride + k - 1 >= hl + wl (tap kw = k - 1).
Strips fwd_strips(const Geom& g)
{
    const int lo = (g.hl + g.stride - 1) / g.stride;
    const int num = g.hl + g.wl - g.k + 1;
    const int hi = g.hr == 0 ? g.wol : (num <= 0 ? 0 : (num + g.stride - 1) / g.stride);
    return strips(lo, hi, g.wol);
}

// grad_input: column xx reads grad_output column (xx + pad - kw)/stride,
// which is left of the slice only if xx + pad - (k - 1) < 0 and right of it
// only if xx + pad >= wol*stride = wl.  Columns of the strips for which no
// quotient is exact have no halo term and are left untouched.
Strips bwd_input_strips(const Geom& g)
{
    const int lo = g.ghl == 0 ? 0 : (g.k - 1 - g.pad > 0 ? g.k - 1 - g.pad : 0);
    const int hi = g.ghr == 0 ? g.wl : g.wl - g.pad;
    return strips(lo, hi, g.wl);
}

__global__ void __launch_bounds__(256)
edge_fwd_kernel(Geom g, Strips sp, const float* __restrict__ xh, const float* __restrict__ w,
                float* __restrict__ y)
{
    const int ne = sp.n();
    const int64_t total = (int64_t)g.n * g.co * g.ho * ne;
    const int hw = g.hl + g.hr;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        int64_t q = t;
        const int e = (int)(q % ne); q /= ne;
        const int i = (int)(q % g.ho); q /= g.ho;
        const int o = (int)(q % g.co);
        const int b = (int)(q / g.co);
        const int j = sp.col(e);
        const int grp = o / g.cog;
        const int e0 = j * g.stride;                         // extended column of tap kw = 0
        int kl = g.hl - e0;                                  // taps kw < kl read the left halo
        kl = kl < 0 ? 0 : (kl > g.k ? g.k : kl);
        int kr = g.hl + g.wl - e0;                           // taps kw >= kr read the right halo
        kr = kr < 0 ? 0 : (kr > g.k ? g.k : kr);
        float acc = 0.0f;
        for (int c = 0; c < g.cig; ++c) {
            const int64_t plane = (int64_t)b * g.ci + grp * g.cig + c;
            const float* wp = w + ((int64_t)o * g.cig + c) * g.k * g.k;
            for (int kh = 0; kh < g.k; ++kh) {
                const int r = i * g.stride + kh - g.pad;
                if (r < 0 || r >= g.h) continue;
                const float* hp = xh + (plane * g.h + r) * hw;
                for (int kw = 0; kw < kl; ++kw) acc = fmaf(wp[kh * g.k + kw], hp[e0 + kw], acc);
                for (int kw = kr; kw < g.k; ++kw) acc = fmaf(wp[kh * g.k + kw], hp[e0 + kw - g.wl], acc);
            }
        }
        y[(((int64_t)b * g.co + o) * g.ho + i) * g.wol + j] += acc;
    }
}

__global__ void __launch_bounds__(256)
edge_bwd_input_kernel(Geom g, Strips sp, const float* __restrict__ gyh, const float* __restrict__ w,
                      float* __restrict__ gx)
{
    const int ne = sp.n();
    const int64_t total = (int64_t)g.n * g.ci * g.h * ne;
    const int ghw = g.ghl + g.ghr;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        int64_t q = t;
        const int e = (int)(q % ne); q /= ne;
        const int yy = (int)(q % g.h); q /= g.h;
        const int c = (int)(q % g.ci);
        const int b = (int)(q / g.ci);
        const int xx = sp.col(e);
        const int grp = c / g.cig, cl = c - grp * g.cig;
        float acc = 0.0f;
        bool any = false;
        for (int oo = 0; oo < g.cog; ++oo) {
            const int o = grp * g.cog + oo;
            const int64_t plane = (int64_t)b * g.co + o;
            const float* wp = w + ((int64_t)o * g.cig + cl) * g.k * g.k;
            for (int kh = 0; kh < g.k; ++kh) {
                const int tr = yy + g.pad - kh;
                if (tr < 0 || tr % g.stride != 0) continue;
                const int i = tr / g.stride;
                if (i >= g.ho) continue;
                const float* hp = gyh + (plane * g.ho + i) * ghw;
                for (int kw = 0; kw < g.k; ++kw) {
                    const int tq = xx + g.pad - kw + g.stride * (g.ghl + 1);   // > 0: floor-safe
                    if (tq % g.stride != 0) continue;
                    const int ec = tq / g.stride - 1;                        // extended column
                    if (ec < 0 || ec >= g.wol + ghw) continue;               // beyond the halo: zero
                    if (ec >= g.ghl && ec < g.ghl + g.wol) continue;         // in the slice: interior
                    const int hidx = ec < g.ghl ? ec : ec - g.wol;
                    acc = fmaf(wp[kh * g.k + kw], hp[hidx], acc);
                    any = true;
                }
            }
        }
        if (any) gx[(((int64_t)b * g.ci + c) * g.h + yy) * g.wl + xx] += acc;
    }
}

__global__ void __launch_bounds__(256)
edge_bwd_weight_kernel(Geom g, const float* __restrict__ xh, const float* __restrict__ gy,
                       float* __restrict__ gw)
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
        // own output columns j whose tap kw reads the halo: j*stride + kw < hl
        // (left) or >= hl + wl (right)
        int jl = g.hl > kw ? (g.hl - kw + g.stride - 1) / g.stride : 0;
        if (jl > g.wol) jl = g.wol;
        const int num = g.hl + g.wl - kw;
        int jr = num <= 0 ? 0 : (num + g.stride - 1) / g.stride;
        if (jr > g.wol) jr = g.wol;
        if (jr < jl) jr = jl;
        if (jl == 0 && jr == g.wol) continue;                // this tap never reads a halo
        float acc = 0.0f;
        for (int b = 0; b < g.n; ++b) {
            const int64_t xplane = (int64_t)b * g.ci + cin;
            const int64_t gplane = (int64_t)b * g.co + o;
            for (int i = 0; i < g.ho; ++i) {
                const int r = i * g.stride + kh - g.pad;
                if (r < 0 || r >= g.h) continue;
                const float* grow = gy + (gplane * g.ho + i) * g.wol;
                const float* hp = xh + (xplane * g.h + r) * hw;
                for (int j = 0; j < jl; ++j) acc = fmaf(grow[j], hp[j * g.stride + kw], acc);
                for (int j = jr; j < g.wol; ++j) acc = fmaf(grow[j], hp[j * g.stride + kw - g.wl], acc);
            }
        }
        gw[t] += acc;
    }
}

// ---- fast paths: stride 1, odd k, pad k/2 (halo widths P = k/2 on both sides
// for the input and the grad_output), slices at least 2P wide ----------------
//
// The strips are then the P first and the P last columns of a row.  Output
// column j < P of the left strip reads halo column j + kw for the taps
// kw < P - j; output column W - P + m of the right strip reads halo column
// m + kw - P (in [P, 2P), the right neighbour's part) for the taps kw >= 2P - m.
// grad_input is the forward on the grad_output halo with the weights
// flipped in both axes (and, for a dense layer, transposed), so one kernel
// serves both.

bool symmetric(const Geom& g)
{
    return g.stride == 1 && g.k % 2 == 1 && g.pad == g.k / 2 && g.wl >= 2 * g.pad && g.pad > 0;
}

bool dw_edge(const Geom& g)
{
    return symmetric(g) && g.groups == g.ci && g.ci == g.co && (g.k == 3 || g.k == 5 || g.k == 7);
}

bool dense_edge(const Geom& g)
{
    return symmetric(g) && g.groups == 1 && (g.k == 3 || g.k == 5);
}

// Depthwise: one thread per (plane, row), both strips of the row.  A block is
// 64 rows of one plane, so the plane's k*k taps are block-uniform (scalar loads).
template <int K, bool FLIP>
__global__ void __launch_bounds__(64)
dw_edge_conv_kernel(const float* __restrict__ sh, const float* __restrict__ w, float* __restrict__ out,
                    int C, int H, int W, int blocks_per_plane)
{
    constexpr int P = K / 2, HW2 = 2 * P;
    const int plane = blockIdx.x / blocks_per_plane;
    const int i = (blockIdx.x - plane * blocks_per_plane) * 64 + threadIdx.x;
    const auto wp = as_const(w) + (int64_t)(plane % C) * K * K;
    float wr[K * K];
#pragma unroll
    for (int k = 0; k < K * K; ++k) wr[k] = wp[FLIP ? K * K - 1 - k : k];
    if (i >= H) return;
    float accl[P], accr[P];
#pragma unroll
    for (int j = 0; j < P; ++j) accl[j] = accr[j] = 0.0f;
    const float* hp = sh + (int64_t)plane * H * HW2;
#pragma unroll
    for (int kh = 0; kh < K; ++kh) {
        const int r = i + kh - P;
        if (r < 0 || r >= H) continue;
        float h[HW2];
#pragma unroll
        for (int q = 0; q < HW2; ++q) h[q] = hp[(int64_t)r * HW2 + q];
#pragma unroll
        for (int j = 0; j < P; ++j)
#pragma unroll
            for (int kw = 0; kw < P - j; ++kw) accl[j] = fmaf(wr[kh * K + kw], h[j + kw], accl[j]);
#pragma unroll
        for (int m = 0; m < P; ++m)
#pragma unroll
            for (int kw = 2 * P - m; kw < K; ++kw) accr[m] = fmaf(wr[kh * K + kw], h[m + kw - P], accr[m]);
    }
    float* op = out + ((int64_t)plane * H + i) * W;
#pragma unroll
    for (int j = 0; j < P; ++j) op[j] += accl[j];
#pragma unroll
    for (int m = 0; m < P; ++m) op[W - P + m] += accr[m];
}

// Depthwise grad_weight: one 256-thread block per channel; each thread sums
// its rows (n, i) for the taps that read a halo (kw < P: left, kw > P:
// right), then each wave adds its lanes' sums (a fixed-order cross-lane
// reduce-scatter) and the block adds the four waves' totals in order.
template <int K>
__global__ void __launch_bounds__(256)
dw_edge_wgrad_kernel(const float* __restrict__ xh, const float* __restrict__ gy, float* __restrict__ gw,
                     int N, int C, int H, int W)
{
    constexpr int P = K / 2, HW2 = 2 * P, NA = K * HW2;   // acc[kh * 2P + q]: kw = q (q < P) or q + 1 (q >= P)
    __shared__ float red[4][NA];
    const int c = blockIdx.x, tid = threadIdx.x;
    float acc[NA];
#pragma unroll
    for (int a = 0; a < NA; ++a) acc[a] = 0.0f;
    for (int row = tid; row < N * H; row += 256) {
        const int n = row / H, i = row - n * H;
        const int64_t plane = (int64_t)n * C + c;
        const float* gp = gy + (plane * H + i) * W;
        float g[HW2];                                     // [left strip | right strip]
#pragma unroll
        for (int j = 0; j < P; ++j) {
            g[j] = gp[j];
            g[P + j] = gp[W - P + j];
        }
        const float* hp = xh + plane * H * HW2;
#pragma unroll
        for (int kh = 0; kh < K; ++kh) {
            const int r = i + kh - P;
            if (r < 0 || r >= H) continue;
            float h[HW2];
#pragma unroll
            for (int q = 0; q < HW2; ++q) h[q] = hp[(int64_t)r * HW2 + q];
#pragma unroll
            for (int kw = 0; kw < P; ++kw)
#pragma unroll
                for (int j = 0; j < P - kw; ++j) acc[kh * HW2 + kw] = fmaf(g[j], h[j + kw], acc[kh * HW2 + kw]);
#pragma unroll
            for (int kw = P + 1; kw < K; ++kw)
#pragma unroll
                for (int m = 2 * P - kw; m < P; ++m)
                    acc[kh * HW2 + kw - 1] = fmaf(g[P + m], h[m + kw - P], acc[kh * HW2 + kw - 1]);
        }
    }
    {
        const int lane = tid & 63, wave = tid >> 6;
        const float s = wave_sum_scatter<NA>(acc, lane);
        const int idx = wave_sum_index<NA>(lane);
        if (idx >= 0) red[wave][idx] = s;
    }
    __syncthreads();
    if (tid < NA) {
        const float sum = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
        const int kh = tid / HW2, q = tid - kh * HW2;
        const int kw = q < P ? q : q + 1;
        gw[((int64_t)c * K + kh) * K + kw] += sum;
    }
}

// Dense forward / grad_input strips.  Roles: O output channels, CR reduction
// channels; the forward reads W[o][c][kh][kw], grad_input (TRANS) reads
// W[c][o][K-1-kh][K-1-kw].  A block is one side (left / right strip), one
// image, 32 output rows and 32 output channels: 128 threads = 32 channels x
// 4 groups of 8 rows (small blocks, so that a layer has several per CU).  The
// reduction runs over chunks of 8 channels.  For a chunk each thread stages
// two (output, reduction) channel pairs: the P taps
// per kernel row that read this side's halo, all loads issued before the
// LDS writes; the chunk's halo rows go to LDS beside them.  Each thread then
// holds its rows' halo window and the chunk's taps in registers while it
// accumulates.  The side is a template parameter of the body, so the tap
// pattern is fixed at compile time.
constexpr int kDO = 32, kDR = 32, kDRG = 8, kDC = 8, kDT = kDO * kDR / kDRG, kDP = kDO * kDC / kDT;
static_assert(kDO * kDC == kDP * kDT, "whole (o, c) pairs per thread in a chunk");

template <int K, bool TRANS, int SIDE>
__device__ __forceinline__ void dense_edge_conv_body(const float* __restrict__ sh, const float* __restrict__ w,
                                                     float* __restrict__ out, int n, int o0, int i0, int O,
                                                     int CR, int H, int W, float* ws, float* hs)
{
    constexpr int P = K / 2, KK = K * K, HW2 = 2 * P, WIN = kDRG + K - 1, HR = kDR + K - 1;
    constexpr int HS = kDC * HR * P, NH = (HS + kDT - 1) / kDT;
    const int tid = threadIdx.x, ol = tid & (kDO - 1), rg = tid / kDO;
    float acc[kDRG][P];
#pragma unroll
    for (int r = 0; r < kDRG; ++r)
#pragma unroll
        for (int j = 0; j < P; ++j) acc[r][j] = 0.0f;
    // a chunk's loads go to registers (issued one chunk ahead, while the
    // chunk before it is multiplied), then to LDS
    float vw[kDP][K][P], vh[NH];
    auto fetch = [&](int c0) {
        // the staged pairs: forward (o, cc) with cc fastest (W[o][c0 .. c0 + 7] adjacent),
        // grad_input (cc, o) with o fastest (W[c][o0 .. o0 + 31] adjacent)
#pragma unroll
        for (int pp = 0; pp < kDP; ++pp) {
            const int pair = tid + kDT * pp;
            const int pcc = TRANS ? pair / kDO : pair % kDC;
            const int pol = TRANS ? pair % kDO : pair / kDC;
            const int o = o0 + pol, c = c0 + pcc;
            const bool ok = o < O && c < CR;
            const float* wp = w + (TRANS ? (int64_t)c * O + o : (int64_t)o * CR + c) * KK;
#pragma unroll
            for (int kh = 0; kh < K; ++kh)
#pragma unroll
                for (int kwl = 0; kwl < P; ++kwl) {
                    const int kw = SIDE ? P + 1 + kwl : kwl;               // as the kernel uses it
                    const int t = TRANS ? KK - 1 - (kh * K + kw) : kh * K + kw;   // in the tensor
                    vw[pp][kh][kwl] = ok ? wp[t] : 0.0f;
                }
        }
#pragma unroll
        for (int k = 0; k < NH; ++k) {
            const int idx = tid + kDT * k;
            const int q = idx % P;
            const int rest = idx / P;
            const int rr = rest % HR, cc = rest / HR;
            const int r = i0 - P + rr, c = c0 + cc;
            vh[k] = 0.0f;
            if (idx < HS && c < CR && r >= 0 && r < H)
                vh[k] = sh[(((int64_t)n * CR + c) * H + r) * HW2 + SIDE * P + q];
        }
    };
    fetch(0);
    for (int c0 = 0; c0 < CR; c0 += kDC) {
#pragma unroll
        for (int pp = 0; pp < kDP; ++pp) {
            const int pair = tid + kDT * pp;
            const int pcc = TRANS ? pair / kDO : pair % kDC;
            const int pol = TRANS ? pair % kDO : pair / kDC;
#pragma unroll
            for (int kh = 0; kh < K; ++kh)
#pragma unroll
                for (int kwl = 0; kwl < P; ++kwl) ws[((pcc * K + kh) * P + kwl) * kDO + pol] = vw[pp][kh][kwl];
        }
#pragma unroll
        for (int k = 0; k < NH; ++k)
            if (tid + kDT * k < HS) hs[tid + kDT * k] = vh[k];
        __syncthreads();
        if (c0 + kDC < CR) fetch(c0 + kDC);
        for (int cc = 0; cc < kDC; ++cc) {
            float wv[K][P], hv[WIN][P];
#pragma unroll
            for (int kh = 0; kh < K; ++kh)
#pragma unroll
                for (int kwl = 0; kwl < P; ++kwl) wv[kh][kwl] = ws[((cc * K + kh) * P + kwl) * kDO + ol];
#pragma unroll
            for (int rr = 0; rr < WIN; ++rr)
#pragma unroll
                for (int q = 0; q < P; ++q) hv[rr][q] = hs[(cc * HR + rg * kDRG + rr) * P + q];
#pragma unroll
            for (int r = 0; r < kDRG; ++r)
#pragma unroll
                for (int kh = 0; kh < K; ++kh) {
                    if constexpr (SIDE == 0) {
#pragma unroll
                        for (int j = 0; j < P; ++j)
#pragma unroll
                            for (int kw = 0; kw < P - j; ++kw)
                                acc[r][j] = fmaf(wv[kh][kw], hv[r + kh][j + kw], acc[r][j]);
                    } else {
#pragma unroll
                        for (int m = 0; m < P; ++m)
#pragma unroll
                            for (int kw = 2 * P - m; kw < K; ++kw)
                                acc[r][m] = fmaf(wv[kh][kw - P - 1], hv[r + kh][m + kw - 2 * P], acc[r][m]);
                    }
                }
        }
        __syncthreads();
    }
    const int o = o0 + ol;
    if (o >= O) return;
#pragma unroll
    for (int r = 0; r < kDRG; ++r) {
        const int i = i0 + rg * kDRG + r;
        if (i >= H) break;
        float* op = out + (((int64_t)n * O + o) * H + i) * W + (SIDE ? W - P : 0);
#pragma unroll
        for (int j = 0; j < P; ++j) op[j] += acc[r][j];
    }
}

template <int K, bool TRANS>
__global__ void __launch_bounds__(kDT)
dense_edge_conv_kernel(const float* __restrict__ sh, const float* __restrict__ w, float* __restrict__ out,
                       int N, int O, int CR, int H, int W, int row_blocks)
{
    constexpr int P = K / 2;
    __shared__ float ws[kDC * K * P * kDO];                // [cc][kh][kwl][o]
    __shared__ float hs[kDC * (kDR + K - 1) * P];          // [cc][rr][q]
    // (row block, n) fastest: the blocks of one (side, channel block) read the
    // same taps and run side by side on one XCD
    int b = xcd_order(blockIdx.x, gridDim.x);
    const int rb = b % row_blocks;
    b /= row_blocks;
    const int n = b % N;
    b /= N;
    const int side = b & 1;
    const int o0 = (b >> 1) * kDO, i0 = rb * kDR;
    if (side == 0) dense_edge_conv_body<K, TRANS, 0>(sh, w, out, n, o0, i0, O, CR, H, W, ws, hs);
    else dense_edge_conv_body<K, TRANS, 1>(sh, w, out, n, o0, i0, O, CR, H, W, ws, hs);
}

// Dense grad_weight: a block owns 16 output x 16 input channels (one (o, c)
// pair per thread, all its halo taps: K x 2P sums) and walks every row of
// every image in chunks of 16 rows staged in LDS: the grad_output strip
// values and the input halo rows.  Each thread sums its rows in order.
constexpr int kWO = 16, kWCI = 16, kWR = 16;

template <int K>
__global__ void __launch_bounds__(256)
dense_edge_wgrad_kernel(const float* __restrict__ xh, const float* __restrict__ gy, float* __restrict__ gw,
                        int N, int CO, int CI, int H, int W, int c_blocks)
{
    constexpr int P = K / 2, HW2 = 2 * P;
    __shared__ float gs[kWR][kWO][HW2];
    __shared__ float xs[kWCI][kWR + K - 1][HW2];
    // input-channel block fastest: the blocks of one output-channel block read
    // the same grad_output strips and run side by side on one XCD
    const int bid = xcd_order(blockIdx.x, gridDim.x);
    const int cb = bid % c_blocks, ob = bid / c_blocks;
    const int o0 = ob * kWO, c0 = cb * kWCI;
    const int tid = threadIdx.x, ol = tid % kWO, cl = tid / kWO;
    float acc[K][HW2];
#pragma unroll
    for (int kh = 0; kh < K; ++kh)
#pragma unroll
        for (int q = 0; q < HW2; ++q) acc[kh][q] = 0.0f;
    // chunks of 16 rows of one image, walked image by image; a chunk's loads
    // go to registers one chunk ahead (while the chunk before it is
    // multiplied), then to LDS
    constexpr int NGS = kWR * kWO * HW2, NXS = kWCI * (kWR + K - 1) * HW2;
    constexpr int NG = (NGS + 255) / 256, NX = (NXS + 255) / 256;
    const int row_chunks = (H + kWR - 1) / kWR, nchunks = N * row_chunks;
    float vg[NG], vx[NX];
    auto fetch = [&](int chunk) {
        const int n = chunk / row_chunks, i0 = (chunk - n * row_chunks) * kWR;
#pragma unroll
        for (int k = 0; k < NG; ++k) {
            const int idx = tid + 256 * k;
            const int q = idx % HW2;
            const int o_l = (idx / HW2) % kWO, r = idx / (HW2 * kWO);
            const int o = o0 + o_l, i = i0 + r;
            vg[k] = 0.0f;
            if (idx < NGS && o < CO && i < H)
                vg[k] = gy[(((int64_t)n * CO + o) * H + i) * W + (q < P ? q : W - 2 * P + q)];
        }
#pragma unroll
        for (int k = 0; k < NX; ++k) {
            const int idx = tid + 256 * k;
            const int q = idx % HW2;
            const int rr = (idx / HW2) % (kWR + K - 1), c_l = idx / (HW2 * (kWR + K - 1));
            const int c = c0 + c_l, r = i0 - P + rr;
            vx[k] = 0.0f;
            if (idx < NXS && c < CI && r >= 0 && r < H) vx[k] = xh[(((int64_t)n * CI + c) * H + r) * HW2 + q];
        }
    };
    fetch(0);
    for (int chunk = 0; chunk < nchunks; ++chunk) {
        {
#pragma unroll
            for (int k = 0; k < NG; ++k)
                if (tid + 256 * k < NGS) (&gs[0][0][0])[tid + 256 * k] = vg[k];
#pragma unroll
            for (int k = 0; k < NX; ++k)
                if (tid + 256 * k < NXS) (&xs[0][0][0])[tid + 256 * k] = vx[k];
            __syncthreads();
            if (chunk + 1 < nchunks) fetch(chunk + 1);
            float xw[K][HW2];                             // halo rows r .. r + K - 1
#pragma unroll
            for (int kh = 0; kh < K - 1; ++kh)
#pragma unroll
                for (int q = 0; q < HW2; ++q) xw[kh + 1][q] = xs[cl][kh][q];
#pragma unroll
            for (int r = 0; r < kWR; ++r) {
#pragma unroll
                for (int kh = 0; kh < K - 1; ++kh)
#pragma unroll
                    for (int q = 0; q < HW2; ++q) xw[kh][q] = xw[kh + 1][q];
#pragma unroll
                for (int q = 0; q < HW2; ++q) xw[K - 1][q] = xs[cl][r + K - 1][q];
                float g[HW2];
#pragma unroll
                for (int q = 0; q < HW2; ++q) g[q] = gs[r][ol][q];
#pragma unroll
                for (int kh = 0; kh < K; ++kh) {
#pragma unroll
                    for (int kw = 0; kw < P; ++kw)
#pragma unroll
                        for (int j = 0; j < P - kw; ++j) acc[kh][kw] = fmaf(g[j], xw[kh][j + kw], acc[kh][kw]);
#pragma unroll
                    for (int kw = P + 1; kw < K; ++kw)
#pragma unroll
                        for (int m = 2 * P - kw; m < P; ++m)
                            acc[kh][kw - 1] = fmaf(g[P + m], xw[kh][m + kw - P], acc[kh][kw - 1]);
                }
            }
            __syncthreads();
        }
    }
    const int o = o0 + ol, c = c0 + cl;
    if (o >= CO || c >= CI) return;
#pragma unroll
    for (int kh = 0; kh < K; ++kh)
#pragma unroll
        for (int q = 0; q < HW2; ++q) {
            const int kw = q < P ? q : q + 1;
            gw[(((int64_t)o * CI + c) * K + kh) * K + kw] += acc[kh][q];
        }
}

template <int K, bool FLIP>
void dw_conv_launch(const Geom& g, const float* sh, const float* w, float* out, hipStream_t st)
{
    const int bpp = (g.h + 63) / 64;
    hipLaunchKernelGGL((dw_edge_conv_kernel<K, FLIP>), dim3((unsigned)((int64_t)g.n * g.ci * bpp)), dim3(64), 0,
                       st, sh, w, out, g.ci, g.h, g.wl, bpp);
}

template <int K, bool TRANS>
void dense_conv_launch(const Geom& g, const float* sh, const float* w, float* out, hipStream_t st)
{
    const int O = TRANS ? g.ci : g.co, CR = TRANS ? g.co : g.ci;
    const int row_blocks = (g.h + kDR - 1) / kDR, o_blocks = (O + kDO - 1) / kDO;
    const int64_t blocks = (int64_t)g.n * row_blocks * o_blocks * 2;
    hipLaunchKernelGGL((dense_edge_conv_kernel<K, TRANS>), dim3((unsigned)blocks), dim3(kDT), 0, st, sh, w, out,
                       g.n, O, CR, g.h, g.wl, row_blocks);
}

int grid_for(int64_t work)
{
    int64_t blocks = (work + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 1 << 20) blocks = 1 << 20;
    return (int)blocks;
}

}  // namespace

hipError_t launch_edge_fwd(const Geom& g, const float* xh, const float* w, float* y, hipStream_t st)
{
    if (g.hl + g.hr == 0) return hipSuccess;
    if (dw_edge(g)) {
        switch (g.k) {
            case 3: dw_conv_launch<3, false>(g, xh, w, y, st); break;
            case 5: dw_conv_launch<5, false>(g, xh, w, y, st); break;
            default: dw_conv_launch<7, false>(g, xh, w, y, st); break;
        }
        return hipGetLastError();
    }
    if (dense_edge(g)) {
        if (g.k == 3) dense_conv_launch<3, false>(g, xh, w, y, st);
        else dense_conv_launch<5, false>(g, xh, w, y, st);
        return hipGetLastError();
    }
    const Strips sp = fwd_strips(g);
    const int64_t total = (int64_t)g.n * g.co * g.ho * sp.n();
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(edge_fwd_kernel, dim3(grid_for(total)), dim3(256), 0, st, g, sp, xh, w, y);
    return hipGetLastError();
}

hipError_t launch_edge_bwd_input(const Geom& g, const float* gyh, const float* w, float* gx,
                                 hipStream_t st)
{
    if (g.ghl + g.ghr == 0) return hipSuccess;
    if (dw_edge(g)) {
        switch (g.k) {
            case 3: dw_conv_launch<3, true>(g, gyh, w, gx, st); break;
            case 5: dw_conv_launch<5, true>(g, gyh, w, gx, st); break;
            default: dw_conv_launch<7, true>(g, gyh, w, gx, st); break;
        }
        return hipGetLastError();
    }
    if (dense_edge(g)) {
        if (g.k == 3) dense_conv_launch<3, true>(g, gyh, w, gx, st);
        else dense_conv_launch<5, true>(g, gyh, w, gx, st);
        return hipGetLastError();
    }
    const Strips sp = bwd_input_strips(g);
    const int64_t total = (int64_t)g.n * g.ci * g.h * sp.n();
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(edge_bwd_input_kernel, dim3(grid_for(total)), dim3(256), 0, st, g, sp, gyh, w, gx);
    return hipGetLastError();
}

hipError_t launch_edge_bwd_weight(const Geom& g, const float* xh, const float* gy, float* gw,
                                  hipStream_t st)
{
    if (g.hl + g.hr == 0) return hipSuccess;
    if (dw_edge(g)) {
        switch (g.k) {
#define SSCNN_DW_EW(K)                                                                                     \
    case K:                                                                                                \
        hipLaunchKernelGGL((dw_edge_wgrad_kernel<K>), dim3(g.ci), dim3(256), 0, st, xh, gy, gw, g.n, g.ci, g.h, g.wl); \
        break;
            SSCNN_DW_EW(3)
            SSCNN_DW_EW(5)
            SSCNN_DW_EW(7)
#undef SSCNN_DW_EW
        }
        return hipGetLastError();
    }
    if (dense_edge(g)) {
        const int o_blocks = (g.co + kWO - 1) / kWO, c_blocks = (g.ci + kWCI - 1) / kWCI;
        const dim3 grid((unsigned)(o_blocks * c_blocks));
        if (g.k == 3)
            hipLaunchKernelGGL((dense_edge_wgrad_kernel<3>), grid, dim3(256), 0, st, xh, gy, gw, g.n, g.co, g.ci,
                               g.h, g.wl, c_blocks);
        else
            hipLaunchKernelGGL((dense_edge_wgrad_kernel<5>), grid, dim3(256), 0, st, xh, gy, gw, g.n, g.co, g.ci,
                               g.h, g.wl, c_blocks);
        return hipGetLastError();
    }
    const int64_t total = (int64_t)g.co * g.cig * g.k * g.k;
    hipLaunchKernelGGL(edge_bwd_weight_kernel, dim3(grid_for(total)), dim3(256), 0, st, g, xh, gy, gw);
    return hipGetLastError();
}

}  // namespace sscnn
