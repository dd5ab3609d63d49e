// mfma_wgrad.hip -- _Partial grad_weight / grad_bias of a dense (groups == 1)
// k x k, stride 1, pad k/2 convolution of one W-shard on the FP32 matrix cores
// (NVIDIA blog "Perception Model Training for Autonomous Vehicles with Tensor
// Parallelism", DTensor section: convolution_backward leaves grad_weight and
// grad_bias as partial sums over each shard's own output columns).
//
// For a tap t = (kh, kw):
//     gW[o, c, t] = sum over pixels px = (n, i, j) of G[n, o, i, j] * Xext[n, c, i + kh - P, j + kw]
// a matrix product with the pixels as the reduction.  D = A x B with
// A = G (rows o, k = px) and B = Xext (k = px, columns c); the two k slots of
// the 32x32x2 instruction take pixels p and p + 32 of the same image row, so
// both operands are read along pixels in LDS.
//
//  * workgroup tile: 64 output channels x 64 input channels x the k taps of
//    one kernel row kh; each of the 4 waves owns a 32 x 32 channel block for
//    all k taps of that row (k accumulator blocks);
//  * the pixel reduction is split over image rows (split-K): a workgroup
//    walks its share of rows, staging per row the grad_output row (64 x 128)
//    and the input row i + kh - P with its halo columns (64 x (128 + k - 1))
//    in LDS, the next row prefetched in registers;
//  * each split writes its partial sums to a workspace laid out tap-major
//    ([split][t][o][c], contiguous along c), and a second kernel adds the
//    splits in split order and writes grad_weight in OIHW order;
//  * the workgroups with the first input-channel tile and kh == 0 also sum
//    grad_output over their rows: the grad_bias partials.
// No atomics: results are bitwise reproducible.
#include "internal.h"
#include "mfma_conv.h"

namespace sscnn {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kNT = 256;    // 4 waves
constexpr int kBO = 64;     // output channels per workgroup
constexpr int kBC = 64;     // input channels per workgroup
constexpr int kSW = 128;    // pixels of a row per stage

struct WgArgs {
    const float* x;      // (N, Ci, H, W) input slice
    const float* halo;   // (N, Ci, H + 2 crh, hl + hr); null with hl = hr = 0 when absent
    const float* up;     // input rows above / below the slice (height and 2-D sharding), null when
    const float* down;   //   absent: rh rows per plane each, rplane floats between planes
    int64_t rplane;
    int rh, crh;         // row-halo height; rows of the column halo above row 0
    const float* g;      // (N, Co, H, W) grad_output slice
    float* ws;           // [splits][k*k][Co][Ci] partial grad_weight, then [splits][Co] grad_bias
    int N, Ci, Co, H, W, hl, hr;
    int tiles_o, tiles_c, segs, rows, splits, rows_per_split;
};

template <int K>
struct WShape {
    static constexpr int KK = K * K;
    static constexpr int P = K / 2;
    static constexpr int GS = kSW + 1;                  // grad_output row stride (odd)
    static constexpr int XS = kSW + K - 1 + ((kSW + K - 1) % 2 == 0 ? 1 : 0);   // odd
    static constexpr int G_FLOATS = kBO * GS;
    static constexpr int X_FLOATS = kBC * XS;
    static constexpr int NG = kBO * kSW / 4 / kNT;      // float4 per thread (grad_output)
    static constexpr int NX = kBC * kSW / 4 / kNT;      // float4 per thread (input, own columns)
    static constexpr int NS = (kBC * 2 * P + kNT - 1) / kNT;   // side columns per thread
};

template <int K>
struct WRegs {
    float4 g[WShape<K>::NG];
    float4 x[WShape<K>::NX];
    float s[WShape<K>::NS];
};

// Input row r of plane pl over the slice's own columns: the slice for
// 0 <= r < H, the row halos for the rh rows beyond it; null (zeros) elsewhere.
__device__ __forceinline__ const float* xrow(const WgArgs& a, int64_t pl, int r)
{
    if (r >= 0 && r < a.H) return a.x + (pl * a.H + r) * a.W;
    if (r < 0) return (a.up && r >= -a.rh) ? a.up + pl * a.rplane + (int64_t)(r + a.rh) * a.W : nullptr;
    return (a.down && r < a.H + a.rh) ? a.down + pl * a.rplane + (int64_t)(r - a.H) * a.W : nullptr;
}

// Extended input value at shard column xcol of row r (column halo outside
// the slice, zero beyond it or outside the rows there are data for).
__device__ __forceinline__ float xext(const WgArgs& a, int64_t pl, int r, int xcol)
{
    if (xcol >= 0 && xcol < a.W) {
        const float* p = xrow(a, pl, r);
        return p ? p[xcol] : 0.f;
    }
    if (r < -a.crh || r >= a.H + a.crh) return 0.f;
    const int hw = a.hl + a.hr;
    const float* hp = a.halo + (pl * (a.H + 2 * a.crh) + (r + a.crh)) * hw;
    if (xcol < 0) return xcol >= -a.hl ? hp[a.hl + xcol] : 0.f;
    return xcol < a.W + a.hr ? hp[a.hl + (xcol - a.W)] : 0.f;
}

// Stage s of a split: flattened (image row, column segment).
template <int K>
__device__ __forceinline__ void fetch(WRegs<K>& R, const WgArgs& a, int stage, int kh, int o0, int c0)
{
    using S = WShape<K>;
    constexpr int P = S::P;
    const int tid = threadIdx.x;
    const int seg = stage % a.segs, rowf = stage / a.segs;
    const int n = rowf / a.H, i = rowf - n * a.H;
    const int j0 = seg * kSW;
    const int r = i + kh - P;                      // input row that meets output row i
    // grad_output: thread -> (channel t/32 + 8k, float4 column t%32)
    {
        const int q = tid % 32, cl = tid / 32;
        const int col = j0 + 4 * q;
        const float* gp = a.g + (((int64_t)n * a.Co + o0 + cl) * a.H + i) * a.W + col;
#pragma unroll
        for (int k = 0; k < S::NG; ++k) {
            const int o = o0 + cl + 8 * k;
            R.g[k] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (o < a.Co && col < a.W) R.g[k] = *reinterpret_cast<const float4*>(gp + (int64_t)8 * k * a.H * a.W);
        }
    }
    // input row r, own columns
    {
        const int q = tid % 32, cl = tid / 32;
        const int col = j0 + 4 * q;
#pragma unroll
        for (int k = 0; k < S::NX; ++k) {
            const int c = c0 + cl + 8 * k;
            const int64_t pl = (int64_t)n * a.Ci + c;
            R.x[k] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (c < a.Ci) {
                if (col + 3 < a.W) {
                    const float* rp = xrow(a, pl, r);
                    if (rp) R.x[k] = *reinterpret_cast<const float4*>(rp + col);
                } else {
                    R.x[k].x = xext(a, pl, r, col);
                    R.x[k].y = xext(a, pl, r, col + 1);
                    R.x[k].z = xext(a, pl, r, col + 2);
                    R.x[k].w = xext(a, pl, r, col + 3);
                }
            }
        }
    }
    // P side columns each side of the segment
#pragma unroll
    for (int k = 0; k < S::NS; ++k) {
        const int idx = tid + k * kNT;
        R.s[k] = 0.f;
        if (idx < kBC * 2 * P) {
            const int cl = idx / (2 * P), e = idx - cl * (2 * P);
            const int c = c0 + cl;
            const int xcol = e < P ? j0 - P + e : j0 + kSW + (e - P);
            if (c < a.Ci) R.s[k] = xext(a, (int64_t)n * a.Ci + c, r, xcol);
        }
    }
}

template <int K>
__device__ __forceinline__ void put(const WRegs<K>& R, float* __restrict__ gs, float* __restrict__ xs)
{
    using S = WShape<K>;
    constexpr int P = S::P;
    const int tid = threadIdx.x;
    const int q = tid % 32, cl = tid / 32;
#pragma unroll
    for (int k = 0; k < S::NG; ++k) {
        float* d = gs + (cl + 8 * k) * S::GS + 4 * q;
        d[0] = R.g[k].x; d[1] = R.g[k].y; d[2] = R.g[k].z; d[3] = R.g[k].w;
    }
#pragma unroll
    for (int k = 0; k < S::NX; ++k) {
        float* d = xs + (cl + 8 * k) * S::XS + P + 4 * q;
        d[0] = R.x[k].x; d[1] = R.x[k].y; d[2] = R.x[k].z; d[3] = R.x[k].w;
    }
#pragma unroll
    for (int k = 0; k < S::NS; ++k) {
        const int idx = tid + k * kNT;
        if (idx < kBC * 2 * P) {
            const int c = idx / (2 * P), e = idx - c * (2 * P);
            xs[c * S::XS + (e < P ? e : kSW + e)] = R.s[k];
        }
    }
}

template <int K>
__global__ void __launch_bounds__(kNT, 2)
mfma_wgrad_kernel(WgArgs a)
{
    using S = WShape<K>;
    constexpr int KK = S::KK;
    __shared__ __align__(16) float gs[S::G_FLOATS];
    __shared__ __align__(16) float xs[S::X_FLOATS];

    // workgroup -> (split, kh, input-channel tile, output-channel tile).  When
    // the splits divide evenly over the 8 XCDs (workgroups are dealt to them
    // round-robin), all tiles of a split run on one XCD, so the grad_output and
    // input rows they share stay in one L2.
    int b = blockIdx.x;
    const int per_split = a.tiles_o * a.tiles_c * K;
    if (a.splits % 8 == 0) {
        const int xcd = b % 8, j = b / 8;
        b = (xcd * (a.splits / 8) + j / per_split) * per_split + j % per_split;
    }
    const int ot = b % a.tiles_o;
    b /= a.tiles_o;
    const int ct = b % a.tiles_c;
    b /= a.tiles_c;
    const int kh = b % K;
    const int split = b / K;
    const int o0 = ot * kBO, c0 = ct * kBC;
    const bool do_bias = (ct == 0 && kh == 0);

    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ob = wave >> 1, cb = wave & 1;
    const int lhalf = lane >> 5, l32 = lane & 31;

    f32x16 acc[K];
#pragma unroll
    for (int kw = 0; kw < K; ++kw)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[kw][r] = 0.f;
    float bsum = 0.f;

    const int s_begin = split * a.rows_per_split * a.segs;
    const int s_end = min(a.rows, (split + 1) * a.rows_per_split) * a.segs;
    WRegs<K> R;
    if (s_begin < s_end) fetch<K>(R, a, s_begin, kh, o0, c0);
    const float* ga = gs + (ob * 32 + l32) * S::GS + 32 * lhalf;
    const float* xb = xs + (cb * 32 + l32) * S::XS + 32 * lhalf;
    for (int st = s_begin; st < s_end; ++st) {
        if (st > s_begin) lds_barrier();
        put<K>(R, gs, xs);
        lds_barrier();
        if (st + 1 < s_end) fetch<K>(R, a, st + 1, kh, o0, c0);
        if (do_bias) {
            // thread -> output channel tid/4, pixels (tid%4)*32 .. +32 of the row
            const float* p = gs + (threadIdx.x >> 2) * S::GS + (threadIdx.x & 3) * 32;
#pragma unroll 8
            for (int m = 0; m < 32; ++m) bsum += p[m];
        }
#pragma unroll 1
        for (int half = 0; half < 2; ++half)
#pragma unroll 4
            for (int p = 0; p < 32; ++p) {
                const int px = half * 64 + p;
                const float av = ga[px];
#pragma unroll
                for (int kw = 0; kw < K; ++kw)
                    acc[kw] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, xb[px + kw], acc[kw], 0, 0, 0);
            }
    }

    // D[o][c]: register r -> output channel 8(r/4) + 4*lhalf + r%4 of the block,
    // lane%32 -> input channel.  Workspace [split][t][o][c].
    const int c = c0 + cb * 32 + l32;
    if (c < a.Ci) {
#pragma unroll
        for (int kw = 0; kw < K; ++kw) {
            float* wsp = a.ws + ((int64_t)split * KK + kh * K + kw) * a.Co * a.Ci;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int o = o0 + ob * 32 + 8 * (r / 4) + 4 * lhalf + (r % 4);
                if (o < a.Co) wsp[(int64_t)o * a.Ci + c] = acc[kw][r];
            }
        }
    }
    if (do_bias) {
        // combine the 4 threads of a channel as (t0 + t1) + (t2 + t3)
        bsum += __shfl_xor(bsum, 1);
        bsum += __shfl_xor(bsum, 2);
        const int o = o0 + (threadIdx.x >> 2);
        if ((threadIdx.x & 3) == 0 && o < a.Co)
            a.ws[(int64_t)a.splits * KK * a.Co * a.Ci + (int64_t)split * a.Co + o] = bsum;
    }
}

// grad_w[o, c, t] = sum over splits (in order) of ws[s][t][o][c]; one thread
// per workspace position so the reads are contiguous; grad_b likewise.
template <int K>
__global__ void __launch_bounds__(256)
mfma_wgrad_reduce_kernel(const float* __restrict__ ws, int splits, int Co, int Ci,
                         float* __restrict__ gw, float* __restrict__ gb)
{
    constexpr int KK = K * K;
    const int64_t plane = (int64_t)Co * Ci;
    const int64_t total = plane * KK;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx < total) {
        float s = ws[idx];
        for (int k = 1; k < splits; ++k) s += ws[(int64_t)k * total + idx];
        const int t = (int)(idx / plane);
        const int64_t oc = idx - t * plane;
        gw[oc * KK + t] = s;
    } else if (gb && idx < total + Co) {
        const int o = (int)(idx - total);
        const float* p = ws + (int64_t)splits * total;
        float s = p[o];
        for (int k = 1; k < splits; ++k) s += p[(int64_t)k * Co + o];
        gb[o] = s;
    }
}

struct Plan {
    int tiles_o, tiles_c, segs, rows, splits, rows_per_split;
};

Plan plan(const Geom& g)
{
    Plan p;
    p.tiles_o = (g.co + kBO - 1) / kBO;
    p.tiles_c = (g.ci + kBC - 1) / kBC;
    p.segs = (g.wl + kSW - 1) / kSW;
    p.rows = g.n * g.h;
    // about 2560 workgroups (5 waves of 2 per CU on 256 CUs), at most one row each
    const int tiles = p.tiles_o * p.tiles_c * g.k;
    int splits = (2560 + tiles - 1) / tiles;
    if (splits > p.rows) splits = p.rows;
    if (splits < 1) splits = 1;
    p.rows_per_split = (p.rows + splits - 1) / splits;
    p.splits = (p.rows + p.rows_per_split - 1) / p.rows_per_split;
    return p;
}

template <int K>
hipError_t launch(const Geom& g, const float* x, const float* xh, const RowHalo& rows, const float* gy,
                  float* gw, float* gb, float* ws, hipStream_t st)
{
    const Plan p = plan(g);
    WgArgs a{};
    a.x = x; a.halo = xh; a.g = gy; a.ws = ws;
    a.up = rows.up; a.down = rows.down; a.rplane = rows.rplane; a.rh = rows.rh; a.crh = xh ? rows.crh : 0;
    a.N = g.n; a.Ci = g.ci; a.Co = g.co; a.H = g.h; a.W = g.wl;
    a.hl = xh ? g.hl : 0; a.hr = xh ? g.hr : 0;     // no halo: xext() reads zeros beyond the slice
    a.tiles_o = p.tiles_o; a.tiles_c = p.tiles_c; a.segs = p.segs; a.rows = p.rows;
    a.splits = p.splits; a.rows_per_split = p.rows_per_split;
    const int64_t grid = (int64_t)p.splits * K * p.tiles_c * p.tiles_o;
    hipLaunchKernelGGL((mfma_wgrad_kernel<K>), dim3((unsigned)grid), dim3(kNT), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t total = (int64_t)g.co * g.ci * K * K + g.co;
    hipLaunchKernelGGL((mfma_wgrad_reduce_kernel<K>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       st, ws, p.splits, g.co, g.ci, gw, gb);
    return hipGetLastError();
}

}  // namespace

size_t mfma_wgrad_workspace_bytes(const Geom& g)
{
    const Plan p = plan(g);
    return ((size_t)p.splits * g.k * g.k * g.co * g.ci + (size_t)p.splits * g.co) * sizeof(float);
}

hipError_t launch_mfma_bwd_weight(const Geom& g, const float* x, const float* xh, const float* gy,
                                  float* gw, float* gb, void* ws, hipStream_t st)
{
    return launch_mfma_bwd_weight_rows(g, x, xh, RowHalo{}, gy, gw, gb, ws, st);
}

hipError_t launch_mfma_bwd_weight_rows(const Geom& g, const float* x, const float* xh, const RowHalo& rows,
                                       const float* gy, float* gw, float* gb, void* ws, hipStream_t st)
{
    float* w = static_cast<float*>(ws);
    return g.k == 3 ? launch<3>(g, x, xh, rows, gy, gw, gb, w, st) : launch<5>(g, x, xh, rows, gy, gw, gb, w, st);
}

}  // namespace sscnn
