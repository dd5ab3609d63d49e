// depthwise.hip -- depthwise (groups == C) k x k, stride 1, pad k/2 convolution
// of one W-shard, the ConvNeXt block convolution run through the sharded path
// (kwkr.cn retelling, section 3.2: the same halo-exchange convolution is used
// for ConvNeXt-XL's depthwise layers).
//
// Work per output: k*k multiply-adds on one channel plane, ~14 FLOP per byte
// of compulsory traffic: below the FP32 ridge of the chip, so these are
// bandwidth kernels.  Their job is to keep HBM busy while the FMAs run:
//
//  * persistent workgroups (as many as fit on the chip) walk a list of output
//    tiles (TH rows x TW columns of one (n, c) plane).  Each tile's input --
//    the shard's own columns with 16-byte loads, k/2 side columns from the halo
//    buffer at the shard's edges (or from the slice itself inside the shard),
//    zero rows above and below the image -- is fetched into registers one tile
//    AHEAD, so the HBM reads of tile t+1 are in flight while tile t computes;
//    the registers are then written to an LDS tile;
//  * each thread owns RH rows x 4 columns of outputs, slides down its RH+k-1
//    input rows reading 4+k-1 values per row from LDS (16-byte reads), and
//    issues k*k*4*RH fused multiply-adds whose weight operand is a scalar
//    register (the plane's k*k weights are wave-uniform);
//  * grad_input is the same kernel on the grad_output tile with the kernel
//    flipped in both axes (stride 1, pad k/2, so the grad_output halo has the
//    same widths as the input halo);
//  * grad_weight: each thread accumulates all k*k taps over its RH x 4 outputs
//    (its grad_output block is prefetched alongside the input tile) and keeps
//    them across the consecutive tiles of one channel that its workgroup
//    owns; at a channel change the waves reduce them with cross-lane swaps,
//    the workgroup adds the waves' totals in a fixed order and writes one
//    partial; a second kernel sums a channel's partials in workgroup order.
//    No atomics: results are bitwise reproducible.
#include "internal.h"
#include "depthwise.h"

#ifndef SSCNN_DW_WGRAD_WAVES
#define SSCNN_DW_WGRAD_WAVES 3
#endif

namespace sscnn {
namespace {

struct DwArgs {
    const float* x;      // (N*C, H, W) shard slice (input, or grad_output for grad_input)
    const float* halo;   // (N*C, H, 2P)
    const float* w;      // (C, k, k)
    const float* b;      // (C) or null
    float* y;            // (N*C, H, W)
    const float* g;      // grad_output (N*C, H, W) for grad_weight
    float* ws;           // grad_weight partials (C, up to N * tiles_h * tiles_w, k*k + 1)
    int H, W, C, N, tiles_h, tiles_w, ntiles;   // ntiles = N * C * tiles_h * tiles_w
};

// Tile t -> (plane, tile row, tile column), column fastest.
struct TileIdx {
    int plane, c, n, trow, tcol, i0, j0;
};

// With clamp, the last row tile is moved up to end at row H (it then
// recomputes some rows of the previous tile, bit-identically), so every row a
// forward tile computes is a real row and its stores need no predicate.
__device__ __forceinline__ TileIdx decode(const DwArgs& a, int t, int th, int tw, bool clamp)
{
    TileIdx d;
    d.tcol = t % a.tiles_w;
    t /= a.tiles_w;
    d.trow = t % a.tiles_h;
    d.plane = t / a.tiles_h;
    d.c = d.plane % a.C;
    d.n = d.plane / a.C;
    d.i0 = d.trow * th;
    if (clamp && d.i0 + th > a.H) d.i0 = a.H - th;
    d.j0 = d.tcol * tw;
    return d;
}

// Input tile.  LDS column cc holds extended column j0 + cc, i.e. shard
// column j0 + cc - P; tile row rr holds image row i0 - P + rr.  A thread's
// 4 + k - 1 inputs per row start at a 16-byte boundary, so they are read with
// 16-byte LDS reads (the fill pays unaligned 4-byte writes instead, once per
// element, against ~2.5 reads per element).
// LDS row pitch (floats): a multiple of 4 (16-byte aligned rows) such that
// the TX lanes of a wave that read one tile row and the next TX lanes, RH
// rows further down, sit a multiple of 4*TX floats apart.  gfx950 serves
// 16-byte LDS reads of such lane groups at full rate (~240 B/clk per CU,
// measured) and at half rate for other pitches.
constexpr int lds_pitch(int lw, int rh, int tx)
{
    int ls = (lw + 3) & ~3;
    while ((rh * ls) % (4 * tx) != 0) ls += 4;
    return ls;
}

template <int K, int TX, int TY, int RH>
struct Tile {
    static constexpr int P = K / 2;
    static constexpr int NT = TX * TY;
    static constexpr int TW = 4 * TX;
    static constexpr int TH = RH * TY;
    static constexpr int LW = TW + K - 1;
    static constexpr int LS = lds_pitch(LW, RH, TX);
    static constexpr int LH = TH + K - 1;
    static constexpr int FLOATS = LH * LS;
    static constexpr int Q = TW / 4;
    static constexpr int NV = (LH * Q + NT - 1) / NT;          // 16-byte loads per thread
    static constexpr int NS = (LH * 2 * P + NT - 1) / NT;      // side-column loads per thread

    struct Regs {
        float4 v[NV];
        float s[NS];
    };

    // Global -> registers (all loads issued back to back).
    __device__ static void fetch(Regs& R, const float* __restrict__ xp, const float* __restrict__ hp,
                                 int H, int W, int i0, int j0)
    {
        const int tid = threadIdx.x;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int idx = tid + k * NT;
            const int rr = idx / Q, q = idx - rr * Q;
            const int r = i0 - P + rr;
            R.v[k] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (idx < LH * Q && r >= 0 && r < H)
                R.v[k] = *reinterpret_cast<const float4*>(xp + (int64_t)r * W + j0 + 4 * q);
        }
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            const int idx = tid + k * NT;
            const int rr = idx / (2 * P), e = idx - rr * (2 * P);
            const int r = i0 - P + rr;
            const int xcol = j0 + (e < P ? e : TW + e) - P;     // shard column, may be < 0 or >= W
            R.s[k] = 0.f;
            if (idx < LH * 2 * P && r >= 0 && r < H) {
                if (xcol < 0) R.s[k] = hp[(int64_t)r * (2 * P) + (xcol + P)];
                else if (xcol >= W) R.s[k] = hp[(int64_t)r * (2 * P) + P + (xcol - W)];
                else R.s[k] = xp[(int64_t)r * W + xcol];
            }
        }
    }

    // Registers -> LDS tile.
    __device__ static void put(float* __restrict__ tile, const Regs& R)
    {
        const int tid = threadIdx.x;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int idx = tid + k * NT;
            if (idx < LH * Q) {
                const int rr = idx / Q, q = idx - rr * Q;
                float* d = tile + rr * LS + P + 4 * q;
                d[0] = R.v[k].x;
                d[1] = R.v[k].y;
                d[2] = R.v[k].z;
                d[3] = R.v[k].w;
            }
        }
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            const int idx = tid + k * NT;
            if (idx < LH * 2 * P) {
                const int rr = idx / (2 * P), e = idx - rr * (2 * P);
                tile[rr * LS + (e < P ? e : TW + e)] = R.s[k];
            }
        }
    }

    // 4 + K - 1 consecutive tile values starting at a 16-byte aligned column.
    __device__ static void read_row(const float* __restrict__ src, float (&in)[4 + K - 1])
    {
        const float4 a = *reinterpret_cast<const float4*>(src);
        in[0] = a.x; in[1] = a.y; in[2] = a.z; in[3] = a.w;
        if constexpr (K - 1 >= 4) {
            const float4 c = *reinterpret_cast<const float4*>(src + 4);
            in[4] = c.x; in[5] = c.y; in[6] = c.z; in[7] = c.w;
            if constexpr (K - 1 == 6) {
                const float2 d = *reinterpret_cast<const float2*>(src + 8);
                in[8] = d.x; in[9] = d.y;
            }
        } else {
            const float2 d = *reinterpret_cast<const float2*>(src + 4);
            in[4] = d.x; in[5] = d.y;
        }
    }
};

template <int K, int TX, int TY, int RH, bool FLIP>
__global__ void __launch_bounds__(TX * TY) __attribute__((amdgpu_waves_per_eu(3)))
dw_conv_kernel(DwArgs a)
{
    using T = Tile<K, TX, TY, RH>;
    constexpr int P = T::P;
    __shared__ __align__(16) float tile[T::FLOATS];
    typename T::Regs R;
    int t = blockIdx.x;
    if (t >= a.ntiles) return;
    {
        const TileIdx d = decode(a, t, T::TH, T::TW, true);
        T::fetch(R, a.x + (int64_t)d.plane * a.H * a.W, a.halo + (int64_t)d.plane * a.H * (2 * P),
                 a.H, a.W, d.i0, d.j0);
    }
    const int tx = threadIdx.x % TX, ty = threadIdx.x / TX;
    for (; t < a.ntiles; t += gridDim.x) {
        const TileIdx d = decode(a, t, T::TH, T::TW, true);
        T::put(tile, R);
        lds_barrier();
        const int tn = t + gridDim.x;
        if (tn < a.ntiles) {
            const TileIdx e = decode(a, tn, T::TH, T::TW, true);
            T::fetch(R, a.x + (int64_t)e.plane * a.H * a.W, a.halo + (int64_t)e.plane * a.H * (2 * P),
                     a.H, a.W, e.i0, e.j0);
        }
        // the plane's weights: wave-uniform, kept in scalar registers
        // The plane's weights are wave-uniform: loaded through the scalar
        // cache, then copied to vector registers, because gfx950 issues
        // v_fmac_f32 at about twice the rate when no operand is a scalar
        // register (measured: ~119 vs ~70 TFLOP/s chip-wide).
        float wr[K * K];
        const auto wp = as_const(a.w) + d.c * K * K;
#pragma unroll
        for (int k = 0; k < K * K; ++k) wr[k] = to_vgpr(wp[FLIP ? K * K - 1 - k : k]);
        const float bias = a.b ? as_const(a.b)[d.c] : 0.f;

        float acc[RH][4];
#pragma unroll
        for (int i = 0; i < RH; ++i)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) acc[i][jj] = bias;
        // Each row is read from LDS one row ahead of its FMAs (a whole row of
        // FMAs covers the read latency); the scheduling barriers keep that
        // order, which the compiler would otherwise tighten to a few FMAs.
        const float* base = tile + (ty * RH) * T::LS + 4 * tx;
        float cur[4 + K - 1], nxt[4 + K - 1];
        T::read_row(base, cur);
#pragma unroll
        for (int r = 0; r < RH + K - 1; ++r) {
            if (r + 1 < RH + K - 1) T::read_row(base + (r + 1) * T::LS, nxt);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < RH; ++i) {
                const int kh = r - i;
                if (kh < 0 || kh >= K) continue;
#pragma unroll
                for (int kw = 0; kw < K; ++kw)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        acc[i][jj] = __builtin_fmaf(wr[kh * K + kw], cur[jj + kw], acc[i][jj]);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = 0; q < 4 + K - 1; ++q) cur[q] = nxt[q];
        }
        float* yp = a.y + (int64_t)d.plane * a.H * a.W + d.j0 + 4 * tx;
#pragma unroll
        for (int i = 0; i < RH; ++i)
            *reinterpret_cast<float4*>(yp + (int64_t)(d.i0 + ty * RH + i) * a.W) =
                make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
        lds_barrier();   // the tile is rewritten by the next iteration's put()
    }
}

// Sum of N per-lane values over the 64 lanes of a wave, leaving one total per
// lane (a reduce-scatter): stage k pairs lanes that differ in one lane bit
// (32, 16, 8, 4, 2, 1) and halves the list, the lower lane of a pair keeping
// the first half of the list and the upper lane the second half.  Bits 5 and
// 4 are exchanged with the gfx950 lane-swap instructions, bits 3..0 with DPP
// (row mirror, half-row mirror, quad permutations; the pairings they make
// split the lanes by the same bits).  wave_sum_index() names the value a lane
// ends with.  Cost ~2.6 VALU per value instead of a 64-step loop per value.
__device__ __forceinline__ float lane_swap_sum(float x, float y, bool bit16)
{
    const auto r = bit16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false)
                         : __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int CTRL>
__device__ __forceinline__ float dpp_pair_sum(float x, float y, bool upper)
{
    const float send = upper ? x : y;
    const float keep = upper ? y : x;
    return keep + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(send), CTRL, 0xf, 0xf, false));
}

template <int N, int STAGE>
__device__ __forceinline__ float wave_sum_stage(const float (&v)[N], int lane)
{
    constexpr int H = (N + 1) / 2;
    float u[H];
#pragma unroll
    for (int i = 0; i < H; ++i) {
        const float x = v[i], y = (i + H < N) ? v[i + H] : 0.f;
        if constexpr (STAGE == 0) u[i] = lane_swap_sum(x, y, false);
        else if constexpr (STAGE == 1) u[i] = lane_swap_sum(x, y, true);
        else if constexpr (STAGE == 2) u[i] = dpp_pair_sum<0x140>(x, y, lane & 8);   // row mirror
        else if constexpr (STAGE == 3) u[i] = dpp_pair_sum<0x141>(x, y, lane & 4);   // half-row mirror
        else if constexpr (STAGE == 4) u[i] = dpp_pair_sum<0x4E>(x, y, lane & 2);    // quad [2,3,0,1]
        else u[i] = dpp_pair_sum<0xB1>(x, y, lane & 1);                               // quad [1,0,3,2]
    }
    if constexpr (STAGE == 5) {
        static_assert(H == 1, "64 lanes reduce at most 64 values");
        return u[0];
    } else {
        return wave_sum_stage<H, STAGE + 1>(u, lane);
    }
}

template <int N>
__device__ __forceinline__ float wave_sum_scatter(const float (&v)[N], int lane)
{
    static_assert(N >= 2 && N <= 64, "values per lane");
    return wave_sum_stage<N, 0>(v, lane);
}

// Index of the total that lane holds after wave_sum_scatter<N>, or -1.
template <int N>
__device__ __forceinline__ int wave_sum_index(int lane)
{
    int n[7];
    n[0] = N;
#pragma unroll
    for (int k = 0; k < 6; ++k) n[k + 1] = (n[k] + 1) / 2;
    const int bit[6] = {32, 16, 8, 4, 2, 1};
    int j = 0;
#pragma unroll
    for (int k = 5; k >= 0; --k) {
        if (lane & bit[k]) j += n[k + 1];
        if (j >= n[k]) return -1;
    }
    return j;
}

// grad_weight partial, tile by tile: the sum over a tile's outputs (i, j) of
// G[i, j] * Xext[i - P + kh, j + kw] for every tap, plus sum G (grad_bias).
// Tiles are numbered channel-major (c, n, tile row, tile column) and each
// workgroup takes one contiguous run of them, so consecutive tiles usually
// share a channel: a thread keeps its k*k + 1 sums in registers across them
// and the workgroup reduces only when the channel changes or its run ends.
// One reduction writes one partial; the partials of channel c are numbered by
// workgroup from the one that owns the channel's first tile.
__device__ __forceinline__ int64_t tile_owner(int64_t t, int64_t T, int64_t G)
{
    return ((t + 1) * G - 1) / T;     // the workgroup w with floor(wT/G) <= t < floor((w+1)T/G)
}

template <int K, int TX, int TY, int RH>
__global__ void __launch_bounds__(TX * TY) __attribute__((amdgpu_waves_per_eu(SSCNN_DW_WGRAD_WAVES)))
dw_wgrad_kernel(DwArgs a)
{
    using T = Tile<K, TX, TY, RH>;
    constexpr int P = T::P;
    constexpr int KK = K * K;
    constexpr int NV = KK + 1;                  // taps + bias
    constexpr int NWAVE = T::NT / 64;
    static_assert(T::NT % 64 == 0, "whole waves");
    __shared__ __align__(16) float sh[T::FLOATS];
    __shared__ float red[NWAVE][NV + 2];
    typename T::Regs R;
    float4 gnext[RH];
    const int tx = threadIdx.x % TX, ty = threadIdx.x / TX;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tiles_c = a.ntiles / a.C;         // N * tiles_h * tiles_w
    const int64_t G = gridDim.x;
    const int beg = (int)((int64_t)blockIdx.x * a.ntiles / G);
    const int end = (int)((int64_t)(blockIdx.x + 1) * a.ntiles / G);
    if (beg >= end) return;

    auto decode_cm = [&](int t) {
        TileIdx d;
        d.tcol = t % a.tiles_w;
        t /= a.tiles_w;
        d.trow = t % a.tiles_h;
        t /= a.tiles_h;
        d.n = t % a.N;
        d.c = t / a.N;
        d.plane = d.n * a.C + d.c;
        d.i0 = d.trow * T::TH;
        d.j0 = d.tcol * T::TW;
        return d;
    };
    auto fetch_all = [&](const TileIdx& d) {
        T::fetch(R, a.x + (int64_t)d.plane * a.H * a.W, a.halo + (int64_t)d.plane * a.H * (2 * P),
                 a.H, a.W, d.i0, d.j0);
        const float* gp = a.g + (int64_t)d.plane * a.H * a.W + d.j0 + 4 * tx;
#pragma unroll
        for (int i = 0; i < RH; ++i) {
            const int row = d.i0 + ty * RH + i;
            gnext[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (row < a.H) gnext[i] = *reinterpret_cast<const float4*>(gp + (int64_t)row * a.W);
        }
    };

    fetch_all(decode_cm(beg));
    for (int t = beg; t < end;) {
        // one run: the workgroup's consecutive tiles of channel c
        const int c = t / tiles_c;
        const int run_end = min(end, (c + 1) * tiles_c);
        float acc[NV];
#pragma unroll
        for (int k = 0; k < NV; ++k) acc[k] = 0.f;
        for (; t < run_end; ++t) {
            T::put(sh, R);
            float gv[RH][4];
#pragma unroll
            for (int i = 0; i < RH; ++i) {
                gv[i][0] = gnext[i].x; gv[i][1] = gnext[i].y; gv[i][2] = gnext[i].z; gv[i][3] = gnext[i].w;
                acc[KK] += (gv[i][0] + gv[i][1]) + (gv[i][2] + gv[i][3]);
            }
            lds_barrier();
            if (t + 1 < end) fetch_all(decode_cm(t + 1));
            // Rows are read one ahead of the FMAs that use them; the
            // scheduling barriers keep the compiler from hoisting every row's
            // reads to the top, which would need ~100 more registers.
            const float* base = sh + (ty * RH) * T::LS + 4 * tx;
            float cur[4 + K - 1], nxt[4 + K - 1];
            T::read_row(base, cur);
#pragma unroll
            for (int r = 0; r < RH + K - 1; ++r) {
                if (r + 1 < RH + K - 1) T::read_row(base + (r + 1) * T::LS, nxt);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < RH; ++i) {
                    const int kh = r - i;
                    if (kh < 0 || kh >= K) continue;
#pragma unroll
                    for (int kw = 0; kw < K; ++kw)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj)
                            acc[kh * K + kw] = __builtin_fmaf(gv[i][jj], cur[jj + kw], acc[kh * K + kw]);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int q = 0; q < 4 + K - 1; ++q) cur[q] = nxt[q];
            }
            lds_barrier();   // the tile is rewritten by the next put()
        }
        // Flush the run: wave totals, then the waves in a fixed order.  red
        // is rewritten only after the next tile's barrier, which every reader
        // below has passed.
        const float s = wave_sum_scatter<NV>(acc, lane);
        const int idx = wave_sum_index<NV>(lane);
        if (idx >= 0) red[wave][idx] = s;
        lds_barrier();
        if (threadIdx.x < NV) {
            float tot = red[0][threadIdx.x];
#pragma unroll
            for (int w = 1; w < NWAVE; ++w) tot += red[w][threadIdx.x];
            const int64_t slot = blockIdx.x - tile_owner((int64_t)c * tiles_c, a.ntiles, G);
            a.ws[((int64_t)c * tiles_c + slot) * NV + threadIdx.x] = tot;
        }
    }
}

// Second pass: grad_w[c, tap] = sum of channel c's partials in workgroup
// order (one per workgroup whose run of tiles meets the channel).
template <int K>
__global__ void __launch_bounds__(256)
dw_wgrad_reduce_kernel(const float* __restrict__ ws, int C, int tiles_c, int64_t ntiles, int64_t grid,
                       float* __restrict__ gw, float* __restrict__ gb)
{
    constexpr int NV = K * K + 1;
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= C * NV) return;
    const int c = idx / NV, t = idx - c * NV;
    const int64_t w0 = tile_owner((int64_t)c * tiles_c, ntiles, grid);
    const int64_t w1 = tile_owner((int64_t)(c + 1) * tiles_c - 1, ntiles, grid);
    const float* p = ws + (int64_t)c * tiles_c * NV + t;
    float s = 0.f;
    for (int64_t k = 0; k <= w1 - w0; ++k) s += p[k * NV];
    if (t < K * K) gw[c * K * K + t] = s;
    else if (gb) gb[c] = s;
}

// Tile shape for a plane of H x W (W a multiple of 16).
struct DwShape {
    int tx, ty, rh;
};

// The tile height TY * RH never exceeds H (the forward's last tile is moved up
// to end at H, see decode()); shapes that do not fit report rh == 0.
DwShape pick_shape(int H, int W)
{
    if (W % 64 == 0) return {16, 16, H >= 64 ? 4 : (H >= 32 ? 2 : (H >= 16 ? 1 : 0))};
    if (W % 32 == 0) return {8, 32, H >= 64 ? 2 : (H >= 32 ? 1 : 0)};
    return {4, 64, H >= 64 ? 1 : 0};
}

// Persistent grid: as many workgroups as are resident at once, at most one per tile.
template <typename Kern>
int persistent_grid(Kern kern, int block, int ntiles)
{
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return ntiles;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return ntiles;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, block, 0) != hipSuccess || per_cu < 1)
        per_cu = 1;
    const int64_t g = (int64_t)cus * per_cu;
    return (int)(g < ntiles ? g : ntiles);
}

template <int K, bool FLIP>
hipError_t launch_conv(DwArgs a, int planes, DwShape sh, hipStream_t st)
{
#define SSCNN_DW_CONV(TX, TY, RH)                                                         \
    if (sh.tx == TX && sh.ty == TY && sh.rh == RH) {                                      \
        auto kern = dw_conv_kernel<K, TX, TY, RH, FLIP>;                                  \
        a.tiles_w = a.W / (4 * TX);                                                       \
        a.tiles_h = (a.H + RH * TY - 1) / (RH * TY);                                      \
        a.ntiles = planes * a.tiles_h * a.tiles_w;                                        \
        const int grid = persistent_grid(kern, TX * TY, a.ntiles);                        \
        hipLaunchKernelGGL(kern, dim3(grid), dim3(TX * TY), 0, st, a);                    \
        return hipGetLastError();                                                         \
    }
    SSCNN_DW_CONV(16, 16, 4)
    SSCNN_DW_CONV(16, 16, 2)
    SSCNN_DW_CONV(16, 16, 1)
    SSCNN_DW_CONV(8, 32, 2)
    SSCNN_DW_CONV(8, 32, 1)
    SSCNN_DW_CONV(4, 64, 1)
#undef SSCNN_DW_CONV
    return hipErrorInvalidValue;
}

template <int K>
hipError_t launch_wgrad(DwArgs a, int planes, DwShape sh, float* gw, float* gb, hipStream_t st)
{
#define SSCNN_DW_WGRAD(TX, TY, RH)                                                          \
    if (sh.tx == TX && sh.ty == TY && sh.rh == RH) {                                        \
        auto kern = dw_wgrad_kernel<K, TX, TY, RH>;                                         \
        a.tiles_w = a.W / (4 * TX);                                                         \
        a.tiles_h = (a.H + RH * TY - 1) / (RH * TY);                                        \
        a.ntiles = planes * a.tiles_h * a.tiles_w;                                          \
        const int grid = persistent_grid(kern, TX * TY, a.ntiles);                          \
        hipLaunchKernelGGL(kern, dim3(grid), dim3(TX * TY), 0, st, a);                      \
        hipError_t e = hipGetLastError();                                                   \
        if (e != hipSuccess) return e;                                                      \
        const int tiles_c = a.ntiles / a.C;                                                 \
        const int total = a.C * (K * K + 1);                                                \
        hipLaunchKernelGGL((dw_wgrad_reduce_kernel<K>), dim3((total + 255) / 256), dim3(256), \
                           0, st, a.ws, a.C, tiles_c, (int64_t)a.ntiles, (int64_t)grid, gw, gb); \
        return hipGetLastError();                                                           \
    }
    SSCNN_DW_WGRAD(16, 16, 4)
    SSCNN_DW_WGRAD(16, 16, 2)
    SSCNN_DW_WGRAD(16, 16, 1)
    SSCNN_DW_WGRAD(8, 32, 2)
    SSCNN_DW_WGRAD(8, 32, 1)
    SSCNN_DW_WGRAD(4, 64, 1)
#undef SSCNN_DW_WGRAD
    return hipErrorInvalidValue;
}

DwArgs make_args(const Geom& g)
{
    DwArgs a{};
    a.H = g.h;
    a.W = g.wl;
    a.C = g.ci;
    a.N = g.n;
    return a;
}

}  // namespace

bool dw_supported(const Geom& g)
{
    return g.groups == g.ci && g.ci == g.co && g.stride == 1 && (g.k == 3 || g.k == 5 || g.k == 7) &&
           g.pad == g.k / 2 && g.wl % 16 == 0 && g.hl == g.pad && g.hr == g.pad &&
           pick_shape(g.h, g.wl).rh > 0 && (int64_t)g.n * g.ci * g.h * g.wl < ((int64_t)1 << 31);
}

size_t dw_wgrad_workspace_bytes(const Geom& g)
{
    const DwShape sh = pick_shape(g.h, g.wl);
    const int64_t tiles = (int64_t)g.n * ((g.h + sh.rh * sh.ty - 1) / (sh.rh * sh.ty)) * (g.wl / (4 * sh.tx));
    return (size_t)(tiles * g.ci * (g.k * g.k + 1)) * sizeof(float);
}

hipError_t launch_dw_fwd(const Geom& g, const float* x, const float* xh, const float* w,
                         const float* b, float* y, hipStream_t st)
{
    DwArgs a = make_args(g);
    a.x = x; a.halo = xh; a.w = w; a.b = b; a.y = y;
    const int planes = g.n * g.ci;
    const DwShape sh = pick_shape(g.h, g.wl);
    switch (g.k) {
        case 3: return launch_conv<3, false>(a, planes, sh, st);
        case 5: return launch_conv<5, false>(a, planes, sh, st);
        default: return launch_conv<7, false>(a, planes, sh, st);
    }
}

hipError_t launch_dw_bwd_input(const Geom& g, const float* gy, const float* gyh, const float* w,
                               float* gx, hipStream_t st)
{
    DwArgs a = make_args(g);
    a.x = gy; a.halo = gyh; a.w = w; a.b = nullptr; a.y = gx;
    const int planes = g.n * g.ci;
    const DwShape sh = pick_shape(g.h, g.wl);
    switch (g.k) {
        case 3: return launch_conv<3, true>(a, planes, sh, st);
        case 5: return launch_conv<5, true>(a, planes, sh, st);
        default: return launch_conv<7, true>(a, planes, sh, st);
    }
}

hipError_t launch_dw_bwd_weight(const Geom& g, const float* x, const float* xh, const float* gy,
                                float* gw, float* gb, void* ws, hipStream_t st)
{
    DwArgs a = make_args(g);
    a.x = x; a.halo = xh; a.g = gy; a.ws = static_cast<float*>(ws);
    const int planes = g.n * g.ci;
    const DwShape sh = pick_shape(g.h, g.wl);
    switch (g.k) {
        case 3: return launch_wgrad<3>(a, planes, sh, gw, gb, st);
        case 5: return launch_wgrad<5>(a, planes, sh, gw, gb, st);
        default: return launch_wgrad<7>(a, planes, sh, gw, gb, st);
    }
}

}  // namespace sscnn
