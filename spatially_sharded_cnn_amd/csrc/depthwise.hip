// depthwise.hip -- depthwise (groups == C) k x k, stride 1, pad k/2 convolution
// of one W-shard, the ConvNeXt block convolution run through the sharded path
// (kwkr.cn retelling, section 3.2: the same halo-exchange convolution is used
// for ConvNeXt-XL's depthwise layers).
//
// Work per output: k*k multiply-adds on one channel plane, ~14 FLOP per byte
// of compulsory traffic: below the FP32 ridge of the chip, so these are
// bandwidth kernels.  Their job is to keep HBM busy while the FMAs run:
//
//  * persistent workgroups walk a list of output tiles (TH rows x TW columns
//    of one (n, c) plane).  A tile's extended input lives in LDS as a main
//    region -- the shard's own TW columns of rows i0-P .. i0+TH+P-1, brought
//    in by buffer loads that write LDS directly (no registers; rows above and
//    below the plane fall outside the buffer and read as zeros) -- and a side
//    region with the P columns on either side (from the halo buffer at the
//    shard's edges, from the slice itself inside it).  Each workgroup has two
//    tile buffers: the loads of its next tile run while it computes the
//    current one, with one barrier per tile; a tile's results are stored
//    after the next tile's barrier;
//  * each thread owns RH rows x 4 columns of outputs, slides down its RH+k-1
//    input rows reading 4+k-1 values per row from LDS (16-byte reads of rows
//    whose lane groups sit a multiple of 64 floats apart, which gfx950 serves
//    at full rate), and issues k*k*4*RH fused multiply-adds with the plane's
//    weights held in vector registers;
//  * grad_input is the same computation on the grad_output tile with the
//    kernel flipped in both axes (stride 1, pad k/2, so the grad_output halo
//    has the same widths as the input halo);
//  * grad_weight: each thread accumulates all k*k taps (and the grad_bias
//    sum) over its RH x 4 outputs and keeps them across the consecutive tiles
//    of one channel that its workgroup owns; at a channel change the waves
//    reduce them with cross-lane swaps, the workgroup adds the waves' totals
//    in a fixed order and writes one partial; a second kernel sums a
//    channel's partials in workgroup order.  No atomics: results are bitwise
//    reproducible;
//  * the fused backward runs both on one grad_output tile: a 512-thread
//    workgroup whose first half computes grad_input from the grad_output tile
//    and whose second half accumulates grad_weight from the input tile and
//    the centre of that same grad_output tile, so grad_output is read from
//    HBM once for both gradients (the pair that a convolution backward call
//    returns together).
#include "internal.h"
#include "depthwise.h"
#include "lds_dma.h"
#include "wavesum.h"

namespace sscnn {
namespace {

struct DwArgs {
    const float* src;    // (N*C, H, W) tile source: the input (forward), grad_output (grad_input)
    const float* src_h;  // (N*C, H, 2P) its halo, or null (kernels instantiated without halo)
    const float* x;      // (N*C, H, W) input, for grad_weight
    const float* x_h;    // (N*C, H, 2P) its halo, or null (kernels instantiated without halo)
    const float* g;      // (N*C, H, W) grad_output, for the stand-alone grad_weight kernel
    const float* w;      // (C, k, k)
    const float* b;      // (C) or null
    float* out;          // (N*C, H, W) output or grad_input
    float* ws;           // grad_weight partials (C, up to N * tiles_h * tiles_w, k*k + 1)
    int H, W, C, N, tiles_h, tiles_w, ntiles;   // ntiles = N * C * tiles_h * tiles_w
    // Height sharding (kernels instantiated with ROWH): the rows above and
    // below the slice, (N*C, up + down, W) -- up rows first, then down rows.
    const float* src_rh;
    const float* x_rh;
    int src_up, src_down, x_up, x_down;
};

// One plane's rows beyond the slice (height sharding): rows -up .. -1 are
// p[0 .. up), rows H .. H + down - 1 are p[up .. up + down).
struct RowHalo {
    const float* p;
    int up, down;
};

__device__ __forceinline__ RowHalo row_halo(const float* base, int64_t plane, int up, int down, int W)
{
    return RowHalo{base + plane * (up + down) * W, up, down};
}

// A plane's column halo, (H, 2P) per plane; with ROWH as well (2-D shards) it
// covers the extended rows, (up + H + down, 2P) per plane, and the pointer
// returned is that of row 0 (so rows -up .. -1 sit before it).
template <bool HALO, bool ROWH>
__device__ __forceinline__ const float* col_halo(const float* base, int64_t plane, int H, int up, int down, int P)
{
    if constexpr (!HALO) return nullptr;
    if constexpr (ROWH) return base + plane * (up + H + down) * (2 * P) + up * (2 * P);
    return base + plane * H * (2 * P);
}

// One tile: its plane and channel, and the rows and columns it covers.  The
// last tile of a column is moved up to end at row H (i0 = H - TH) so every
// row it computes is a real row and its stores need no predicate; it then
// recomputes rows [i0, i_own) of the tile above it bit-identically, and
// i_own = trow * TH is the first row it owns (grad_weight counts only those).
struct TileIdx {
    int plane, c, n, i0, i_own, j0;
};

__device__ __forceinline__ void place(TileIdx& d, const DwArgs& a, int trow, int tcol, int th, int tw)
{
    d.plane = d.n * a.C + d.c;
    d.i_own = trow * th;
    d.i0 = d.i_own + th > a.H ? a.H - th : d.i_own;
    d.j0 = tcol * tw;
}

// A tile number as four mixed-radix digits (d0 fastest): plane-major order
// (forward and grad_input) is t = (n, c, row, column), channel-major order
// (grad_weight, fused backward) t = (c, n, row, column), so that a
// contiguous run of tiles mostly stays on one channel.  The digits are split
// once per workgroup and then advanced by carries: the runtime divisions of
// a decode cost ~20 scalar instructions each, which a wave would otherwise
// issue on every tile in place of its FMAs.
struct TileDigits {
    int d0, d1, d2, d3;     // column tile, row tile, then (c, n) or (n, c)
};

__device__ __forceinline__ TileDigits split_tile(int t, int r0, int r1, int r2)
{
    TileDigits g;
    g.d0 = t % r0;
    t /= r0;
    g.d1 = t % r1;
    t /= r1;
    g.d2 = t % r2;
    g.d3 = t / r2;
    return g;
}

// a + g digit by digit with carries (every digit of both below its radix, so
// one subtraction per digit suffices).
__device__ __forceinline__ TileDigits add_tile(TileDigits a, const TileDigits& g, int r0, int r1, int r2)
{
    int x = a.d0 + g.d0;
    int cy = x >= r0;
    a.d0 = cy ? x - r0 : x;
    x = a.d1 + g.d1 + cy;
    cy = x >= r1;
    a.d1 = cy ? x - r1 : x;
    x = a.d2 + g.d2 + cy;
    cy = x >= r2;
    a.d2 = cy ? x - r2 : x;
    a.d3 += g.d3 + cy;
    return a;
}

// The next tile, one step along the list.
__device__ __forceinline__ TileDigits next_tile(TileDigits a, int r0, int r1, int r2)
{
    return add_tile(a, TileDigits{1, 0, 0, 0}, r0, r1, r2);
}

__device__ __forceinline__ TileIdx plane_major_idx(const DwArgs& a, const TileDigits& g, int th, int tw)
{
    TileIdx d;
    d.c = g.d2;
    d.n = g.d3;
    place(d, a, g.d1, g.d0, th, tw);
    return d;
}

__device__ __forceinline__ TileIdx channel_major_idx(const DwArgs& a, const TileDigits& g, int th, int tw)
{
    TileIdx d;
    d.n = g.d2;
    d.c = g.d3;
    place(d, a, g.d1, g.d0, th, tw);
    return d;
}

// The extended input of one tile in LDS, for a 256-thread group (TX x TY
// threads, each owning RH rows x 4 columns of outputs).
//   main  LH rows x TW floats, pitch TW: main[rr][c] = plane[i0 - P + rr][j0 + c]
//   side  LH rows x 8 floats:  side[rr][4 - P + e] = column j0 - P + e   (e < P)
//                              side[rr][4 + e]     = column j0 + TW + e  (e < P)
template <int K, int TX, int TY, int RH>
struct Tile {
    static constexpr int P = K / 2;
    static constexpr int NT = TX * TY;
    static constexpr int NWAVE = NT / 64;
    static constexpr int TW = 4 * TX;
    static constexpr int TH = RH * TY;
    static constexpr int LH = TH + K - 1;
    static constexpr int MAIN = LH * TW;
    static constexpr int PIECES = LH * TX;                 // 16-byte pieces of the main region
    static constexpr int NLOAD = (PIECES + 63) / 64;       // 64-lane direct loads per tile
    static constexpr int SP = 8;
    static constexpr int FLOATS = MAIN + LH * SP;
    static constexpr int NS = (LH * 2 * P + NT - 1) / NT;  // side values per thread
    static_assert(NT % 64 == 0, "whole waves");
    static_assert((RH * TW) % (4 * TX) == 0, "row groups a multiple of the lane group apart");

    struct Side {
        float s[NS];
    };

    // Main region: buffer loads straight into LDS.  Piece f (lane f % 64 of
    // load f / 64) is 16 bytes of row f / TX; LDS receives load m's 64 pieces
    // contiguously, which is exactly main[] since TW = 4 TX.  Rows outside
    // the plane have offsets outside the buffer (negative offsets wrap to
    // huge ones) and read as zeros.
    // ROWH (height sharding): rows above and below the slice come from its
    // row halo instead; those loads are issued by the lanes they concern, so
    // each piece of LDS is still written by exactly one load.
    template <bool ROWH>
    __device__ static void load_main(float* buf, const float* plane, int H, int W, int i0, int j0, int tid,
                                     const RowHalo& rh)
    {
        const i32x4 rs = plane_rsrc(plane, H * W * 4);
        i32x4 rsh{};
        if constexpr (ROWH) rsh = plane_rsrc(rh.p, (rh.up + rh.down) * W * 4);
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
#pragma unroll
        for (int k = 0; k < (NLOAD + NWAVE - 1) / NWAVE; ++k) {
            const int m = wave + k * NWAVE;                    // wave-uniform
            if (m < NLOAD) {
                const int f = m * 64 + lane;
                const int rr = f / TX, q = f - rr * TX;
                const int r = i0 - P + rr;
                const int off = (r * W + j0 + 4 * q) * 4;
                if (f < PIECES) {
                    if constexpr (ROWH) {
                        if ((unsigned)r < (unsigned)H) {
                            dma16(rs, buf + m * 256, off);
                        } else {
                            // halo row; rows beyond it fall outside the halo buffer and read zeros
                            const int hr = r < 0 ? rh.up + r : rh.up + (r - H);
                            dma16(rsh, buf + m * 256, (hr * W + j0 + 4 * q) * 4);
                        }
                    } else {
                        dma16(rs, buf + m * 256, off);
                    }
                }
            }
        }
    }

    // Side columns: ordinary loads into registers, written by put_side().
    // Without a halo (HALO false: the interior half of a split convolution)
    // the columns beyond the slice are zeros.
    // ROWH: rows beyond the slice take their columns from its row halo.  Both
    // (2-D shards): the column halo covers the extended rows -up .. H+down-1
    // (hp points at its row 0), so the corners come from it too.
    template <bool HALO, bool ROWH>
    __device__ static void load_side(Side& S, const float* __restrict__ xp, const float* __restrict__ hp,
                                     int H, int W, int i0, int j0, int tid, const RowHalo& rh)
    {
        if constexpr (HALO && ROWH) {
#pragma unroll
            for (int k = 0; k < NS; ++k) {
                const int idx = tid + k * NT;
                const int rr = idx / (2 * P), e = idx - rr * (2 * P);
                const int r = i0 - P + rr;
                const int xcol = j0 + (e < P ? e : TW + e) - P;
                S.s[k] = 0.f;
                if (idx < LH * 2 * P && r >= -rh.up && r < H + rh.down) {
                    if (xcol < 0)
                        S.s[k] = hp[(int64_t)r * (2 * P) + (xcol + P)];
                    else if (xcol >= W)
                        S.s[k] = hp[(int64_t)r * (2 * P) + P + (xcol - W)];
                    else if (r >= 0 && r < H)
                        S.s[k] = xp[(int64_t)r * W + xcol];
                    else
                        S.s[k] = rh.p[(int64_t)(r < 0 ? rh.up + r : rh.up + (r - H)) * W + xcol];
                }
            }
            return;
        }
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            const int idx = tid + k * NT;
            const int rr = idx / (2 * P), e = idx - rr * (2 * P);
            const int r = i0 - P + rr;
            const int xcol = j0 + (e < P ? e : TW + e) - P;     // shard column, may be < 0 or >= W
            S.s[k] = 0.f;
            if (idx < LH * 2 * P && r >= 0 && r < H) {
                if (xcol < 0) {
                    if constexpr (HALO) S.s[k] = hp[(int64_t)r * (2 * P) + (xcol + P)];
                } else if (xcol >= W) {
                    if constexpr (HALO) S.s[k] = hp[(int64_t)r * (2 * P) + P + (xcol - W)];
                } else {
                    S.s[k] = xp[(int64_t)r * W + xcol];
                }
            } else if constexpr (ROWH) {
                const int hr = r < 0 ? rh.up + r : rh.up + (r - H);
                if (idx < LH * 2 * P && xcol >= 0 && xcol < W && hr >= 0 && hr < rh.up + rh.down)
                    S.s[k] = rh.p[(int64_t)hr * W + xcol];
            }
        }
    }

    __device__ static void put_side(float* buf, const Side& S, int tid)
    {
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            const int idx = tid + k * NT;
            if (idx < LH * 2 * P) {
                const int rr = idx / (2 * P), e = idx - rr * (2 * P);
                buf[MAIN + rr * SP + (e < P ? 4 - P + e : 4 + e - P)] = S.s[k];
            }
        }
    }

    // Where a thread's window of row R (4 + K - 1 values from column 4 tx - P)
    // comes from: A = the 4 floats left of its own 4 (side region for tx = 0),
    // B = its own 4, C = the 4 on the right (side region for tx = TX - 1).
    // A and C move down by a per-lane pitch; next() advances them one row
    // at a time (the empty asm keeps the compiler from precomputing and
    // holding every row's offset).
    typedef float nf4 __attribute__((ext_vector_type(4)));
    typedef float nf2 __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(3))) const float lfloat;
    typedef __attribute__((address_space(3))) const nf4 lfloat4;
    typedef __attribute__((address_space(3))) const nf2 lfloat2;

    struct Win {
        lfloat* a;
        lfloat* b;
        lfloat* c;
        int sa, sc;        // row pitches of a and c
        __device__ void next()
        {
            a += sa;
            c += sc;
            b += TW;
            asm volatile("" : "+v"(a), "+v"(c));
        }
    };

    __device__ static Win window(const float* buf_generic, int tx, int ty)
    {
        lfloat* buf = (lfloat*)buf_generic;
        Win w;
        const int r0 = ty * RH;
        w.b = buf + r0 * TW + 4 * tx;
        if (tx == 0) { w.a = buf + MAIN + r0 * SP; w.sa = SP; }
        else { w.a = w.b - 4; w.sa = TW; }
        if (tx == TX - 1) { w.c = buf + MAIN + r0 * SP + 4; w.sc = SP; }
        else { w.c = w.b + 4; w.sc = TW; }
        return w;
    }

    __device__ static void read_row(const Win& w, float (&in)[4 + K - 1])
    {
        const nf4 bb = *reinterpret_cast<lfloat4*>(w.b);
        if constexpr (P == 3) {
            const nf4 aa = *reinterpret_cast<lfloat4*>(w.a);
            const nf4 cc = *reinterpret_cast<lfloat4*>(w.c);
            in[0] = aa.y; in[1] = aa.z; in[2] = aa.w;
            in[7] = cc.x; in[8] = cc.y; in[9] = cc.z;
        } else if constexpr (P == 2) {
            const nf2 aa = *reinterpret_cast<lfloat2*>(w.a + 2);
            const nf2 cc = *reinterpret_cast<lfloat2*>(w.c);
            in[0] = aa.x; in[1] = aa.y;
            in[6] = cc.x; in[7] = cc.y;
        } else {
            in[0] = w.a[3];
            in[5] = w.c[0];
        }
        in[P] = bb.x; in[P + 1] = bb.y; in[P + 2] = bb.z; in[P + 3] = bb.w;
    }
};

// Forward / grad_input on one LDS tile: acc[i][jj] += sum over (kh, kw) of
// wr[kh*K + kw] * (extended input)[row i + kh, column jj + kw] for the
// thread's RH x 4 outputs.  Each row is read one row ahead of its FMAs; the
// scheduling barriers keep that order.
template <int K, int TX, int TY, int RH>
__device__ __forceinline__ void conv_tile(const float* buf, const float (&wr)[K * K], float (&acc)[RH][4],
                                          int tx, int ty)
{
    using T = Tile<K, TX, TY, RH>;
    typename T::Win w = T::window(buf, tx, ty);
    float cur[4 + K - 1], nxt[4 + K - 1];
    T::read_row(w, cur);
#pragma unroll
    for (int r = 0; r < RH + K - 1; ++r) {
        if (r + 1 < RH + K - 1) {
            w.next();
            T::read_row(w, nxt);
        }
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
}

// grad_weight on one LDS input tile: acc[kh*K + kw] += sum over the thread's
// outputs (i, jj) of gv[i][jj] * (extended input)[row i + kh, column jj + kw].
template <int K, int TX, int TY, int RH>
__device__ __forceinline__ void wgrad_tile(const float* buf, const float (&gv)[RH][4],
                                           float (&acc)[K * K + 1], int tx, int ty)
{
    using T = Tile<K, TX, TY, RH>;
    typename T::Win w = T::window(buf, tx, ty);
    float cur[4 + K - 1], nxt[4 + K - 1];
    T::read_row(w, cur);
#pragma unroll
    for (int r = 0; r < RH + K - 1; ++r) {
        if (r + 1 < RH + K - 1) {
            w.next();
            T::read_row(w, nxt);
        }
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
}

// The plane's weights (flipped in both axes for grad_input) in vector
// registers: loaded through the scalar cache, then copied, because gfx950
// issues v_fmac_f32 at about twice the rate when no operand is a scalar
// register (measured: ~119 vs ~70 TFLOP/s chip-wide).
template <int K, bool FLIP>
__device__ __forceinline__ void load_weights(const float* w, int c, float (&wr)[K * K])
{
    const auto wp = as_const(w) + c * K * K;
#pragma unroll
    for (int k = 0; k < K * K; ++k) wr[k] = to_vgpr(wp[FLIP ? K * K - 1 - k : k]);
}

// Results leave with non-temporal stores: nothing in these kernels reads
// them back, and streaming them past the caches took 8-16% off the forward
// (A/B on one GPU, depthwise 7x7 shards of 16x32 to 128x256 planes).
template <int RH>
__device__ __forceinline__ void store_rows(float* out, const TileIdx& d, int H, int W, int tx, int ty,
                                           const float (&acc)[RH][4])
{
    typedef float f4v __attribute__((ext_vector_type(4)));
    float* yp = out + (int64_t)d.plane * H * W + d.j0 + 4 * tx;
#pragma unroll
    for (int i = 0; i < RH; ++i) {
        const f4v v = {acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
        __builtin_nontemporal_store(v, reinterpret_cast<f4v*>(yp + (int64_t)(d.i0 + ty * RH + i) * W));
    }
}

template <int K, int TX, int TY, int RH, bool FLIP, bool HALO, bool ROWH>
__global__ void __launch_bounds__(TX * TY) __attribute__((amdgpu_waves_per_eu(4)))
dw_conv_kernel(DwArgs a)
{
    using T = Tile<K, TX, TY, RH>;
    constexpr int P = T::P;
    __shared__ __align__(16) float buf[2][T::FLOATS];
    typename T::Side S;
    const int tid = threadIdx.x;
    const int tx = tid % TX, ty = tid / TX;
    const int64_t HW = (int64_t)a.H * a.W;
    auto issue = [&](const TileIdx& e, float* b) {
        const RowHalo rh = ROWH ? row_halo(a.src_rh, e.plane, a.src_up, a.src_down, a.W) : RowHalo{};
        T::template load_main<ROWH>(b, a.src + e.plane * HW, a.H, a.W, e.i0, e.j0, tid, rh);
        T::template load_side<HALO, ROWH>(S, a.src + e.plane * HW,
                                          col_halo<HALO, ROWH>(a.src_h, e.plane, a.H, a.src_up, a.src_down, P),
                                          a.H, a.W, e.i0, e.j0, tid, rh);
    };
    int t = blockIdx.x;
    if (t >= a.ntiles) return;
    // Tiles t, t + G, t + 2G, ... (G = gridDim.x): the digits of t and of the
    // stride G are split once, then added.
    TileDigits cur = split_tile(t, a.tiles_w, a.tiles_h, a.C);
    const TileDigits step = split_tile(gridDim.x, a.tiles_w, a.tiles_h, a.C);
    issue(plane_major_idx(a, cur, T::TH, T::TW), buf[0]);
    // A tile's stores are issued after the next tile's barrier, so the wait
    // before that barrier only covers operations a whole tile old.
    float acc[RH][4];
    TileIdx dprev{};
    float wr[K * K];
    int wc = -1;                     // channel whose weights wr holds
    for (int it = 0; t < a.ntiles; t += gridDim.x, ++it) {
        float* cb = buf[it & 1];
        const TileIdx d = plane_major_idx(a, cur, T::TH, T::TW);
        cur = add_tile(cur, step, a.tiles_w, a.tiles_h, a.C);
        T::put_side(cb, S, tid);
        wait_vmem();
        lds_barrier();
        if (it > 0) store_rows<RH>(a.out, dprev, a.H, a.W, tx, ty, acc);
        if (t + (int)gridDim.x < a.ntiles) issue(plane_major_idx(a, cur, T::TH, T::TW), buf[(it + 1) & 1]);
        if (d.c != wc) {             // consecutive tiles often share a channel
            load_weights<K, FLIP>(a.w, d.c, wr);
            wc = d.c;
        }
        const float bias = a.b ? as_const(a.b)[d.c] : 0.f;
#pragma unroll
        for (int i = 0; i < RH; ++i)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) acc[i][jj] = bias;
        conv_tile<K, TX, TY, RH>(cb, wr, acc, tx, ty);
        dprev = d;
    }
    store_rows<RH>(a.out, dprev, a.H, a.W, tx, ty, acc);
}

// Workgroups of the grad_weight kernels take contiguous runs of the
// channel-major tile list: workgroup w owns tiles [floor(wT/G), floor((w+1)T/G)).
// One flush per (workgroup, channel) writes one partial; channel c's partials
// are numbered by workgroup from the one that owns its first tile.
__device__ __forceinline__ int64_t tile_owner(int64_t t, int64_t T, int64_t G)
{
    return ((t + 1) * G - 1) / T;     // the workgroup w with floor(wT/G) <= t < floor((w+1)T/G)
}

// Flush of a run, first step: each wave's totals (a reduce-scatter over its
// lanes) into red[wave][].
template <int NV, int NWAVE>
__device__ __forceinline__ void flush_write(const float (&acc)[NV], float (*red)[NV + 2], int gtid)
{
    const int lane = gtid & 63, wave = gtid >> 6;
    const float s = wave_sum_scatter<NV>(acc, lane);
    const int idx = wave_sum_index<NV>(lane);
    if (idx >= 0) red[wave][idx] = s;
}

// Second step (after a barrier): the waves' totals added in a fixed order.
template <int NV, int NWAVE>
__device__ __forceinline__ void flush_sum(float (*red)[NV + 2], int gtid, float* ws, int64_t slot)
{
    if (gtid < NV) {
        float tot = red[0][gtid];
#pragma unroll
        for (int w = 1; w < NWAVE; ++w) tot += red[w][gtid];
        ws[slot * NV + gtid] = tot;
    }
}

// grad_weight partial (stand-alone): the input tile comes through LDS, the
// thread's grad_output block straight from global memory.
template <int K, int TX, int TY, int RH, bool HALO, bool ROWH>
__global__ void __launch_bounds__(TX * TY) __attribute__((amdgpu_waves_per_eu(3)))
dw_wgrad_kernel(DwArgs a)
{
    using T = Tile<K, TX, TY, RH>;
    constexpr int P = T::P;
    constexpr int KK = K * K;
    constexpr int NV = KK + 1;                  // taps + bias
    constexpr int NWAVE = T::NWAVE;
    __shared__ __align__(16) float buf[2][T::FLOATS];
    __shared__ float red[NWAVE][NV + 2];
    typename T::Side S;
    float4 gnext[RH];
    const int tid = threadIdx.x;
    const int tx = tid % TX, ty = tid / TX;
    const int tiles_c = a.ntiles / a.C;         // N * tiles_h * tiles_w
    const int64_t G = gridDim.x;
    const int64_t HW = (int64_t)a.H * a.W;
    const int beg = (int)((int64_t)blockIdx.x * a.ntiles / G);
    const int end = (int)((int64_t)(blockIdx.x + 1) * a.ntiles / G);
    if (beg >= end) return;
    auto issue = [&](const TileIdx& e, float* b) {
        const RowHalo rh = ROWH ? row_halo(a.x_rh, e.plane, a.x_up, a.x_down, a.W) : RowHalo{};
        T::template load_main<ROWH>(b, a.x + e.plane * HW, a.H, a.W, e.i0, e.j0, tid, rh);
        T::template load_side<HALO, ROWH>(S, a.x + e.plane * HW,
                                          col_halo<HALO, ROWH>(a.x_h, e.plane, a.H, a.x_up, a.x_down, P), a.H,
                                          a.W, e.i0, e.j0, tid, rh);
        const float* gp = a.g + e.plane * HW + e.j0 + 4 * tx;
#pragma unroll
        for (int i = 0; i < RH; ++i) {
            const int row = e.i0 + ty * RH + i;
            gnext[i] = *reinterpret_cast<const float4*>(gp + (int64_t)row * a.W);
            const float m = row >= e.i_own ? 1.f : 0.f;       // rows the tile above owns
            gnext[i].x *= m; gnext[i].y *= m; gnext[i].z *= m; gnext[i].w *= m;
        }
    };
    TileDigits cur = split_tile(beg, a.tiles_w, a.tiles_h, a.N);    // tile t, channel-major
    issue(channel_major_idx(a, cur, T::TH, T::TW), buf[0]);
    int it = 0;
    for (int t = beg; t < end;) {
        const int c = cur.d3;
        const int run_end = min(end, (c + 1) * tiles_c);
        float acc[NV];
#pragma unroll
        for (int k = 0; k < NV; ++k) acc[k] = 0.f;
        for (; t < run_end; ++t, ++it) {
            float* cb = buf[it & 1];
            T::put_side(cb, S, tid);
            float gv[RH][4];
#pragma unroll
            for (int i = 0; i < RH; ++i) {
                gv[i][0] = gnext[i].x; gv[i][1] = gnext[i].y; gv[i][2] = gnext[i].z; gv[i][3] = gnext[i].w;
                acc[KK] += (gv[i][0] + gv[i][1]) + (gv[i][2] + gv[i][3]);
            }
            wait_vmem();
            lds_barrier();
            cur = next_tile(cur, a.tiles_w, a.tiles_h, a.N);
            if (t + 1 < end) issue(channel_major_idx(a, cur, T::TH, T::TW), buf[(it + 1) & 1]);
            wgrad_tile<K, TX, TY, RH>(cb, gv, acc, tx, ty);
        }
        flush_write<NV, NWAVE>(acc, red, tid);
        lds_barrier();
        flush_sum<NV, NWAVE>(red, tid, a.ws, (int64_t)c * tiles_c + blockIdx.x -
                                                 tile_owner((int64_t)c * tiles_c, a.ntiles, G));
    }
}

// Fused backward: threads [0, NT) compute grad_input from the grad_output
// tile, threads [NT, 2 NT) accumulate grad_weight from the input tile and the
// grad_output tile's centre.  Both halves walk the same tiles with the same
// barriers in the same order (two loops with identical barrier sequences, so
// each half's registers are allocated on their own).
template <int K, int TX, int TY, int RH, bool HALO, bool ROWH>
__global__ void __launch_bounds__(2 * TX * TY) __attribute__((amdgpu_waves_per_eu(4)))
dw_bwd_kernel(DwArgs a)
{
    using T = Tile<K, TX, TY, RH>;
    constexpr int P = T::P;
    constexpr int KK = K * K;
    constexpr int NV = KK + 1;
    constexpr int NWAVE = T::NWAVE;
    __shared__ __align__(16) float bufg[2][T::FLOATS];   // grad_output tiles (extended)
    __shared__ __align__(16) float bufx[2][T::FLOATS];   // input tiles (extended)
    __shared__ float red[NWAVE][NV + 2];
    typename T::Side S;
    const bool wgrad_half = threadIdx.x >= T::NT;    // wave-uniform
    const int tid = threadIdx.x - (wgrad_half ? T::NT : 0);
    const int tx = tid % TX, ty = tid / TX;
    const int tiles_c = a.ntiles / a.C;
    const int64_t G = gridDim.x;
    const int64_t HW = (int64_t)a.H * a.W;
    const int beg = (int)((int64_t)blockIdx.x * a.ntiles / G);
    const int end = (int)((int64_t)(blockIdx.x + 1) * a.ntiles / G);
    if (beg >= end) return;
    const float* const src = wgrad_half ? a.x : a.src;
    const float* const src_h = wgrad_half ? a.x_h : a.src_h;
    const float* const src_rh = wgrad_half ? a.x_rh : a.src_rh;
    const int up = wgrad_half ? a.x_up : a.src_up, down = wgrad_half ? a.x_down : a.src_down;
    float (*const mybuf)[T::FLOATS] = wgrad_half ? bufx : bufg;
    auto issue = [&](const TileIdx& e, float* b) {
        const RowHalo rh = ROWH ? row_halo(src_rh, e.plane, up, down, a.W) : RowHalo{};
        T::template load_main<ROWH>(b, src + e.plane * HW, a.H, a.W, e.i0, e.j0, tid, rh);
        T::template load_side<HALO, ROWH>(S, src + e.plane * HW,
                                          col_halo<HALO, ROWH>(src_h, e.plane, a.H, up, down, P), a.H, a.W,
                                          e.i0, e.j0, tid, rh);
    };
    TileDigits cur = split_tile(beg, a.tiles_w, a.tiles_h, a.N);    // tile t, channel-major
    issue(channel_major_idx(a, cur, T::TH, T::TW), mybuf[0]);

    if (!wgrad_half) {
        int it = 0;
        float acc[RH][4];
        TileIdx dprev{};
        for (int t = beg; t < end;) {
            const int c = cur.d3;
            const int run_end = min(end, (c + 1) * tiles_c);
            float wr[KK];
            load_weights<K, true>(a.w, c, wr);
            for (; t < run_end; ++t, ++it) {
                float* cb = bufg[it & 1];
                const TileIdx d = channel_major_idx(a, cur, T::TH, T::TW);
                cur = next_tile(cur, a.tiles_w, a.tiles_h, a.N);
                T::put_side(cb, S, tid);
                wait_vmem();
                lds_barrier();
                if (it > 0) store_rows<RH>(a.out, dprev, a.H, a.W, tx, ty, acc);   // previous tile's
                if (t + 1 < end) issue(channel_major_idx(a, cur, T::TH, T::TW), bufg[(it + 1) & 1]);
#pragma unroll
                for (int i = 0; i < RH; ++i)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) acc[i][jj] = 0.f;
                conv_tile<K, TX, TY, RH>(cb, wr, acc, tx, ty);
                dprev = d;
            }
            lds_barrier();   // the flush's barrier
        }
        store_rows<RH>(a.out, dprev, a.H, a.W, tx, ty, acc);
    } else {
        int it = 0;
        for (int t = beg; t < end;) {
            const int c = cur.d3;
            const int run_end = min(end, (c + 1) * tiles_c);
            float acc[NV];
#pragma unroll
            for (int k = 0; k < NV; ++k) acc[k] = 0.f;
            for (; t < run_end; ++t, ++it) {
                float* cb = bufx[it & 1];
                const TileIdx d = channel_major_idx(a, cur, T::TH, T::TW);
                cur = next_tile(cur, a.tiles_w, a.tiles_h, a.N);
                T::put_side(cb, S, tid);
                wait_vmem();
                lds_barrier();
                if (t + 1 < end) issue(channel_major_idx(a, cur, T::TH, T::TW), bufx[(it + 1) & 1]);
                // grad_output at the thread's outputs: the centre of this
                // tile's grad_output buffer (main region row P + i, column j)
                float gv[RH][4];
                const float* gp = bufg[it & 1] + (ty * RH + P) * T::TW + 4 * tx;
#pragma unroll
                for (int i = 0; i < RH; ++i) {
                    const float4 v = *reinterpret_cast<const float4*>(gp + i * T::TW);
                    const float m = d.i0 + ty * RH + i >= d.i_own ? 1.f : 0.f;   // rows the tile above owns
                    gv[i][0] = v.x * m; gv[i][1] = v.y * m; gv[i][2] = v.z * m; gv[i][3] = v.w * m;
                    acc[KK] += (gv[i][0] + gv[i][1]) + (gv[i][2] + gv[i][3]);
                }
                wgrad_tile<K, TX, TY, RH>(cb, gv, acc, tx, ty);
            }
            flush_write<NV, NWAVE>(acc, red, tid);
            lds_barrier();
            flush_sum<NV, NWAVE>(red, tid, a.ws, (int64_t)c * tiles_c + blockIdx.x -
                                                     tile_owner((int64_t)c * tiles_c, a.ntiles, G));
        }
    }
}

// Second pass: grad_w[c, tap] = sum of channel c's partials in workgroup
// order (one per workgroup whose run of tiles meets the channel).
// The owners are computed in 32-bit arithmetic (U32) whenever
// (ntiles + 1) * grid fits in 32 bits, as it does for every layer here: the
// 64-bit division is a long software sequence that dominated this small
// kernel.
template <int K, bool U32>
__global__ void __launch_bounds__(256)
dw_wgrad_reduce_kernel(const float* __restrict__ ws, int C, int tiles_c, int64_t ntiles, int64_t grid,
                       float* __restrict__ gw, float* __restrict__ gb)
{
    constexpr int NV = K * K + 1;
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= C * NV) return;
    const int c = idx / NV, t = idx - c * NV;
    int64_t w0, w1;
    if constexpr (U32) {
        const uint32_t T = (uint32_t)ntiles, G = (uint32_t)grid;
        w0 = (((uint32_t)c * tiles_c + 1) * G - 1) / T;
        w1 = (((uint32_t)(c + 1) * tiles_c) * G - 1) / T;
    } else {
        w0 = tile_owner((int64_t)c * tiles_c, ntiles, grid);
        w1 = tile_owner((int64_t)(c + 1) * tiles_c - 1, ntiles, grid);
    }
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
    if (W % 32 == 0) {
        if (H >= 64) return {8, 32, 2};
        // Two rows per thread where the plane is 32 or 16 rows high: each
        // input row read from LDS feeds two output rows, and the workgroups
        // get smaller (128 or 64 threads).  Against one row per thread in
        // 256- or 128-thread groups, on one GPU: (7,1024,32,32) forward
        // 17.5 -> 15.7 us, fused backward 35.8 -> 29.8 us; (7,2048,16,32)
        // 17.8 -> 16.0 and 35.8 -> 30.9 us.
        if (H >= 32) return {8, 16, 2};
        return {8, 8, H >= 16 ? 2 : 0};
    }
    if (H >= 64) return {4, 64, 1};
    return {4, 16, H >= 16 ? 1 : 0};          // 16-row tiles of 64 threads
}

// The fused backward keeps two rows per thread where the other kernels keep
// four: each half then fits in 128 registers, so two 512-thread workgroups
// share a compute unit (four waves per SIMD) without spilling.
DwShape bwd_shape(int H, int W)
{
    DwShape sh = pick_shape(H, W);
    if (sh.tx == 16 && sh.ty == 16 && sh.rh == 4) sh.rh = 2;
    return sh;
}

int64_t tiles_per_channel(int N, int H, int W, DwShape sh)
{
    return (int64_t)N * ((H + sh.rh * sh.ty - 1) / (sh.rh * sh.ty)) * (W / (4 * sh.tx));
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

void set_tiles(DwArgs& a, int planes, int tx, int ty, int rh)
{
    a.tiles_w = a.W / (4 * tx);
    a.tiles_h = (a.H + rh * ty - 1) / (rh * ty);
    a.ntiles = planes * a.tiles_h * a.tiles_w;
}

template <int K>
hipError_t launch_reduce(const DwArgs& a, int grid, float* gw, float* gb, hipStream_t st)
{
    const int tiles_c = a.ntiles / a.C;
    const int total = a.C * (K * K + 1);
    if (((int64_t)a.ntiles + 1) * grid < ((int64_t)1 << 32))
        hipLaunchKernelGGL((dw_wgrad_reduce_kernel<K, true>), dim3((total + 255) / 256), dim3(256), 0, st, a.ws,
                           a.C, tiles_c, (int64_t)a.ntiles, (int64_t)grid, gw, gb);
    else
        hipLaunchKernelGGL((dw_wgrad_reduce_kernel<K, false>), dim3((total + 255) / 256), dim3(256), 0, st, a.ws,
                           a.C, tiles_c, (int64_t)a.ntiles, (int64_t)grid, gw, gb);
    return hipGetLastError();
}

// The instantiated tile shapes (pick_shape() returns one of these).
#define SSCNN_DW_SHAPES(X) X(16, 16, 4) X(16, 16, 2) X(16, 16, 1) X(8, 32, 2) X(8, 16, 2) X(8, 8, 2) \
    X(4, 64, 1) X(4, 16, 1)
// and the ones bwd_shape() returns
#define SSCNN_DW_BWD_SHAPES(X) X(16, 16, 2) X(16, 16, 1) X(8, 32, 2) X(8, 16, 2) X(8, 8, 2) X(4, 64, 1) \
    X(4, 16, 1)

template <int K, bool FLIP, bool HALO, bool ROWH>
hipError_t launch_conv(DwArgs a, int planes, DwShape sh, hipStream_t st)
{
#define SSCNN_DW_CONV(TX, TY, RH)                                                  \
    if (sh.tx == TX && sh.ty == TY && sh.rh == RH) {                               \
        auto kern = dw_conv_kernel<K, TX, TY, RH, FLIP, HALO, ROWH>;               \
        set_tiles(a, planes, TX, TY, RH);                                          \
        const int grid = persistent_grid(kern, TX * TY, a.ntiles);                 \
        hipLaunchKernelGGL(kern, dim3(grid), dim3(TX * TY), 0, st, a);             \
        return hipGetLastError();                                                  \
    }
    SSCNN_DW_SHAPES(SSCNN_DW_CONV)
#undef SSCNN_DW_CONV
    return hipErrorInvalidValue;
}

template <int K, bool HALO, bool ROWH>
hipError_t launch_wgrad(DwArgs a, int planes, DwShape sh, float* gw, float* gb, hipStream_t st)
{
#define SSCNN_DW_WGRAD(TX, TY, RH)                                                 \
    if (sh.tx == TX && sh.ty == TY && sh.rh == RH) {                               \
        auto kern = dw_wgrad_kernel<K, TX, TY, RH, HALO, ROWH>;                    \
        set_tiles(a, planes, TX, TY, RH);                                          \
        const int grid = persistent_grid(kern, TX * TY, a.ntiles);                 \
        hipLaunchKernelGGL(kern, dim3(grid), dim3(TX * TY), 0, st, a);             \
        const hipError_t e = hipGetLastError();                                    \
        return e != hipSuccess ? e : launch_reduce<K>(a, grid, gw, gb, st);        \
    }
    SSCNN_DW_SHAPES(SSCNN_DW_WGRAD)
#undef SSCNN_DW_WGRAD
    return hipErrorInvalidValue;
}

template <int K, bool HALO, bool ROWH>
hipError_t launch_bwd(DwArgs a, int planes, DwShape sh, float* gw, float* gb, hipStream_t st)
{
#define SSCNN_DW_BWD(TX, TY, RH)                                                   \
    if (sh.tx == TX && sh.ty == TY && sh.rh == RH) {                               \
        auto kern = dw_bwd_kernel<K, TX, TY, RH, HALO, ROWH>;                      \
        set_tiles(a, planes, TX, TY, RH);                                          \
        const int grid = persistent_grid(kern, 2 * TX * TY, a.ntiles);             \
        hipLaunchKernelGGL(kern, dim3(grid), dim3(2 * TX * TY), 0, st, a);         \
        const hipError_t e = hipGetLastError();                                    \
        return e != hipSuccess ? e : launch_reduce<K>(a, grid, gw, gb, st);        \
    }
    SSCNN_DW_BWD_SHAPES(SSCNN_DW_BWD)
#undef SSCNN_DW_BWD
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

// One partial slot per tile of a channel at most, for whichever of the
// grad_weight kernel and the fused backward has more tiles.
size_t dw_wgrad_workspace_bytes(const Geom& g)
{
    const int64_t t1 = tiles_per_channel(g.n, g.h, g.wl, pick_shape(g.h, g.wl));
    const int64_t t2 = tiles_per_channel(g.n, g.h, g.wl, bwd_shape(g.h, g.wl));
    const int64_t tiles = t1 > t2 ? t1 : t2;
    return (size_t)(tiles * g.ci * (g.k * g.k + 1)) * sizeof(float);
}

hipError_t launch_dw_fwd(const Geom& g, const float* x, const float* xh, const float* w,
                         const float* b, float* y, hipStream_t st)
{
    DwArgs a = make_args(g);
    a.src = x; a.src_h = xh; a.w = w; a.b = b; a.out = y;
    const int planes = g.n * g.ci;
    const DwShape sh = pick_shape(g.h, g.wl);
    switch (g.k) {
        case 3: return xh ? launch_conv<3, false, true, false>(a, planes, sh, st) : launch_conv<3, false, false, false>(a, planes, sh, st);
        case 5: return xh ? launch_conv<5, false, true, false>(a, planes, sh, st) : launch_conv<5, false, false, false>(a, planes, sh, st);
        default: return xh ? launch_conv<7, false, true, false>(a, planes, sh, st) : launch_conv<7, false, false, false>(a, planes, sh, st);
    }
}

hipError_t launch_dw_bwd_input(const Geom& g, const float* gy, const float* gyh, const float* w,
                               float* gx, hipStream_t st)
{
    DwArgs a = make_args(g);
    a.src = gy; a.src_h = gyh; a.w = w; a.b = nullptr; a.out = gx;
    const int planes = g.n * g.ci;
    const DwShape sh = pick_shape(g.h, g.wl);
    switch (g.k) {
        case 3: return gyh ? launch_conv<3, true, true, false>(a, planes, sh, st) : launch_conv<3, true, false, false>(a, planes, sh, st);
        case 5: return gyh ? launch_conv<5, true, true, false>(a, planes, sh, st) : launch_conv<5, true, false, false>(a, planes, sh, st);
        default: return gyh ? launch_conv<7, true, true, false>(a, planes, sh, st) : launch_conv<7, true, false, false>(a, planes, sh, st);
    }
}

hipError_t launch_dw_bwd_weight(const Geom& g, const float* x, const float* xh, const float* gy,
                                float* gw, float* gb, void* ws, hipStream_t st)
{
    DwArgs a = make_args(g);
    a.x = x; a.x_h = xh; a.g = gy; a.ws = static_cast<float*>(ws);
    const int planes = g.n * g.ci;
    const DwShape sh = pick_shape(g.h, g.wl);
    switch (g.k) {
        case 3: return xh ? launch_wgrad<3, true, false>(a, planes, sh, gw, gb, st) : launch_wgrad<3, false, false>(a, planes, sh, gw, gb, st);
        case 5: return xh ? launch_wgrad<5, true, false>(a, planes, sh, gw, gb, st) : launch_wgrad<5, false, false>(a, planes, sh, gw, gb, st);
        default: return xh ? launch_wgrad<7, true, false>(a, planes, sh, gw, gb, st) : launch_wgrad<7, false, false>(a, planes, sh, gw, gb, st);
    }
}

hipError_t launch_dw_bwd(const Geom& g, const float* x, const float* xh, const float* gy, const float* gyh,
                         const float* w, float* gx, float* gw, float* gb, void* ws, hipStream_t st)
{
    DwArgs a = make_args(g);
    a.src = gy; a.src_h = gyh; a.x = x; a.x_h = xh; a.w = w; a.out = gx; a.ws = static_cast<float*>(ws);
    const int planes = g.n * g.ci;
    const DwShape sh = bwd_shape(g.h, g.wl);
    if ((xh == nullptr) != (gyh == nullptr)) return hipErrorInvalidValue;   // both halos or neither
    switch (g.k) {
        case 3: return xh ? launch_bwd<3, true, false>(a, planes, sh, gw, gb, st) : launch_bwd<3, false, false>(a, planes, sh, gw, gb, st);
        case 5: return xh ? launch_bwd<5, true, false>(a, planes, sh, gw, gb, st) : launch_bwd<5, false, false>(a, planes, sh, gw, gb, st);
        default: return xh ? launch_bwd<7, true, false>(a, planes, sh, gw, gb, st) : launch_bwd<7, false, false>(a, planes, sh, gw, gb, st);
    }
}

// Height sharding: rows beyond the slice's top and bottom from its row halos
// (N*C, up + down, W); the slice spans the whole width, so no column halo.
hipError_t launch_dw_fwd_rows(const Geom& g, const float* x, const float* x_rh, int up, int down,
                              const float* w, const float* b, float* y, hipStream_t st)
{
    DwArgs a = make_args(g);
    a.src = x; a.src_rh = x_rh; a.src_up = up; a.src_down = down; a.w = w; a.b = b; a.out = y;
    const int planes = g.n * g.ci;
    const DwShape sh = pick_shape(g.h, g.wl);
    switch (g.k) {
        case 3: return launch_conv<3, false, false, true>(a, planes, sh, st);
        case 5: return launch_conv<5, false, false, true>(a, planes, sh, st);
        default: return launch_conv<7, false, false, true>(a, planes, sh, st);
    }
}

hipError_t launch_dw_bwd_input_rows(const Geom& g, const float* gy, const float* gy_rh, int up, int down,
                                    const float* w, float* gx, hipStream_t st)
{
    DwArgs a = make_args(g);
    a.src = gy; a.src_rh = gy_rh; a.src_up = up; a.src_down = down; a.w = w; a.b = nullptr; a.out = gx;
    const int planes = g.n * g.ci;
    const DwShape sh = pick_shape(g.h, g.wl);
    switch (g.k) {
        case 3: return launch_conv<3, true, false, true>(a, planes, sh, st);
        case 5: return launch_conv<5, true, false, true>(a, planes, sh, st);
        default: return launch_conv<7, true, false, true>(a, planes, sh, st);
    }
}

hipError_t launch_dw_bwd_weight_rows(const Geom& g, const float* x, const float* x_rh, int up, int down,
                                     const float* gy, float* gw, float* gb, void* ws, hipStream_t st)
{
    DwArgs a = make_args(g);
    a.x = x; a.x_rh = x_rh; a.x_up = up; a.x_down = down; a.g = gy; a.ws = static_cast<float*>(ws);
    const int planes = g.n * g.ci;
    const DwShape sh = pick_shape(g.h, g.wl);
    switch (g.k) {
        case 3: return launch_wgrad<3, false, true>(a, planes, sh, gw, gb, st);
        case 5: return launch_wgrad<5, false, true>(a, planes, sh, gw, gb, st);
        default: return launch_wgrad<7, false, true>(a, planes, sh, gw, gb, st);
    }
}

hipError_t launch_dw_bwd_rows(const Geom& g, const float* x, const float* x_rh, int x_up, int x_down,
                              const float* gy, const float* gy_rh, int g_up, int g_down, const float* w, float* gx,
                              float* gw, float* gb, void* ws, hipStream_t st)
{
    DwArgs a = make_args(g);
    a.src = gy; a.src_rh = gy_rh; a.src_up = g_up; a.src_down = g_down;
    a.x = x; a.x_rh = x_rh; a.x_up = x_up; a.x_down = x_down;
    a.w = w; a.out = gx; a.ws = static_cast<float*>(ws);
    const int planes = g.n * g.ci;
    const DwShape sh = bwd_shape(g.h, g.wl);
    switch (g.k) {
        case 3: return launch_bwd<3, false, true>(a, planes, sh, gw, gb, st);
        case 5: return launch_bwd<5, false, true>(a, planes, sh, gw, gb, st);
        default: return launch_bwd<7, false, true>(a, planes, sh, gw, gb, st);
    }
}

// 2-D shards: rows beyond the block from its row halo (N*C, up + down, W),
// columns beside it from its column halo over the extended rows
// (N*C, up + H + down, 2P), corners included.
hipError_t launch_dw_fwd_grid(const Geom& g, const float* x, const float* x_rh, const float* x_ch, int up, int down,
                              const float* w, const float* b, float* y, hipStream_t st)
{
    DwArgs a = make_args(g);
    a.src = x; a.src_rh = x_rh; a.src_h = x_ch; a.src_up = up; a.src_down = down; a.w = w; a.b = b; a.out = y;
    const int planes = g.n * g.ci;
    const DwShape sh = pick_shape(g.h, g.wl);
    switch (g.k) {
        case 3: return launch_conv<3, false, true, true>(a, planes, sh, st);
        case 5: return launch_conv<5, false, true, true>(a, planes, sh, st);
        default: return launch_conv<7, false, true, true>(a, planes, sh, st);
    }
}

hipError_t launch_dw_bwd_input_grid(const Geom& g, const float* gy, const float* gy_rh, const float* gy_ch, int up,
                                    int down, const float* w, float* gx, hipStream_t st)
{
    DwArgs a = make_args(g);
    a.src = gy; a.src_rh = gy_rh; a.src_h = gy_ch; a.src_up = up; a.src_down = down; a.w = w; a.b = nullptr;
    a.out = gx;
    const int planes = g.n * g.ci;
    const DwShape sh = pick_shape(g.h, g.wl);
    switch (g.k) {
        case 3: return launch_conv<3, true, true, true>(a, planes, sh, st);
        case 5: return launch_conv<5, true, true, true>(a, planes, sh, st);
        default: return launch_conv<7, true, true, true>(a, planes, sh, st);
    }
}

hipError_t launch_dw_bwd_weight_grid(const Geom& g, const float* x, const float* x_rh, const float* x_ch, int up,
                                     int down, const float* gy, float* gw, float* gb, void* ws, hipStream_t st)
{
    DwArgs a = make_args(g);
    a.x = x; a.x_rh = x_rh; a.x_h = x_ch; a.x_up = up; a.x_down = down; a.g = gy; a.ws = static_cast<float*>(ws);
    const int planes = g.n * g.ci;
    const DwShape sh = pick_shape(g.h, g.wl);
    switch (g.k) {
        case 3: return launch_wgrad<3, true, true>(a, planes, sh, gw, gb, st);
        case 5: return launch_wgrad<5, true, true>(a, planes, sh, gw, gb, st);
        default: return launch_wgrad<7, true, true>(a, planes, sh, gw, gb, st);
    }
}

hipError_t launch_dw_bwd_grid(const Geom& g, const float* x, const float* x_rh, const float* x_ch, int x_up,
                              int x_down, const float* gy, const float* gy_rh, const float* gy_ch, int g_up,
                              int g_down, const float* w, float* gx, float* gw, float* gb, void* ws, hipStream_t st)
{
    DwArgs a = make_args(g);
    a.src = gy; a.src_rh = gy_rh; a.src_h = gy_ch; a.src_up = g_up; a.src_down = g_down;
    a.x = x; a.x_rh = x_rh; a.x_h = x_ch; a.x_up = x_up; a.x_down = x_down;
    a.w = w; a.out = gx; a.ws = static_cast<float*>(ws);
    const int planes = g.n * g.ci;
    const DwShape sh = bwd_shape(g.h, g.wl);
    switch (g.k) {
        case 3: return launch_bwd<3, true, true>(a, planes, sh, gw, gb, st);
        case 5: return launch_bwd<5, true, true>(a, planes, sh, gw, gb, st);
        default: return launch_bwd<7, true, true>(a, planes, sh, gw, gb, st);
    }
}

}  // namespace sscnn
