// patchify.hip -- dense convolutions whose kernel equals their stride (k = s,
// pad 0, groups 1) on the FP32 matrix cores of gfx950 (v_mfma_f32_32x32x2_f32):
// the 4x4/4 stem and the 2x2/2 downsamples of the ConvNeXt-style stack that
// the pages shard (NVIDIA blog "Perception Model Training for Autonomous
// Vehicles with Tensor Parallelism", DTensor section: ConvNeXt-XL trained with
// Shard(3) activations), and the 1x1 expansion and projection of the
// ConvNeXt block (k = s = 1).  Such a layer needs no halo (its patches never
// straddle a shard edge), and it is a matrix product after a reshape: with
// K = (ci, kh, kw) and the output pixels p = (i, j) of one image,
//     forward       Y[co][p]   = b[co] + sum_K W[co][K] * Xp[K][p]
//     grad_input    dXp[K][p]  = sum_co W[co][K] * G[co][p]
//     grad_weight   gW[co][K]  = sum_(n,p) G[co][p] * Xp[K][p],  gB[co] = sum G
// where Xp[K][p] = X[ci][i*s + kh][j*s + kw].  The reshape is never
// materialised: operand tiles are gathered from NCHW straight into LDS (s
// consecutive floats per (K group, pixel)), and grad_input's result is
// scattered back to NCHW with one s-wide store per lane.
// For the 1x1 expansion the block follows with GELU: its forward can write
// GELU(Y) beside Y from the same registers, and the projection's grad_input
// can leave dX * GELU'(pre) instead of dX, reading pre at the address it
// stores to, so the elementwise passes over the 4C-channel tensor vanish.
//
// One kernel template serves the three products: a 256-thread workgroup
// computes a 128 x 128 tile of the result, each of its 4 waves a 64 x 64
// block (2 x 2 MFMA blocks of 32 x 32).  The reduction is gathered in
// sub-chunks of 16 (the unit every operand gather below is written for) and
// staged in LDS kKS sub-chunks at a time (k-major rows, double-buffered), one
// barrier per stage, the next stage's global loads in flight while the
// current one multiplies; a reduction that is not a whole number of stages
// ends on zero-filled sub-chunks.  One sub-chunk per stage (40 KB of LDS) is
// the measured best on gfx950: two (80 KB) allow only two workgroups per CU
// instead of four, and the downsamples ran 5-7% slower.
// grad_weight splits the pixel reduction over workgroups (a fixed split
// count; grad_bias fused into the first column tile).  Each split writes one
// slab of partials, and the slabs are summed in split order, in two
// fixed-order stages when there are many: no atomics, bitwise reproducible.
#include <cstdlib>
#include <cstring>

#include "internal.h"
#include "patchify.h"
#include "gelu.h"
#include "lds_dma.h"

namespace sscnn {
namespace {

// Outputs leave with non-temporal stores (the buffer-store cache-policy bit
// for it, and __builtin_nontemporal_store): no kernel here reads them back,
// and streaming them past the caches measured faster for the bandwidth-heavy
// epilogues.
constexpr int kNonTemporal = 2;
typedef float f2v __attribute__((ext_vector_type(2)));

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kNT = 256;
constexpr int kSub = 16;         // reduction per gathered sub-chunk
constexpr int kKS = 1;           // sub-chunks per LDS stage
constexpr int kBK = kSub * kKS;  // reduction per LDS stage
// The K = (ci, kh, kw) side of grad_input (rows) and grad_weight (columns) is
// tiled by 64 when ci * k * k <= 64 (the 3-channel stem: 48), by 128 otherwise.
constexpr int kNarrowK = 64;
// A workgroup computes a TM x TN tile of the result (TM, TN in {64, 128}).
// LDS rows of an operand tile of width T have a pitch of T + 4 floats (4 mod
// 64 banks).  At MFMA step s the two half-waves read k rows s and s + 8 of a
// sub-chunk (both operands pair k the same way), which 8 * (T + 4) = 32 mod 64
// puts in disjoint banks; and the operand gathers' writes of k rows 4 apart
// (grad_weight's grad_output tile) or 8 apart (the forward's weight tile) land
// 16 or 32 banks apart instead of on one bank.
constexpr int pitch(int width) { return width + 4; }

enum Mode { FWD = 0, BWI = 1, BWW = 2 };

struct PArgs {
    const float* x;       // input X (N, Ci, H, W)           FWD, BWW
    const float* g;       // grad_output G (N, Co, Ho, Wo)   BWI, BWW
    const float* w;       // weight (Co, Ci, s, s)           FWD, BWI
    const float* b;       // bias (Co) or null               FWD
    float* out;           // Y (FWD), dX (BWI), partial slabs (BWW): per split Co * Kt weights then Co biases
    int N, Ci, Co, H, W, Ho, Wo, P, Kt;
    int tiles_m, tiles_n;             // result tiles (columns: pixels of one image for FWD / BWI)
    int splits, chunks;               // BWW: pixel sub-chunks of kSub, split into `splits` ranges
    int with_bias;                    // BWW: also sum grad_output per channel
    float* act;           // FWD, pointwise only: GELU(Y) as well, or null
    const float* pre;     // BWI, pointwise only: dX is scaled by GELU'(pre) (pre shaped like X), or null
    // FWD, BWI: the push form of the next layer's halo exchange (all null: none), for the pushed
    // tensor Y (FWD) or dX (BWI); the halo buffers have rows ph_l + ph_r wide.
    float* push_l;        // left neighbour's halo: this slice's first ph_r columns go to [ph_l, ph_l + ph_r)
    float* push_r;        // right neighbour's halo: this slice's last ph_l columns go to [0, ph_l)
    float* push_own;      // own halo: the side without a neighbour is zeroed
    int ph_l, ph_r;
    // BWW with a single split (dma_bww_kernel): the sums go straight to grad_weight / grad_bias
    float* gw_out;
    float* gb_out;
};

__device__ __forceinline__ int64_t slab_floats(const PArgs& a) { return (int64_t)a.Co * (a.Kt + 1); }

__device__ __forceinline__ bool pushes(const PArgs& a) { return a.push_l || a.push_r || a.push_own; }

// Value v at column j of row (plane, i) of the pushed tensor (rows of w columns, rows_per_plane rows):
// the copies the neighbours' halos need, and the zeros of the own halo's sides that have no
// neighbour (columns j < ph_l stand for the left side's ph_l halo columns, the last ph_r for the
// right side's, so each is written once per row).
__device__ __forceinline__ void push_value(const PArgs& a, int64_t plane, int rows_per_plane, int i, int j, int w,
                                           float v)
{
    const int hw = a.ph_l + a.ph_r;
    const int64_t base = (plane * rows_per_plane + i) * hw;
    if (a.push_l) {
        if (j < a.ph_r) a.push_l[base + a.ph_l + j] = v;                   // left neighbour's right side
    } else if (j < a.ph_l) {
        a.push_own[base + j] = 0.f;                                        // no left neighbour
    }
    if (a.push_r) {
        if (j >= w - a.ph_l) a.push_r[base + (j - (w - a.ph_l))] = v;      // right neighbour's left side
    } else if (j >= w - a.ph_r) {
        a.push_own[base + a.ph_l + (j - (w - a.ph_r))] = 0.f;              // no right neighbour
    }
}

// Global -> registers for one sub-chunk of kSub reduction rows (8 A values
// and 8 B values per thread), then registers -> LDS.  Each mode gathers its
// own operands; a sub-chunk past the end of the reduction (ok_k false) loads
// zeros.
template <int MODE, int S, int TM, int TN>
struct Sub {
    static constexpr int LDA = pitch(TM), LDB = pitch(TN);
    // 64-wide tiles: the output channels of the forward (TM), and the K =
    // (ci, kh, kw) side of grad_input (TM) and grad_weight (TN)
    static_assert((MODE == FWD && TN == 128) || (MODE == BWI && TN == 128) || (MODE == BWW && TM >= 128),
                  "tile shape");
    float ra[TM / 16];       // kSub x TM operand values over 256 threads
    float rb[TN / 16];

    // k0: reduction offset.  FWD: K; BWI: co; BWW: pixel of image img.
    __device__ void load(const PArgs& a, int img, int m0, int n0, int k0, bool ok_k)
    {
        const int t = threadIdx.x;
        if constexpr (MODE == FWD) {
            // A[m][k] = W[m0 + m][k0 + k]: per row 16 contiguous floats, 256 / TM threads a row
            constexpr int TPR = kNT / TM, PER = kSub / TPR;          // threads per row, floats per thread
            const int m = t / TPR, kh = (t % TPR) * PER;
            const bool ok = ok_k && m0 + m < a.Co;
            const float* src = a.w + (int64_t)(m0 + m) * a.Kt + k0 + kh;
#pragma unroll
            for (int v = 0; v < PER / 4; ++v) {
                const float4 q = ok ? *reinterpret_cast<const float4*>(src + 4 * v) : make_float4(0.f, 0.f, 0.f, 0.f);
                ra[4 * v] = q.x; ra[4 * v + 1] = q.y; ra[4 * v + 2] = q.z; ra[4 * v + 3] = q.w;
            }
            // B[k][p] = X[img][ci][i*s + kh][j*s + kw]: item (group, pixel) = s floats
            const float* xi = a.x + (int64_t)img * a.Ci * a.H * a.W;
            if constexpr (S == 1) {
                // 1x1: B[k][p] = X[img][k0 + k][p], 4 consecutive pixels (one row: Wo % 16 == 0) per item
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const int idx = t + kNT * r;
                    const int k = idx / 32, p4 = (idx % 32) * 4;
                    const int pp = n0 + p4;
                    const bool okp = ok_k && pp < a.P;
                    const float4 v = okp ? *reinterpret_cast<const float4*>(xi + (int64_t)(k0 + k) * a.P + pp)
                                         : make_float4(0.f, 0.f, 0.f, 0.f);
                    rb[4 * r] = v.x; rb[4 * r + 1] = v.y; rb[4 * r + 2] = v.z; rb[4 * r + 3] = v.w;
                }
                return;
            }
#pragma unroll
            for (int r = 0; r < 8 / S; ++r) {
                const int idx = t + kNT * r;
                const int gl = idx / TN, p = idx % TN;
                const int gg = k0 / S + gl;                 // global K group = ci * s + kh
                const int ci = gg / S, kh = gg - ci * S;
                const int pp = n0 + p;
                const bool okp = ok_k && pp < a.P;
                const int i = pp / a.Wo, j = pp - i * a.Wo;
                const float* s_ = xi + ((int64_t)ci * a.H + i * S + kh) * a.W + j * S;
                if constexpr (S == 2) {
                    const float2 v = okp ? *reinterpret_cast<const float2*>(s_) : make_float2(0.f, 0.f);
                    rb[2 * r] = v.x; rb[2 * r + 1] = v.y;
                } else {
                    const float4 v = okp ? *reinterpret_cast<const float4*>(s_) : make_float4(0.f, 0.f, 0.f, 0.f);
                    rb[4 * r] = v.x; rb[4 * r + 1] = v.y; rb[4 * r + 2] = v.z; rb[4 * r + 3] = v.w;
                }
            }
        } else if constexpr (MODE == BWI) {
            // A[m][c] = W[k0 + c][m0 + m] (the weight read transposed): rows along m
#pragma unroll
            for (int r = 0; r < TM / 64; ++r) {
                const int idx = t + kNT * r;
                const int c = idx / (TM / 4), m4 = (idx % (TM / 4)) * 4;
                const bool ok = ok_k && m0 + m4 < a.Kt;
                const float4 v = ok ? *reinterpret_cast<const float4*>(a.w + (int64_t)(k0 + c) * a.Kt + m0 + m4)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
                ra[4 * r] = v.x; ra[4 * r + 1] = v.y; ra[4 * r + 2] = v.z; ra[4 * r + 3] = v.w;
            }
            // B[c][p] = G[img][k0 + c][n0 + p]: rows along p
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int idx = t + kNT * r;
                const int c = idx / 32, p4 = (idx % 32) * 4;
                const bool ok = ok_k && n0 + p4 < a.P;
                const float4 v = ok ? *reinterpret_cast<const float4*>(
                                          a.g + ((int64_t)img * a.Co + k0 + c) * a.P + n0 + p4)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
                rb[4 * r] = v.x; rb[4 * r + 1] = v.y; rb[4 * r + 2] = v.z; rb[4 * r + 3] = v.w;
            }
        } else {
            // A[m][q] = G[img][m0 + m][k0 + q]: per row 16 contiguous floats (pixels)
#pragma unroll
            for (int r = 0; r < TM / 64; ++r) {
                const int idx = t + kNT * r;
                const int m = idx / 4, q4 = (idx % 4) * 4;
                const bool ok = ok_k && m0 + m < a.Co;
                const float4 v = ok ? *reinterpret_cast<const float4*>(
                                          a.g + ((int64_t)img * a.Co + m0 + m) * a.P + k0 + q4)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
                ra[4 * r] = v.x; ra[4 * r + 1] = v.y; ra[4 * r + 2] = v.z; ra[4 * r + 3] = v.w;
            }
            // B[q][n] = Xp[n0 + n][k0 + q]: the 16 pixels of the sub-chunk lie in one output row
            const int i = k0 / a.Wo, j0 = k0 - i * a.Wo;
            const float* xi = a.x + (int64_t)img * a.Ci * a.H * a.W;
            if constexpr (S == 1) {
                // 1x1: n is the input channel; 4 consecutive pixels per item
#pragma unroll
                for (int r = 0; r < TN / 64; ++r) {
                    const int idx = t + kNT * r;
                    const int nn = idx / 4, q4 = (idx % 4) * 4;
                    const int ci = n0 + nn;
                    const bool ok = ok_k && ci < a.Kt;
                    const float4 v = ok ? *reinterpret_cast<const float4*>(xi + ((int64_t)ci * a.H + i) * a.W + j0 + q4)
                                        : make_float4(0.f, 0.f, 0.f, 0.f);
                    rb[4 * r] = v.x; rb[4 * r + 1] = v.y; rb[4 * r + 2] = v.z; rb[4 * r + 3] = v.w;
                }
                return;
            }
#pragma unroll
            for (int r = 0; r < TN / (16 * S); ++r) {
                const int idx = t + kNT * r;
                const int q = idx % kSub, gl = idx / kSub;
                const int gg = n0 / S + gl;
                const int ci = gg / S, kh = gg - ci * S;
                const bool ok = ok_k && gg * S < a.Kt;
                const float* s_ = xi + ((int64_t)ci * a.H + i * S + kh) * a.W + (j0 + q) * S;
                if constexpr (S == 2) {
                    const float2 v = ok ? *reinterpret_cast<const float2*>(s_) : make_float2(0.f, 0.f);
                    rb[2 * r] = v.x; rb[2 * r + 1] = v.y;
                } else {
                    const float4 v = ok ? *reinterpret_cast<const float4*>(s_) : make_float4(0.f, 0.f, 0.f, 0.f);
                    rb[4 * r] = v.x; rb[4 * r + 1] = v.y; rb[4 * r + 2] = v.z; rb[4 * r + 3] = v.w;
                }
            }
        }
    }

    // LDS rows of this sub-chunk: As[k][m], Bs[k][n] (k-major rows of pitch LDA, LDB).
    __device__ void put(float* __restrict__ As, float* __restrict__ Bs) const
    {
        const int t = threadIdx.x;
        if constexpr (MODE == FWD) {
            constexpr int TPR = kNT / TM, PER = kSub / TPR;
            const int m = t / TPR, kh = (t % TPR) * PER;
#pragma unroll
            for (int e = 0; e < PER; ++e) As[(kh + e) * LDA + m] = ra[e];
            if constexpr (S == 1) {
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const int idx = t + kNT * r;
                    const int k = idx / 32, p4 = (idx % 32) * 4;
                    *reinterpret_cast<float4*>(Bs + k * LDB + p4) =
                        make_float4(rb[4 * r], rb[4 * r + 1], rb[4 * r + 2], rb[4 * r + 3]);
                }
                return;
            }
#pragma unroll
            for (int r = 0; r < 8 / S; ++r) {
                const int idx = t + kNT * r;
                const int gl = idx / TN, p = idx % TN;
#pragma unroll
                for (int kw = 0; kw < S; ++kw) Bs[(gl * S + kw) * LDB + p] = rb[S * r + kw];
            }
        } else if constexpr (MODE == BWI) {
#pragma unroll
            for (int r = 0; r < TM / 64; ++r) {
                const int idx = t + kNT * r;
                const int c = idx / (TM / 4), x4 = (idx % (TM / 4)) * 4;
                *reinterpret_cast<float4*>(As + c * LDA + x4) = make_float4(ra[4 * r], ra[4 * r + 1], ra[4 * r + 2], ra[4 * r + 3]);
            }
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int idx = t + kNT * r;
                const int c = idx / 32, x4 = (idx % 32) * 4;
                *reinterpret_cast<float4*>(Bs + c * LDB + x4) = make_float4(rb[4 * r], rb[4 * r + 1], rb[4 * r + 2], rb[4 * r + 3]);
            }
        } else {
#pragma unroll
            for (int r = 0; r < TM / 64; ++r) {
                const int idx = t + kNT * r;
                const int m = idx / 4, q4 = (idx % 4) * 4;
#pragma unroll
                for (int e = 0; e < 4; ++e) As[(q4 + e) * LDA + m] = ra[4 * r + e];
            }
            if constexpr (S == 1) {
#pragma unroll
                for (int r = 0; r < TN / 64; ++r) {
                    const int idx = t + kNT * r;
                    const int nn = idx / 4, q4 = (idx % 4) * 4;
#pragma unroll
                    for (int e = 0; e < 4; ++e) Bs[(q4 + e) * LDB + nn] = rb[4 * r + e];
                }
                return;
            }
#pragma unroll
            for (int r = 0; r < TN / (16 * S); ++r) {
                const int idx = t + kNT * r;
                const int q = idx % kSub, gl = idx / kSub;
#pragma unroll
                for (int kw = 0; kw < S; ++kw) Bs[q * LDB + gl * S + kw] = rb[S * r + kw];
            }
        }
    }
};

template <int MODE, int S, int TM, int TN>
__global__ void __launch_bounds__(kNT, 2)
patch_kernel(PArgs a)
{
    using Stage = Sub<MODE, S, TM, TN>;
    constexpr int LDA = Stage::LDA, LDB = Stage::LDB;
    constexpr int XB = TM / 64, YB = TN / 64;    // 32 x 32 MFMA blocks per wave (waves in a 2 x 2 grid)
    __shared__ __align__(16) float As[2][kBK * LDA];
    __shared__ __align__(16) float Bs[2][kBK * LDB];

    // tile -> (img or split, m tile, n tile); m fastest, so workgroups that
    // share the large operand (the pixels) run side by side on one XCD
    int bid = xcd_order(blockIdx.x, gridDim.x);
    const int mt = bid % a.tiles_m;
    bid /= a.tiles_m;
    const int nt = bid % a.tiles_n;
    const int outer = bid / a.tiles_n;           // image (FWD / BWI) or split (BWW)
    const int m0 = mt * TM, n0 = nt * TN;

    // reduction range in sub-chunks of kSub
    int c_beg, c_end;
    if constexpr (MODE == FWD) { c_beg = 0; c_end = a.Kt / kSub; }
    else if constexpr (MODE == BWI) { c_beg = 0; c_end = a.Co / kSub; }
    else {
        c_beg = (int)((int64_t)outer * a.chunks / a.splits);
        c_end = (int)((int64_t)(outer + 1) * a.chunks / a.splits);
    }
    const int nstage = (c_end - c_beg + kKS - 1) / kKS;
    const int cpi = a.P / kSub;                  // BWW: sub-chunks per image

    Stage sub[kKS];
    auto load_stage = [&](int stg) {
#pragma unroll
        for (int u = 0; u < kKS; ++u) {
            const int c = c_beg + stg * kKS + u;
            const bool ok = c < c_end;
            int img, k0;
            if constexpr (MODE == BWW) {
                const int cc = ok ? c : c_beg;
                img = cc / cpi;
                k0 = (cc - img * cpi) * kSub;
            } else {
                img = outer;
                k0 = (ok ? c : 0) * kSub;
            }
            sub[u].load(a, img, m0, n0, k0, ok);
        }
    };

    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int hi = lane >> 5, l32 = lane & 31;
    f32x16 acc[XB][YB];
#pragma unroll
    for (int x = 0; x < XB; ++x)
#pragma unroll
        for (int y = 0; y < YB; ++y)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.f;
    float bias_acc = 0.f;
    const bool with_bias = MODE == BWW && a.with_bias && nt == 0;

    if (nstage > 0) load_stage(0);
    for (int stg = 0; stg < nstage; ++stg) {
        float* as = As[stg & 1];
        float* bs = Bs[stg & 1];
#pragma unroll
        for (int u = 0; u < kKS; ++u) sub[u].put(as + u * kSub * LDA, bs + u * kSub * LDB);
        lds_barrier();
        if (stg + 1 < nstage) load_stage(stg + 1);
        if (with_bias && threadIdx.x < TM) {
#pragma unroll
            for (int q = 0; q < kBK; ++q) bias_acc += as[q * LDA + threadIdx.x];
        }
        // operands of step s2 + 1 are read before the MFMAs of step s2 are
        // issued (the scheduling barriers keep that order), so the LDS
        // latency overlaps the matrix pipe instead of stalling it
        // k-slot pairing of step s2 in sub-chunk u: rows 16 u + s2 (lanes 0..31)
        // and 16 u + s2 + 8 (lanes 32..63)
        const float* ap = as + hi * (kSub / 2) * LDA + wm * (TM / 2) + l32;
        const float* bp = bs + hi * (kSub / 2) * LDB + wn * (TN / 2) + l32;
        auto row = [](int s2) { return (s2 / (kSub / 2)) * kSub + s2 % (kSub / 2); };
        float av[XB], bv[YB];
#pragma unroll
        for (int x = 0; x < XB; ++x) av[x] = ap[32 * x];
#pragma unroll
        for (int y = 0; y < YB; ++y) bv[y] = bp[32 * y];
#pragma unroll
        for (int s2 = 0; s2 < kBK / 2; ++s2) {
            float na[XB], nb[YB];
#pragma unroll
            for (int x = 0; x < XB; ++x) na[x] = s2 + 1 < kBK / 2 ? ap[row(s2 + 1) * LDA + 32 * x] : 0.f;
#pragma unroll
            for (int y = 0; y < YB; ++y) nb[y] = s2 + 1 < kBK / 2 ? bp[row(s2 + 1) * LDB + 32 * y] : 0.f;
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int x = 0; x < XB; ++x)
#pragma unroll
                for (int y = 0; y < YB; ++y)
                    acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[x], bv[y], acc[x][y], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int x = 0; x < XB; ++x) av[x] = na[x];
#pragma unroll
            for (int y = 0; y < YB; ++y) bv[y] = nb[y];
        }
        // the buffer just read is rewritten two stages later, after the next barrier
    }

    // D block (x, y): register 4 q + r holds row 4 hi + 8 q + r, column l32
#pragma unroll
    for (int x = 0; x < XB; ++x)
#pragma unroll
        for (int y = 0; y < YB; ++y) {
            const int rb = m0 + wm * (TM / 2) + x * 32;     // block's first row (a multiple of 4)
            const int col = n0 + wn * (TN / 2) + y * 32 + l32;
            // the lane's pixel, and whether its column (or, for grad_input, one of its s input
            // columns) lies within the pushed halo widths of either edge: only such lanes push
            const int pi = col / a.Wo, pj = col - pi * a.Wo;
            const int pmax = a.ph_l > a.ph_r ? a.ph_l : a.ph_r;
            const int pw = MODE == FWD ? a.Wo : a.W, c0 = MODE == FWD ? pj : pj * S;
            const bool edge = pushes(a) && (c0 < pmax || c0 + (MODE == FWD ? 0 : S - 1) >= pw - pmax);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row = rb + 4 * hi + 8 * q;  // rows row .. row + 3 in registers 4q .. 4q + 3
                if constexpr (MODE == FWD) {
                    if (col < a.P) {
                        float* yp = a.out + ((int64_t)outer * a.Co) * a.P + col;
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (row + r < a.Co) {
                                const float v = acc[x][y][4 * q + r] + (a.b ? a.b[row + r] : 0.f);
                                yp[(int64_t)(row + r) * a.P] = v;
                                if (a.act) a.act[((int64_t)outer * a.Co + row + r) * a.P + col] = gelu(v);
                                if (edge) push_value(a, (int64_t)outer * a.Co + row + r, a.Ho, pi, pj, a.Wo, v);
                            }
                    }
                } else if constexpr (MODE == BWI) {
                    // rows = K = (ci, kh, kw), kw fastest: the 4 registers are s-wide runs of kw
                    if (col < a.P && row < a.Kt) {
                        const int i = col / a.Wo, j = col - i * a.Wo;
                        float* dxi = a.out + (int64_t)outer * a.Ci * a.H * a.W;
                        if constexpr (S == 1) {
                            // rows are input channels: 4 channels of one pixel
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const int64_t o = ((int64_t)(row + r) * a.H + i) * a.W + j;
                                float v = acc[x][y][4 * q + r];
                                if (a.pre) v = v * gelu_grad(a.pre[(int64_t)outer * a.Ci * a.H * a.W + o]);
                                dxi[o] = v;
                                if (edge) push_value(a, (int64_t)outer * a.Ci + row + r, a.H, i, j, a.W, v);
                            }
                        } else if constexpr (S == 4) {
                            const int ci = row / 16, kh = (row / 4) % 4;
                            *reinterpret_cast<float4*>(dxi + ((int64_t)ci * a.H + i * 4 + kh) * a.W + j * 4) =
                                make_float4(acc[x][y][4 * q], acc[x][y][4 * q + 1], acc[x][y][4 * q + 2],
                                            acc[x][y][4 * q + 3]);
                            if (edge) {
#pragma unroll
                                for (int kw = 0; kw < 4; ++kw)
                                    push_value(a, (int64_t)outer * a.Ci + ci, a.H, i * 4 + kh, j * 4 + kw, a.W,
                                               acc[x][y][4 * q + kw]);
                            }
                        } else {
#pragma unroll
                            for (int h = 0; h < 2; ++h) {
                                const int rr = row + 2 * h;
                                const int ci = rr / 4, kh = (rr / 2) % 2;
                                *reinterpret_cast<float2*>(dxi + ((int64_t)ci * a.H + i * 2 + kh) * a.W + j * 2) =
                                    make_float2(acc[x][y][4 * q + 2 * h], acc[x][y][4 * q + 2 * h + 1]);
                                if (edge) {
#pragma unroll
                                    for (int kw = 0; kw < 2; ++kw)
                                        push_value(a, (int64_t)outer * a.Ci + ci, a.H, i * 2 + kh, j * 2 + kw, a.W,
                                                   acc[x][y][4 * q + 2 * h + kw]);
                                }
                            }
                        }
                    }
                } else {
                    if (col < a.Kt) {
                        float* wp = a.out + outer * slab_floats(a) + col;
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (row + r < a.Co) wp[(int64_t)(row + r) * a.Kt] = acc[x][y][4 * q + r];
                    }
                }
            }
        }
    if (with_bias && threadIdx.x < TM && m0 + threadIdx.x < a.Co)
        a.out[outer * slab_floats(a) + (int64_t)a.Co * a.Kt + m0 + threadIdx.x] = bias_acc;
}

// Forward of a 2x2/2 layer in wide tiles.  The product runs over the pixels
// of all the images at once, in result tiles of 128 output channels x 32 NB
// pixels (NB MFMA blocks of 32) that may straddle two images: the
// ConvNeXt-style stack's downsamples have 7 x 2^j output pixels per channel,
// so 224-pixel tiles (NB = 7) divide them into a whole multiple of the CU
// count, where 128-pixel tiles per image leave the last round of workgroups
// partly empty.  Where 224-pixel tiles are fewer than the CUs (the deepest
// downsample of a narrow shard: 128 tiles), 128-pixel tiles (NB = 4) give
// each CU at most one tile of 4/7 the work.  Wave w computes rows
// 32 w .. 32 w + 31 of the tile against all NB pixel blocks.  A stage is 4 input channels (16 reduction rows), loaded from HBM
// straight into LDS (buffer_load ... lds, no registers) one stage ahead:
//   A  W[m0 + m][(4 c .. 4 c + 3) + 16 s]: 16-byte units, unit (m, c) at
//      slot m * 4 + (c ^ ((m >> 2) & 3)) (the swizzle spreads a wave's reads
//      of one c over the banks);
//   B  per (c, kh), the input rows 2 i + kh of the tile's pixels as they lie
//      in memory: pixel n's two columns kw at 2 n + kw of a 512-float segment.
// MFMA step (c, kh) pairs k-slot 0 with kw = 0 and k-slot 1 with kw = 1, so
// the B operand of lane (hi, n) is segment word 2 n + hi (64 consecutive
// words per wave) and the A operand is word 2 kh + hi of unit (m, c).
constexpr int kWideTM = 128, kWideNB = 7, kWideTN = 32 * kWideNB, kWideSeg = 512;
constexpr int kWideAF = kWideTM * 16, kWideBF = 8 * kWideSeg, kWideST = kWideAF + kWideBF;

// KS = 2 (launches with no more tiles than CUs, where one 256-thread
// workgroup per CU would leave one wave per SIMD): 512 threads, whose halves
// take the even and the odd stages, each with its own two stage buffers;
// at the end the second half hands its sums to the first through LDS and the
// first adds them (the same order for every tile) and stores.
template <int NB, int KS>
__global__ void __launch_bounds__(kNT * KS, KS == 1 ? 3 : 2)
wide_fwd_kernel(PArgs a, int ntot)
{
    constexpr int TN = 32 * NB;                  // the tile's pixels
    constexpr int NH = (2 * TN + 255) / 256;     // 64-lane B loads per (channel, kh): 256 floats each
    static_assert(NB <= kWideNB, "B segments hold 512 floats");
    static_assert(KS == 1 || KS == 2, "one or two reduction halves");
    __shared__ __align__(16) float lds[2 * KS * kWideST];
    __shared__ float bias_s[kWideTM];
    const int bid = xcd_order(blockIdx.x, gridDim.x);   // output-channel tiles of one pixel tile side by side
    const int mt = bid % a.tiles_m, nt = bid / a.tiles_m;
    const int m0 = mt * kWideTM, n0 = nt * TN;
    const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane((t >> 6) & 3);
    const int half = KS == 1 ? 0 : __builtin_amdgcn_readfirstlane(t >> 8);
    if (t < kWideTM) bias_s[t] = (a.b && m0 + t < a.Co) ? a.b[m0 + t] : 0.f;
    const int nstage = a.Ci / 4;
    const int njs = (nstage + KS - 1) / KS;       // iterations; iteration j is stage KS j + half

    // A: instruction i of wave w covers LDS units 64 (2 w + i) + lane
    const i32x4 ra = plane_rsrc(a.w, a.Co * a.Kt * 4);
    int avoff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int m = 16 * (2 * wave + i) + lane / 4;
        const int c = (lane & 3) ^ ((m >> 2) & 3);
        avoff[i] = ((m0 + m) * a.Kt + 4 * c) * 4;
    }
    // B: wave w loads channel 4 s + w, rows kh = 0, 1, in two halves of 64 units (pixel pairs);
    // pixels past the tile or past the last image read as zeros
    const i32x4 rb = plane_rsrc(a.x, a.N * a.Ci * a.H * a.W * 4);
    int bvoff[NH][2];
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
        const int n = 2 * (64 * hf + lane);
        const int gp = n0 + n;
        const int img = gp / a.P, pl = gp - img * a.P;
        const int i = pl / a.Wo, j = pl - i * a.Wo;
        const bool ok = n < TN && gp < ntot;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
            bvoff[hf][kh] = ok ? (((img * a.Ci + wave) * a.H + 2 * i + kh) * a.W + 2 * j) * 4 : (int)0x80000000;
    }
    const int a_step = 64, b_step = 4 * a.H * a.W * 4;
    // stage KS j + half into this half's buffer j & 1
    auto issue = [&](int j) {
        const int s = KS * j + half;
        float* st = lds + (2 * half + (j & 1)) * kWideST;
#pragma unroll
        for (int i = 0; i < 2; ++i) dma16(ra, st + (2 * wave + i) * 256, avoff[i] + s * a_step);
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int hf = 0; hf < NH; ++hf)
                dma16(rb, st + kWideAF + (2 * wave + kh) * kWideSeg + 256 * hf, bvoff[hf][kh] + s * b_step);
    };

    const int hi = lane >> 5, l32 = lane & 31;
    f32x16 acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[b][r] = 0.f;
    const int sw = (l32 >> 2) & 3;
    const int arow = (32 * wave + l32) * 4;
    const int boff = kWideAF + 2 * l32 + hi;

    if (half < nstage) issue(0);
    for (int j = 0; j < njs; ++j) {
        // iteration j's stage has landed (this wave's loads, then everyone's); the other buffer is free
        wait_vmem();
        lds_barrier();
        if (KS * (j + 1) + half < nstage) issue(j + 1);
        if (KS * j + half >= nstage) continue;   // the second half's last iteration when nstage is odd
        const float* st = lds + (2 * half + (j & 1)) * kWideST;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int ao = (arow + (c ^ sw)) * 4 + hi;
            const float a0 = st[ao], a1 = st[ao + 2];
            float b0[NB], b1[NB];
#pragma unroll
            for (int yb = 0; yb < NB; ++yb) {
                b0[yb] = st[boff + (2 * c) * kWideSeg + 64 * yb];
                b1[yb] = st[boff + (2 * c + 1) * kWideSeg + 64 * yb];
            }
#pragma unroll
            for (int yb = 0; yb < NB; ++yb)
                acc[yb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0[yb], acc[yb], 0, 0, 0);
#pragma unroll
            for (int yb = 0; yb < NB; ++yb)
                acc[yb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1[yb], acc[yb], 0, 0, 0);
        }
    }
    if constexpr (KS == 2) {
        // the odd stages' sums into the first half: up to 4 blocks per lane and round, laid out
        // [wave][block][register][lane] so that a wave's 64 lanes write and read 64 consecutive floats
        lds_barrier();   // every wave is past its last products; the stage buffers are free
#pragma unroll
        for (int r0 = 0; r0 < NB; r0 += 4) {
            if (half == 1) {
#pragma unroll
                for (int yb = r0; yb < NB && yb < r0 + 4; ++yb)
#pragma unroll
                    for (int k = 0; k < 16; ++k) lds[((wave * 4 + yb - r0) * 16 + k) * 64 + lane] = acc[yb][k];
            }
            lds_barrier();
            if (half == 0) {
#pragma unroll
                for (int yb = r0; yb < NB && yb < r0 + 4; ++yb)
#pragma unroll
                    for (int k = 0; k < 16; ++k) acc[yb][k] += lds[((wave * 4 + yb - r0) * 16 + k) * 64 + lane];
            }
            lds_barrier();
        }
        if (half == 1) return;
    }

    // D block yb: register 4 q + r holds row 8 q + 4 hi + r of the wave's 32, column l32
    const int pmax = a.ph_l > a.ph_r ? a.ph_l : a.ph_r;
#pragma unroll
    for (int yb = 0; yb < NB; ++yb) {
        const int gp = n0 + 32 * yb + l32;
        if (gp >= ntot) continue;
        const int img = gp / a.P, pl = gp - img * a.P;
        const int pi = pl / a.Wo, pj = pl - pi * a.Wo;
        const bool edge = pushes(a) && (pj < pmax || pj >= a.Wo - pmax);
        float* yp = a.out + (int64_t)img * a.Co * a.P + pl;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + 32 * wave + 8 * q + 4 * hi + r;
                if (row < a.Co) {
                    const float v = acc[yb][4 * q + r] + bias_s[row - m0];
                    __builtin_nontemporal_store(v, yp + (int64_t)row * a.P);
                    if (edge) push_value(a, (int64_t)img * a.Co + row, a.Ho, pi, pj, a.Wo, v);
                }
            }
    }
}

// grad_input of a 2x2/2 layer in wide tiles: dXp[K][p] = sum_co W[co][K]
// G[co][p] over the pixels of all the images, result tiles of 128 rows of
// K = (ci, kh, kw) x 224 pixels, 16 output channels (reduction rows) per
// stage, loaded straight into LDS one stage ahead.  Both operands are rows of
// memory that are contiguous along the tile's own index (W rows along K,
// grad_output rows along the pixels), so LDS holds them k-major:
//   A  16 rows of 128 floats, W[k0 + kr][m0 .. m0 + 127];
//   B  16 rows of 256 floats, G[co = k0 + kr][the tile's 224 pixels] (the
//      last 32 floats zero);
// 16-byte unit u of row kr sits at slot u ^ (8 (kr >> 3 & 1)).  MFMA step t
// pairs k-slot 0 with row t and k-slot 1 with row t + 8, whose slots the
// swizzle puts 32 banks apart, so a wave's 64 reads of one step never share a
// bank.  The result's rows come in groups of 4 = (kh, kw) of one input
// channel: each lane scatters two 2-float runs back to NCHW.
constexpr int kWiBF = 16 * 256, kWiAF = 16 * kWideTM, kWiST = kWiAF + kWiBF;

__global__ void __launch_bounds__(kNT, 3)
wide_bwi_kernel(PArgs a, int ntot)
{
    __shared__ __align__(16) float lds[2 * kWiST];
    const int bid = xcd_order(blockIdx.x, gridDim.x);   // K tiles of one pixel tile side by side
    const int mt = bid % a.tiles_m, nt = bid / a.tiles_m;
    const int m0 = mt * kWideTM, n0 = nt * kWideTN;
    const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int nstage = a.Co / 16;

    // A: instruction i of wave w fills rows kr = 2 (2 w + i) + lane / 32; lane's slot lane % 32
    const i32x4 ra = plane_rsrc(a.w, a.Co * a.Kt * 4);
    int avoff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int kr = 2 * (2 * wave + i) + lane / 32;
        const int u = (lane & 31) ^ (8 * ((kr >> 3) & 1));
        const int m = m0 + 4 * u;
        avoff[i] = m < a.Kt ? (kr * a.Kt + m) * 4 : (int)0x80000000;
    }
    // B: wave w fills rows kr = 4 w .. 4 w + 3, one instruction each; lane's slot lane
    const i32x4 rb = plane_rsrc(a.g, a.N * a.Co * a.P * 4);
    int bvoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int kr = 4 * wave + i;
        const int n = 4 * (lane ^ (8 * ((kr >> 3) & 1)));
        const int gp = n0 + n;
        const int img = gp / a.P, pl = gp - img * a.P;
        bvoff[i] = (n < kWideTN && gp < ntot) ? (((img * a.Co) + kr) * a.P + pl) * 4 : (int)0x80000000;
    }
    const int a_step = 16 * a.Kt * 4, b_step = 16 * a.P * 4;
    auto issue = [&](int s) {
        float* st = lds + (s & 1) * kWiST;
#pragma unroll
        for (int i = 0; i < 2; ++i) dma16(ra, st + (2 * wave + i) * 256, avoff[i] + s * a_step);
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16(rb, st + kWiAF + (4 * wave + i) * 256, bvoff[i] + s * b_step);
    };

    const int hi = lane >> 5, l32 = lane & 31;
    f32x16 acc[kWideNB];
#pragma unroll
    for (int b = 0; b < kWideNB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[b][r] = 0.f;
    // lane's A word in row t + 8 hi: m = 32 w + l32 at slot (m >> 2) ^ 8 hi; its B word for pixel
    // block yb: n = 32 yb + l32 at slot (n >> 2) ^ 8 hi, i.e. word 32 (yb ^ hi) + l32
    const int aw = 4 * (((32 * wave + l32) >> 2) ^ (8 * hi)) + (l32 & 3) + 8 * hi * 128;
    int bw[kWideNB];
#pragma unroll
    for (int yb = 0; yb < kWideNB; ++yb) bw[yb] = kWiAF + 8 * hi * 256 + 32 * (yb ^ hi) + l32;

    issue(0);
    for (int s = 0; s < nstage; ++s) {
        wait_vmem();
        lds_barrier();
        if (s + 1 < nstage) issue(s + 1);
        const float* st = lds + (s & 1) * kWiST;
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
            const float av = st[aw + tt * 128];
            float bv[kWideNB];
#pragma unroll
            for (int yb = 0; yb < kWideNB; ++yb) bv[yb] = st[bw[yb] + tt * 256];
#pragma unroll
            for (int yb = 0; yb < kWideNB; ++yb)
                acc[yb] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv[yb], acc[yb], 0, 0, 0);
        }
    }

    // D block yb: register 4 q + r holds K row 32 w + 8 q + 4 hi + r, pixel column l32;
    // K = 4 ci + 2 kh + kw, so registers 4 q .. 4 q + 3 are (kh, kw) of one input channel
    const int pmax = a.ph_l > a.ph_r ? a.ph_l : a.ph_r;
#pragma unroll
    for (int yb = 0; yb < kWideNB; ++yb) {
        const int gp = n0 + 32 * yb + l32;
        if (gp >= ntot) continue;
        const int img = gp / a.P, pl = gp - img * a.P;
        const int i = pl / a.Wo, j = pl - i * a.Wo;
        const bool edge = pushes(a) && (2 * j < pmax || 2 * j + 1 >= a.W - pmax);
        float* dxi = a.out + (int64_t)img * a.Ci * a.H * a.W;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int row = m0 + 32 * wave + 8 * q + 4 * hi;
            if (row >= a.Kt) continue;
            const int ci = row / 4;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const float v0 = acc[yb][4 * q + 2 * kh], v1 = acc[yb][4 * q + 2 * kh + 1];
                const f2v v01 = {v0, v1};
                __builtin_nontemporal_store(v01, reinterpret_cast<f2v*>(dxi + ((int64_t)ci * a.H + 2 * i + kh) * a.W + 2 * j));
                if (edge) {
                    push_value(a, (int64_t)img * a.Ci + ci, a.H, 2 * i + kh, 2 * j, a.W, v0);
                    push_value(a, (int64_t)img * a.Ci + ci, a.H, 2 * i + kh, 2 * j + 1, a.W, v1);
                }
            }
        }
    }
}

// grad_weight of a 2x2/2 layer with its operands loaded straight into LDS:
// gW[co][K] = sum_p G[co][p] Xp[K][p] over the pixels of all the images,
// result tiles of 128 output channels x 128 of K = (ci, kh, kw).  The pixel
// reduction is split into `splits` ranges of 16-pixel chunks (a chunk lies in
// one output row of one image), so that tiles x splits is a multiple of the
// CU count; with one split the sums go straight to grad_weight, otherwise to
// per-split slabs that slab_sum_kernel adds in split order.  A stage is two
// chunks (64 KB of LDS for the two stages in flight, which the two
// workgroups per CU that the split count aims for still fit; against one
// chunk per stage, half the barriers per product: c5 downsample backward
// 978/939/919 -> 953/930/908 us, one GPU), loaded one stage ahead; each
// chunk's operands:
//   A  G[img][m0 + m][the chunk's 16 pixels]: 128 rows of 4 units, unit u of
//      row m at slot u ^ ((m >> 2) & 3);
//   B  x[img][ci][2 i + kh][2 j0 .. 2 j0 + 31] for the tile's 32 input
//      channels and kh = 0, 1, as they lie in memory (pixel pairs x kw):
//      64 segments of 8 units, unit u of segment sg = 2 ci + kh at slot
//      u ^ ((sg >> 1) & 7).
// Step group tg (4 MFMA steps e) pairs k-slot 0 with pixel 8 tg + e and
// k-slot 1 with pixel 8 tg + 4 + e: lane (hi, m) reads unit 2 tg + hi of its
// A row with one 16-byte read, lane (hi, n = 4 ci + 2 kh + kw) words kw and
// kw + 2 of units 4 tg + 2 hi and 4 tg + 2 hi + 1 of its B segment.  The
// swizzles keep both kinds of read off shared banks.  grad_bias: the first K
// tile's threads t < 128 add row t of each A stage.
constexpr int kBwwAF = 128 * 16, kBwwBF = 64 * 32, kBwwST = kBwwAF + kBwwBF;

__global__ void __launch_bounds__(kNT, 2)
dma_bww_kernel(PArgs a)
{
    constexpr int CPS = 2;   // chunks per stage
    __shared__ __align__(16) float lds[2 * CPS * kBwwST];
    int bid = xcd_order(blockIdx.x, gridDim.x);   // output-channel tiles of one (K tile, split) side by side
    const int mt = bid % a.tiles_m;
    bid /= a.tiles_m;
    const int nt = bid % a.tiles_n;
    const int split = bid / a.tiles_n;
    const int m0 = mt * 128, n0 = nt * 128;
    const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int c_beg = (int)((int64_t)split * a.chunks / a.splits);
    const int nst = (int)((int64_t)(split + 1) * a.chunks / a.splits) - c_beg;

    const i32x4 ra = plane_rsrc(a.g, a.N * a.Co * a.P * 4);
    const i32x4 rb = plane_rsrc(a.x, a.N * a.Ci * a.H * a.W * 4);
    int avoff[2], bvoff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int pos = 64 * (2 * wave + i) + lane;
        const int m = pos >> 2, u = (pos & 3) ^ ((m >> 2) & 3);
        avoff[i] = m0 + m < a.Co ? ((m0 + m) * a.P + 4 * u) * 4 : (int)0x80000000;
        const int sg = pos >> 3, ub = (pos & 7) ^ ((sg >> 1) & 7);
        const int ci = n0 / 4 + sg / 2, kh = sg & 1;
        bvoff[i] = ci < a.Ci ? ((ci * a.H + kh) * a.W + 4 * ub) * 4 : (int)0x80000000;
    }
    // chunk c: its first pixel's image, row and column give the two operands' byte offsets
    auto issue = [&](int s) {          // stage s: chunks CPS s .. CPS s + CPS - 1 (those below nst)
#pragma unroll
        for (int cc = 0; cc < CPS; ++cc) {
            const int ch = CPS * s + cc;
            if (ch >= nst) break;
            const int gp = 16 * (c_beg + ch);
            const int img = gp / a.P, pl = gp - img * a.P;
            const int i = pl / a.Wo, j0 = pl - i * a.Wo;
            const int abase = (img * a.Co * a.P + pl) * 4;
            const int bbase = ((img * a.Ci * a.H + 2 * i) * a.W + 2 * j0) * 4;
            float* st = lds + ((s & 1) * CPS + cc) * kBwwST;
#pragma unroll
            for (int k = 0; k < 2; ++k) dma16(ra, st + (2 * wave + k) * 256, avoff[k] + abase);
#pragma unroll
            for (int k = 0; k < 2; ++k) dma16(rb, st + kBwwAF + (2 * wave + k) * 256, bvoff[k] + bbase);
        }
    };

    const int hi = lane >> 5, l32 = lane & 31;
    const int wm = wave >> 1, wn = wave & 1;
    f32x16 acc[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.f;
    float bias_acc = 0.f;
    const bool with_bias = a.with_bias && nt == 0;
    const int asw = (l32 >> 2) & 3, bsw = (l32 >> 2) & 7;
    // lane's B segment (n = 64 wn + 32 yb + l32): 2 (n >> 2) + ((n >> 1) & 1), word kw = n & 1
    int bseg[2];
#pragma unroll
    for (int y = 0; y < 2; ++y) {
        const int n = 64 * wn + 32 * y + l32;
        bseg[y] = kBwwAF + 32 * (2 * (n >> 2) + ((n >> 1) & 1)) + (n & 1);
    }

    const int nstg = (nst + CPS - 1) / CPS;
    if (nstg > 0) issue(0);
    for (int s = 0; s < nstg; ++s) {
        wait_vmem();
        lds_barrier();
        if (s + 1 < nstg) issue(s + 1);
#pragma unroll
        for (int cc = 0; cc < CPS; ++cc) {
            if (CPS * s + cc >= nst) break;
            const float* st = lds + ((s & 1) * CPS + cc) * kBwwST;
            if (with_bias && t < 128) {
                const int bs = (t >> 2) & 3;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float4 v = *reinterpret_cast<const float4*>(st + 16 * t + 4 * (u ^ bs));
                    bias_acc += v.x; bias_acc += v.y; bias_acc += v.z; bias_acc += v.w;
                }
            }
#pragma unroll
            for (int tg = 0; tg < 2; ++tg) {
                float4 av[2];
#pragma unroll
                for (int x = 0; x < 2; ++x)
                    av[x] = *reinterpret_cast<const float4*>(st + 16 * (64 * wm + 32 * x + l32) + 4 * ((2 * tg + hi) ^ asw));
                float bv[2][4];
#pragma unroll
                for (int y = 0; y < 2; ++y)
#pragma unroll
                    for (int d = 0; d < 2; ++d) {
                        const float* bp = st + bseg[y] + 4 * ((4 * tg + 2 * hi + d) ^ bsw);
                        bv[y][2 * d] = bp[0];
                        bv[y][2 * d + 1] = bp[2];
                    }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float a0 = e == 0 ? av[0].x : e == 1 ? av[0].y : e == 2 ? av[0].z : av[0].w;
                    const float a1 = e == 0 ? av[1].x : e == 1 ? av[1].y : e == 2 ? av[1].z : av[1].w;
#pragma unroll
                    for (int y = 0; y < 2; ++y) {
                        acc[0][y] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, bv[y][e], acc[0][y], 0, 0, 0);
                        acc[1][y] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, bv[y][e], acc[1][y], 0, 0, 0);
                    }
                }
            }
        }
    }

    float* wo = a.splits == 1 ? a.gw_out : a.out + split * slab_floats(a);
    float* bo = a.splits == 1 ? a.gb_out : a.out + split * slab_floats(a) + (int64_t)a.Co * a.Kt;
    // D block (x, y): register 4 q + r holds row 8 q + 4 hi + r, column l32
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) {
            const int col = n0 + 64 * wn + 32 * y + l32;
            if (col >= a.Kt) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = m0 + 64 * wm + 32 * x + 8 * q + 4 * hi + r;
                    if (row < a.Co) wo[(int64_t)row * a.Kt + col] = acc[x][y][4 * q + r];
                }
        }
    if (with_bias && t < 128 && m0 + t < a.Co && bo) bo[m0 + t] = bias_acc;
}

// Forward of a 4x4/4 stem (k = s = 4, CI input channels, 16 CI <= 64
// reduction rows, at most 256 output channels, a multiple of 8).  Its reduction is too short
// to amortise staging a weight tile per pixel tile, so each workgroup of 8
// waves keeps the weights in registers (wave w: output channels 32 w .. 32 w
// + 31, as the MFMA A operand of all 8 CI k-steps) and walks pixel tiles of
// 64 (persistent: tile blockIdx.x, then + gridDim.x, ...).  A tile's input --
// for each of the 4 CI rows (ci, kh) of its pixels, the 4 columns kw of each
// pixel (16 bytes) -- is loaded straight into LDS one tile ahead, one row per
// instruction with lane = pixel.  MFMA step (ci, kh, kwp) pairs k-slot 0 with
// kw = kwp and k-slot 1 with kw = kwp + 2, so one 8-byte read per lane and
// row serves two steps.  The epilogue stores 32 consecutive pixels per row
// and instruction through a buffer resource (row offsets in scalar
// registers, no store under a per-lane branch but the push's); the push
// form's halo writes run only for the lanes holding edge columns, after the
// block's stores.  A tile's stores are issued after the next tile's barrier:
// a wave's wait for its next tile's input also waits for its own stores (one
// vector-memory counter), so storing right after the products would put the
// whole drain of the stores under that wait.
constexpr int kStemNT = 512;

template <int CI, bool PUSH>
__global__ void __launch_bounds__(kStemNT, 4)
stem_fwd_kernel(PArgs a, int ntot)
{
    constexpr int ROWS = 4 * CI, TN = 64, SEG = 4 * TN, KS = 8 * CI;
    __shared__ __align__(16) float xs[2][ROWS * SEG];
    __shared__ __align__(16) float bias_s[256];
    const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int hi = lane >> 5, l32 = lane & 31;
    const int ntiles = (ntot + TN - 1) / TN;

    const i32x4 rx = plane_rsrc(a.x, a.N * CI * a.H * a.W * 4);
    // pixel tile -> its 64 pixels, one per lane, in the DMA; row r by wave r % 8
    auto issue = [&](int tile, int buf) {
        const int gp = tile * TN + lane;
        const int img = gp / a.P, pl = gp - img * a.P;
        const int i = pl / a.Wo, j = pl - i * a.Wo;
        const int base = gp < ntot ? (((img * CI) * a.H + 4 * i) * a.W + 4 * j) * 4 : (int)0x80000000;
#pragma unroll
        for (int r = wave; r < ROWS; r += 8) {
            const int ci = r / 4, kh = r % 4;
            dma16_lds(rx, (lds_float*)&xs[buf][r * SEG], base + ((ci * a.H + kh) * a.W) * 4);
        }
    };

    int tile = blockIdx.x;
    // the lane's weights (A operand): step (ci, kh, kwp) of row m = W[m][16 ci + 4 kh + kwp + 2 hi]
    const int m = 32 * wave + l32;
    float wa[KS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        float2 v = make_float2(0.f, 0.f);
        if (m < a.Co) v = *reinterpret_cast<const float2*>(a.w + (int64_t)m * a.Kt + 4 * r + 2 * hi);
        wa[2 * r] = v.x;
        wa[2 * r + 1] = v.y;
    }
    if (t < 256) bias_s[t] = (a.b && t < a.Co) ? a.b[t] : 0.f;
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(a.out, 0, a.N * a.Co * a.P * 4, 0x00020000);
    const int hbytes = a.N * a.Co * a.Ho * (a.ph_l + a.ph_r) * 4;
    const __amdgpu_buffer_rsrc_t hl = __builtin_amdgcn_make_buffer_rsrc(a.push_l, 0, a.push_l ? hbytes : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc(a.push_r, 0, a.push_r ? hbytes : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t hown = __builtin_amdgcn_make_buffer_rsrc(a.push_own, 0, a.push_own ? hbytes : 0, 0x00020000);
    const int pmax = a.ph_l > a.ph_r ? a.ph_l : a.ph_r;
    constexpr int kOut = (int)0x80000000;     // an offset beyond every buffer here: the store drops

    // One tile's results.  D block y: register 4 q + r holds channel 32 w + 8 q + 4 hi + r, pixel
    // 32 y + l32.  Stored through a buffer resource: the lane's part of the offset (image, 4 hi,
    // pixel) in a vector register, the channel's part 4 P (32 w + 8 q + r) in a scalar one.  Lanes
    // past the last pixel take an offset the buffer drops; the output channel count is a multiple
    // of 8, so whether channels 32 w + 8 q .. + 7 exist is the same for the whole wave.
    // The lane's 16 channels (32 w + 8 q + 4 hi + r at [4 q + r]) take their biases from LDS in four
    // 16-byte reads per tile; the bias is added in place (the accumulators are cleared after the
    // stores), so the halo pushes reuse the sums instead of holding a second copy of them.
    auto store_tile = [&](int tl, f32x16 (&ac)[2]) {
        float bl[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 v = *reinterpret_cast<const float4*>(&bias_s[32 * wave + 8 * q + 4 * hi]);
            bl[4 * q] = v.x; bl[4 * q + 1] = v.y; bl[4 * q + 2] = v.z; bl[4 * q + 3] = v.w;
        }
#pragma unroll
        for (int y = 0; y < 2; ++y) {
            const int gp = tl * TN + 32 * y + l32;
            const bool live = gp < ntot;
            const int img = gp / a.P, pl = gp - img * a.P;
            const int voff = live ? ((img * a.Co + 4 * hi) * a.P + pl) * 4 : kOut;
#pragma unroll
            for (int k = 0; k < 16; ++k) ac[y][k] += bl[k];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (32 * wave + 8 * q >= a.Co) continue;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int cu = 32 * wave + 8 * q + r;
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ac[y][4 * q + r]), ry, voff, cu * a.P * 4,
                                                          kNonTemporal);
                }
            }
            if (PUSH) {
                // the push of push_value, through buffer resources (a missing buffer has no
                // records, so its stores drop): the lane's column offsets into the left and right
                // neighbours' halos and its own halo's two zeroed sides (or out of range)
                const int pi = pl / a.Wo, pj = pl - pi * a.Wo;
                if (live && (pj < pmax || pj >= a.Wo - pmax)) {
                    const int hw = a.ph_l + a.ph_r;
                    const int row0 = ((img * a.Co + 4 * hi) * a.Ho + pi) * hw;
                    const int ol = a.push_l ? (pj < a.ph_r ? (row0 + a.ph_l + pj) * 4 : kOut)
                                            : (pj < a.ph_l ? (row0 + pj) * 4 : kOut);
                    const int rj = pj - (a.Wo - a.ph_l), oj = pj - (a.Wo - a.ph_r);
                    const int orr = a.push_r ? (rj >= 0 ? (row0 + rj) * 4 : kOut)
                                             : (oj >= 0 ? (row0 + a.ph_l + oj) * 4 : kOut);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if (32 * wave + 8 * q >= a.Co) continue;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int cu = 32 * wave + 8 * q + r;
                            const float v = ac[y][4 * q + r];
                            const int so = cu * a.Ho * hw * 4;
                            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a.push_l ? v : 0.f),
                                                                  a.push_l ? hl : hown, ol, so, 0);
                            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a.push_r ? v : 0.f),
                                                                  a.push_r ? hr : hown, orr, so, 0);
                        }
                    }
                }
            }
        }
    };

    // A tile's results are stored after the next tile's barrier, so that the stores drain while
    // the waves compute that tile instead of under the wait for its input.
    if (tile < ntiles) issue(tile, 0);
    f32x16 acc[2];
    int prev = -1;
    for (int it = 0; tile < ntiles; ++it, tile += gridDim.x) {
        const int buf = it & 1;
        wait_vmem();
        lds_barrier();
        if (prev >= 0) store_tile(prev, acc);
        __builtin_amdgcn_sched_barrier(0);   // the stores read acc before it is cleared
        if (tile + (int)gridDim.x < ntiles) issue(tile + gridDim.x, buf ^ 1);
#pragma unroll
        for (int y = 0; y < 2; ++y)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[y][r] = 0.f;
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            float2 bv[2];
#pragma unroll
            for (int y = 0; y < 2; ++y)
                bv[y] = *reinterpret_cast<const float2*>(&xs[buf][r * SEG + 4 * (32 * y + l32) + 2 * hi]);
#pragma unroll
            for (int y = 0; y < 2; ++y) {
                acc[y] = __builtin_amdgcn_mfma_f32_32x32x2f32(wa[2 * r], bv[y].x, acc[y], 0, 0, 0);
                acc[y] = __builtin_amdgcn_mfma_f32_32x32x2f32(wa[2 * r + 1], bv[y].y, acc[y], 0, 0, 0);
            }
        }
        prev = tile;
    }
    if (prev >= 0) store_tile(prev, acc);
}

// grad_input of the 4x4/4 stem on 3 channels (K = 48): dXp[K][p] =
// sum_co W[co][K] G[co][p] over the pixels of all the images, in tiles of all
// 48 rows of K x 128 pixels, 16 output channels (reduction rows) per stage,
// loaded straight into LDS one stage ahead.  16 x 16 x 4 MFMA blocks fit K =
// 48 exactly; wave w owns pixel blocks 2 w, 2 w + 1 and all three K blocks.
//   A  W[k0 .. k0 + 15][0 .. 47] as it lies in memory (rows 48 floats apart,
//      which puts a step's 4 rows in different banks);
//   B  G[k0 + kr][the tile's 128 pixels], 16-byte unit u of row kr at slot
//      u ^ 4 (kr & 3), so a step's 4 rows x 16 pixels hit distinct banks.
// The 4 registers of a lane are kw = 0..3 of one (ci, kh, pixel): one 16-byte
// store each.
constexpr int kSiTN = 128, kSiAF = 16 * 48, kSiBF = 16 * kSiTN, kSiST = kSiAF + kSiBF;

__global__ void __launch_bounds__(kNT, 4)
stem_bwi_kernel(PArgs a, int ntot)
{
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    __shared__ __align__(16) float lds[2 * kSiST];
    const int n0 = blockIdx.x * kSiTN;
    const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int l16 = lane & 15, lq = lane >> 4;
    const int nstage = a.Co / 16;

    // A: 768 floats per stage = 3 instructions (waves 0-2); B: 16 rows of 32 units = 8 instructions, 2 per wave
    const i32x4 ra = plane_rsrc(a.w, a.Co * 48 * 4);
    const i32x4 rb = plane_rsrc(a.g, a.N * a.Co * a.P * 4);
    int bvoff[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int pos = 64 * (2 * wave + k) + lane;
        const int kr = pos >> 5, u = (pos & 31) ^ (4 * (kr & 3));
        const int gp = n0 + 4 * u;
        const int img = gp / a.P, pl = gp - img * a.P;
        bvoff[k] = gp < ntot ? ((img * a.Co + kr) * a.P + pl) * 4 : (int)0x80000000;
    }
    auto issue = [&](int s) {
        float* st = lds + (s & 1) * kSiST;
        if (wave < 3) dma16(ra, st + wave * 256, (s * 16 * 48 + 4 * (64 * wave + lane)) * 4);
#pragma unroll
        for (int k = 0; k < 2; ++k) dma16(rb, st + kSiAF + (2 * wave + k) * 256, bvoff[k] + s * 16 * a.P * 4);
    };

    f32x4 acc[3][2];
#pragma unroll
    for (int m = 0; m < 3; ++m)
#pragma unroll
        for (int h = 0; h < 2; ++h) acc[m][h] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the lane's B word in row kr = 4 q + lq of a step q: pixel n = 32 w + 16 h + l16 at slot (n >> 2) ^ 4 lq
    int bw[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int n = 32 * wave + 16 * h + l16;
        bw[h] = kSiAF + lq * kSiTN + 4 * ((n >> 2) ^ (4 * lq)) + (n & 3);
    }

    issue(0);
    for (int s = 0; s < nstage; ++s) {
        wait_vmem();
        lds_barrier();
        if (s + 1 < nstage) issue(s + 1);
        const float* st = lds + (s & 1) * kSiST;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float av[3], bv[2];
#pragma unroll
            for (int m = 0; m < 3; ++m) av[m] = st[(4 * q + lq) * 48 + 16 * m + l16];
#pragma unroll
            for (int h = 0; h < 2; ++h) bv[h] = st[bw[h] + 4 * q * kSiTN];
#pragma unroll
            for (int m = 0; m < 3; ++m)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    acc[m][h] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[m], bv[h], acc[m][h], 0, 0, 0);
        }
    }

    // block (m, h): register r of lane (lq, l16) is K row 16 m + 4 lq + r = (ci = m, kh = lq, kw = r)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int gp = n0 + 32 * wave + 16 * h + l16;
        if (gp >= ntot) continue;
        const int img = gp / a.P, pl = gp - img * a.P;
        const int i = pl / a.Wo, j = pl - i * a.Wo;
#pragma unroll
        for (int m = 0; m < 3; ++m)
            __builtin_nontemporal_store(acc[m][h], reinterpret_cast<f32x4*>(
                                                       a.out + (((int64_t)(img * 3 + m) * a.H + 4 * i + lq) * a.W + 4 * j)));
    }
}

// grad_weight / grad_bias partials of the 4x4/4 stem on 3 channels (K = 48,
// at most 256 output channels): gW[co][K] = sum_p G[co][p] Xp[K][p].  The
// whole result is 16 x 3 blocks of 16 x 16 (16 x 16 x 4 MFMA blocks fit K =
// 48 exactly); each workgroup sums a contiguous range of 16-pixel chunks (a
// chunk lies in one output row of one image) into its own slab, and the slabs
// are added in workgroup order afterwards.  Wave w owns output-channel blocks
// 4 w .. 4 w + 3 and all three K blocks.  A stage is one chunk, loaded
// straight into LDS one stage ahead:
//   A  G[img][co][the chunk's 16 pixels]: 256 rows of 4 units, unit u of row
//      co at slot u ^ ((co >> 2) & 3);
//   B  x[img][ci][4 i + kh][the chunk's 16 pixels x 4 kw]: 12 rows (ci, kh),
//      pixel u of row r at slot u ^ 4 (r & 3).
// The swizzles put a step's 16 rows x 4 pixels (A) and 4 rows x 4 pixels x 4
// kw (B) in distinct banks.  Threads t < Co add row t of each A stage for
// grad_bias.
constexpr int kSwAF = 256 * 16, kSwBF = 12 * 64, kSwST = kSwAF + kSwBF;

__global__ void __launch_bounds__(kNT, 2)
stem_bww_kernel(PArgs a, float* slabs)
{
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    __shared__ __align__(16) float lds[2 * kSwST];
    const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int l16 = lane & 15, lq = lane >> 4;
    const int c_beg = (int)((int64_t)blockIdx.x * a.chunks / gridDim.x);
    const int nst = (int)((int64_t)(blockIdx.x + 1) * a.chunks / gridDim.x) - c_beg;

    const i32x4 rg = plane_rsrc(a.g, a.N * a.Co * a.P * 4);
    const i32x4 rx = plane_rsrc(a.x, a.N * 3 * a.H * a.W * 4);
    int gvoff[4], xvoff = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int pos = 64 * (4 * wave + k) + lane;
        const int co = pos >> 2, u = (pos & 3) ^ ((co >> 2) & 3);
        gvoff[k] = co < a.Co ? (co * a.P + 4 * u) * 4 : (int)0x80000000;
    }
    if (wave < 3) {
        const int pos = 64 * wave + lane;
        const int r = pos >> 4, u = (pos & 15) ^ (4 * (r & 3));
        xvoff = (((r / 4) * a.H + r % 4) * a.W + 4 * u) * 4;
    }
    auto issue = [&](int s) {
        const int gp = 16 * (c_beg + s);
        const int img = gp / a.P, pl = gp - img * a.P;
        const int i = pl / a.Wo, j0 = pl - i * a.Wo;
        const int gbase = (img * a.Co * a.P + pl) * 4;
        const int xbase = ((img * 3 * a.H + 4 * i) * a.W + 4 * j0) * 4;
        float* st = lds + (s & 1) * kSwST;
#pragma unroll
        for (int k = 0; k < 4; ++k) dma16(rg, st + (4 * wave + k) * 256, gvoff[k] + gbase);
        if (wave < 3) dma16(rx, st + kSwAF + wave * 256, xvoff + xbase);
    };

    f32x4 acc[4][3];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int k = 0; k < 3; ++k) acc[c][k] = f32x4{0.f, 0.f, 0.f, 0.f};
    float bsum = 0.f;
    const bool bias_thread = t < a.Co && a.with_bias;

    if (nst > 0) issue(0);
    for (int s = 0; s < nst; ++s) {
        wait_vmem();
        lds_barrier();
        if (s + 1 < nst) issue(s + 1);
        const float* st = lds + (s & 1) * kSwST;
        if (bias_thread) {
            const int f = (t >> 2) & 3;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float4 v = *reinterpret_cast<const float4*>(st + 16 * t + 4 * (u ^ f));
                bsum += v.x; bsum += v.y; bsum += v.z; bsum += v.w;
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            // step q: k-slot lq is pixel 4 q + lq
            float av[4], bv[3];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int co = 16 * (4 * wave + c) + l16;
                av[c] = st[16 * co + 4 * (q ^ ((co >> 2) & 3)) + lq];
            }
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                const int r = 4 * k + (l16 >> 2);
                bv[k] = st[kSwAF + 64 * r + 4 * ((4 * q + lq) ^ (4 * (r & 3))) + (l16 & 3)];
            }
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int k = 0; k < 3; ++k)
                    acc[c][k] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[c], bv[k], acc[c][k], 0, 0, 0);
        }
    }

    // block (c, k): register r of lane (lq, l16) is output channel 16 (4 w + c) + 4 lq + r, K = 16 k + l16
    float* slab = slabs + (int64_t)blockIdx.x * a.Co * 49;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        if (16 * (4 * wave + c) >= a.Co) continue;
#pragma unroll
        for (int k = 0; k < 3; ++k)
#pragma unroll
            for (int r = 0; r < 4; ++r) slab[(16 * (4 * wave + c) + 4 * lq + r) * 48 + 16 * k + l16] = acc[c][k][r];
    }
    if (bias_thread) slab[a.Co * 48 + t] = bsum;
}

// dst[grp][e] = sum of src[k][e] over the slabs k of group grp (slabs
// [grp * per, min(n, (grp + 1) * per))), added in slab order, in float4
// units.  The loads of 8 slabs are issued before their adds so that they are
// in flight together; the order of the adds is unchanged.  With dw non-null
// (the last stage), element e goes to dw (e < nw4) or db, instead of dst.
__global__ void __launch_bounds__(256)
slab_sum_kernel(const float4* __restrict__ src, int64_t count4, int n, int per, float4* __restrict__ dst,
                float4* __restrict__ dw, float4* __restrict__ db, int64_t nw4)
{
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= count4) return;
    const int grp = blockIdx.y;
    const int k0 = grp * per;
    const int m = (n - k0 < per ? n - k0 : per);
    const float4* p = src + (int64_t)k0 * count4 + e;
    float4 s = p[0];
    int k = 1;
    for (; k + 8 <= m; k += 8) {
        float4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = p[(int64_t)(k + u) * count4];
#pragma unroll
        for (int u = 0; u < 8; ++u) { s.x += v[u].x; s.y += v[u].y; s.z += v[u].z; s.w += v[u].w; }
    }
    for (; k < m; ++k) {
        const float4 v = p[(int64_t)k * count4];
        s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    if (dw) {
        if (e < nw4) dw[e] = s;
        else if (db) db[e - nw4] = s;
    } else {
        dst[(int64_t)grp * count4 + e] = s;
    }
}

PArgs make_args(const Geom& g)
{
    PArgs a{};
    a.N = g.n;
    a.Ci = g.ci;
    a.Co = g.co;
    a.H = g.h;
    a.W = g.wl;
    a.Ho = g.ho;
    a.Wo = g.wol;
    a.P = g.ho * g.wol;
    a.Kt = g.ci * g.k * g.k;
    return a;
}

constexpr int kSlabsPerGroup = 16;   // first-stage group size of the split sum
constexpr int kOneStageMax = 32;     // at most this many splits are summed in one stage

// grad_weight's tiling: the K side is 64 wide for ci * k * k <= 64; the
// output-channel side is 256 (waves of 128 x 64, two workgroups per CU) when
// there are at least 256 channels, else 128.  The pixel reduction is split so
// that there are about two (256-row tiles) or four (128-row tiles) workgroups
// per CU.
struct WgradPlan {
    int tm, tn, tiles_m, tiles_n, splits;
};

WgradPlan wgrad_plan(const PArgs& a)
{
    WgradPlan p;
    p.tn = a.Kt <= kNarrowK ? kNarrowK : 128;
    p.tm = (p.tn == 128 && a.Co >= 256) ? 256 : 128;
    p.tiles_m = (a.Co + p.tm - 1) / p.tm;
    p.tiles_n = (a.Kt + p.tn - 1) / p.tn;
    const int target = p.tm == 256 ? 512 : 1024;
    const int tiles = p.tiles_m * p.tiles_n;
    const int chunks = a.N * (a.P / kSub);
    int s = (target + tiles - 1) / tiles;
    if (s > chunks) s = chunks;
    p.splits = s < 1 ? 1 : s;
    return p;
}

int split_groups(int splits) { return splits > kOneStageMax ? (splits + kSlabsPerGroup - 1) / kSlabsPerGroup : 0; }

template <int MODE, int TM, int TN>
hipError_t launch(const PArgs& a, int s, int grid, hipStream_t st)
{
    if (s == 1) hipLaunchKernelGGL((patch_kernel<MODE, 1, TM, TN>), dim3(grid), dim3(kNT), 0, st, a);
    else if (s == 2) hipLaunchKernelGGL((patch_kernel<MODE, 2, TM, TN>), dim3(grid), dim3(kNT), 0, st, a);
    else hipLaunchKernelGGL((patch_kernel<MODE, 4, TM, TN>), dim3(grid), dim3(kNT), 0, st, a);
    return hipGetLastError();
}


// The rows of the forward (output channels) and of grad_input (K) are tiled
// by 64 instead of 128 when that spreads the work more evenly over the CUs:
// when the busiest CU's share, counted in 64-row tiles, is smaller
// (ceil(T64 / CUs) < 2 ceil(T128 / CUs)), or when 128-row tiles would leave
// CUs idle.  Measured on the ConvNeXt-XL downsamples' forward: 64 rows for
// 896 or 224 tiles of 128 rows, 128 rows for 448.
bool rows_narrow(int rows, const PArgs& a)
{
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const int64_t cols = (int64_t)((a.P + 127) / 128) * a.N;
    const int64_t wide = (int64_t)((rows + 127) / 128) * cols, narrow = (int64_t)((rows + 63) / 64) * cols;
    const int64_t per_wide = (wide + cus - 1) / cus, per_narrow = (narrow + cus - 1) / cus;
    return per_narrow < 2 * per_wide || wide < cus;
}

}  // namespace

bool patch_supported(const Geom& g)
{
    const int64_t p = (int64_t)g.ho * g.wol;
    return g.groups == 1 && g.pad == 0 && g.k == g.stride && (g.k == 1 || g.k == 2 || g.k == 4) &&
           (g.ci * g.k * g.k) % kSub == 0 && g.co % kSub == 0 && g.wol % kSub == 0 && g.h == g.ho * g.k &&
           g.wl == g.wol * g.k && (int64_t)g.n * g.ci * g.h * g.wl < ((int64_t)1 << 31) &&
           (int64_t)g.n * g.co * p < ((int64_t)1 << 31);
}

// dma_bww_kernel's split count for 2x2/2 layers whose operands fit 32-bit
// byte offsets: tiles x splits a multiple of the CU count, about two
// workgroups per CU (0: not taken).  SSCNN_PATCH_BWW=dma / =tiled force the
// choice, =dma1 the kernel with a single split.
static int dma_bww_splits(const PArgs& a)
{
    if (a.Kt != 4 * a.Ci || a.P % kSub || a.Wo % kSub || (int64_t)a.N * a.Co * a.P * 4 >= ((int64_t)1 << 31) ||
        (int64_t)a.N * a.Ci * a.H * a.W * 4 >= ((int64_t)1 << 31))
        return 0;
    const char* env = getenv("SSCNN_PATCH_BWW");
    if (env && !strcmp(env, "tiled")) return 0;
    if (env && !strcmp(env, "dma1")) return 1;      // one split: the sums go straight to grad_weight
    const bool force = env && !strcmp(env, "dma");
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const int tiles = ((a.Co + 127) / 128) * ((a.Kt + 127) / 128);
    const int chunks = a.N * a.P / kSub;
    int splits = 0;
    if (cus > 0 && tiles % cus == 0) splits = 1;
    else if (cus > 0 && (2 * cus) % tiles == 0) splits = 2 * cus / tiles;
    else if (force) splits = (2 * cus + tiles - 1) / tiles;
    if (splits > chunks) splits = force ? chunks : 0;
    return splits;
}

// The stem's grad_weight kernel (stem_bww_kernel): 4x4/4 layers on 3 input
// channels with at most 256 outputs whose tensors fit 32-bit byte offsets,
// two workgroups per CU, each one slab (0: not taken; SSCNN_PATCH_STEM=tiled
// switches it off).
static int stem_bww_grid(const Geom& g, const PArgs& a)
{
    if (g.k != 4 || g.ci != 3 || g.co > 256 || g.co % 16 || (int64_t)a.N * a.Co * a.P * 4 >= ((int64_t)1 << 31) ||
        (int64_t)a.N * 3 * a.H * a.W * 4 >= ((int64_t)1 << 31) || a.Wo % kSub)
        return 0;
    const char* env = getenv("SSCNN_PATCH_STEM");
    if (env && !strcmp(env, "tiled")) return 0;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const int chunks = a.N * a.P / kSub;
    return chunks < 2 * cus ? chunks : 2 * cus;
}

size_t patch_wgrad_workspace_bytes(const Geom& g)
{
    const PArgs a = make_args(g);
    const int64_t slab = (int64_t)a.Co * (a.Kt + 1);
    // enough for either plan, so that the choice made at launch always fits
    const int64_t s = wgrad_plan(a).splits;
    int64_t floats = (s + split_groups((int)s)) * slab;
    if (g.k == 2) {
        const int64_t d = dma_bww_splits(a);
        const int64_t fd = d > 1 ? (d + split_groups((int)d)) * slab : 0;
        if (fd > floats) floats = fd;
    }
    const int64_t sw = stem_bww_grid(g, a);
    if (sw > 0 && (sw + split_groups((int)sw)) * slab > floats) floats = (sw + split_groups((int)sw)) * slab;
    return (size_t)floats * sizeof(float);
}

// Rows of the result tile of the forward (output channels) and grad_input (K).
// (256 rows, which pays for grad_weight, measured slower for both: the
// forward of the c4 stem 54 -> 71 us, a c4 downsample's grad_input +25 us.)
int row_tile(int rows, const PArgs& a, bool narrow_k)
{
    return narrow_k || rows_narrow(rows, a) ? 64 : 128;
}

template <int MODE>
hipError_t launch_rows(PArgs& a, int rows, int tm, int s, hipStream_t st)
{
    a.tiles_m = (rows + tm - 1) / tm;
    const int grid = a.tiles_m * a.tiles_n * a.N;
    return tm == 64 ? launch<MODE, 64, 128>(a, s, grid, st) : launch<MODE, 128, 128>(a, s, grid, st);
}

static bool pushes_any(const Push* push) { return push && (push->to_left || push->to_right || push->own); }

static void set_push(PArgs& a, const Push* push)
{
    if (!push) return;
    a.push_l = push->to_left;
    a.push_r = push->to_right;
    a.push_own = push->own;
    a.ph_l = push->hl;
    a.ph_r = push->hr;
}

// Wide forward tiles (wide_fwd_kernel): 2x2/2 layers whose operands fit
// 32-bit byte offsets, when the tile count is a whole multiple of the CU
// count (the 7 x 2^j-pixel downsamples of the stack) -- elsewhere the
// per-image tiles balance as well or better.  The environment variable
// (SSCNN_PATCH_FWD for the forward) set to wide forces them wherever they
// apply, set to tiled never.
static int wide_fwd_tiles(const PArgs& a, int nb = kWideNB)
{
    const int64_t ntot = (int64_t)a.N * a.P;
    if (a.Kt != 4 * a.Ci || a.Ci % 4 || (int64_t)a.N * a.Ci * a.H * a.W * 4 >= ((int64_t)1 << 31) ||
        (int64_t)(a.Co + kWideTM) * a.Kt * 4 >= ((int64_t)1 << 31) || ntot >= ((int64_t)1 << 31))
        return 0;
    return (int)(((a.Co + kWideTM - 1) / kWideTM) * ((ntot + 32 * nb - 1) / (32 * nb)));
}

static int cu_count()
{
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    return cus > 0 ? cus : 256;
}

// 128-pixel wide forward tiles (NB = 4) where 224-pixel ones would leave
// CUs without a tile and the 128-pixel ones still fit in one round
// (SSCNN_PATCH_FWD=wide4 forces them, =wide or =tiled the other forms).
static bool use_wide4(const PArgs& a)
{
    const int t7 = wide_fwd_tiles(a, 7), t4 = wide_fwd_tiles(a, 4);
    if (t7 == 0) return false;
    const char* env = getenv("SSCNN_PATCH_FWD");
    if (env && !strcmp(env, "wide4")) return true;
    if (env && (!strcmp(env, "wide") || !strcmp(env, "tiled"))) return false;
    const int cus = cu_count();
    return t7 < cus && t4 <= cus;
}

// The stem kernel (stem_fwd_kernel): 4x4/4 layers on 3 input channels whose
// input and output fit 32-bit byte offsets; SSCNN_PATCH_STEM=tiled switches
// it off.
static bool use_stem_fwd(const PArgs& a)
{
    if ((int64_t)a.N * a.Ci * a.H * a.W * 4 >= ((int64_t)1 << 31) || (int64_t)a.N * a.Co * a.P * 4 >= ((int64_t)1 << 31))
        return false;
    const char* env = getenv("SSCNN_PATCH_STEM");
    return !(env && !strcmp(env, "tiled"));
}

// The wide forward with two reduction halves per workgroup (KS = 2) where the
// tiles are no more than the CUs, so that each CU still runs two waves per
// SIMD; SSCNN_WIDE_HALVES=1 / =0 forces the choice.
static bool wide_halves(int tiles)
{
    const char* env = getenv("SSCNN_WIDE_HALVES");
    if (env && !strcmp(env, "1")) return true;
    if (env && !strcmp(env, "0")) return false;
    return tiles <= cu_count();
}

static bool use_wide(int tiles, const char* var)
{
    if (tiles == 0) return false;
    const char* env = getenv(var);
    if (env && !strcmp(env, "wide")) return true;
    if (env && !strcmp(env, "tiled")) return false;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    return cus > 0 && tiles % cus == 0;
}

hipError_t launch_patch_fwd(const Geom& g, const float* x, const float* w, const float* b, float* y,
                            hipStream_t st, float* act, const Push* push)
{
    if (act && g.k != 1) return hipErrorInvalidValue;
    PArgs a = make_args(g);
    a.x = x; a.w = w; a.b = b; a.out = y; a.act = act;
    set_push(a, push);
    if (g.k == 4 && g.ci == 3 && g.co <= 256 && g.co % 8 == 0 && use_stem_fwd(a)) {
        const int tiles = (int)(((int64_t)a.N * a.P + 63) / 64);
        int dev = 0, cus = 256;
        if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        const bool push_ = push && (push->to_left || push->to_right || push->own);
        const int grid = tiles < 2 * cus ? tiles : 2 * cus;
        if (push_) hipLaunchKernelGGL((stem_fwd_kernel<3, true>), dim3(grid), dim3(kStemNT), 0, st, a, a.N * a.P);
        else hipLaunchKernelGGL((stem_fwd_kernel<3, false>), dim3(grid), dim3(kStemNT), 0, st, a, a.N * a.P);
        return hipGetLastError();
    }
    if (g.k == 2 && use_wide4(a)) {
        a.tiles_m = (a.Co + kWideTM - 1) / kWideTM;
        const int grid = wide_fwd_tiles(a, 4);
        if (wide_halves(grid))
            hipLaunchKernelGGL((wide_fwd_kernel<4, 2>), dim3(grid), dim3(2 * kNT), 0, st, a, a.N * a.P);
        else
            hipLaunchKernelGGL((wide_fwd_kernel<4, 1>), dim3(grid), dim3(kNT), 0, st, a, a.N * a.P);
        return hipGetLastError();
    }
    if (g.k == 2 && use_wide(wide_fwd_tiles(a), "SSCNN_PATCH_FWD")) {
        a.tiles_m = (a.Co + kWideTM - 1) / kWideTM;
        const int grid = wide_fwd_tiles(a);
        if (wide_halves(grid))
            hipLaunchKernelGGL((wide_fwd_kernel<kWideNB, 2>), dim3(grid), dim3(2 * kNT), 0, st, a, a.N * a.P);
        else
            hipLaunchKernelGGL((wide_fwd_kernel<kWideNB, 1>), dim3(grid), dim3(kNT), 0, st, a, a.N * a.P);
        return hipGetLastError();
    }
    a.tiles_n = (a.P + 127) / 128;
    return launch_rows<FWD>(a, a.Co, row_tile(a.Co, a, false), g.k, st);
}

// Wide grad_input tiles (wide_bwi_kernel), chosen like the forward's: 2x2/2
// layers whose operands fit 32-bit byte offsets, when the tile count is a
// whole multiple of the CU count; SSCNN_PATCH_BWI=wide / =tiled force the
// choice.
static int wide_bwi_tiles(const PArgs& a)
{
    const int64_t ntot = (int64_t)a.N * a.P;
    if (a.Kt != 4 * a.Ci || a.Co % 16 || (int64_t)a.N * a.Co * a.P * 4 >= ((int64_t)1 << 31) ||
        (int64_t)a.Co * a.Kt * 4 >= ((int64_t)1 << 31) || (int64_t)a.N * a.Ci * a.H * a.W >= ((int64_t)1 << 31))
        return 0;
    return (int)(((a.Kt + kWideTM - 1) / kWideTM) * ((ntot + kWideTN - 1) / kWideTN));
}

hipError_t launch_patch_bwd_input(const Geom& g, const float* gy, const float* w, float* gx, hipStream_t st,
                                  const float* pre, const Push* push)
{
    if (pre && g.k != 1) return hipErrorInvalidValue;
    PArgs a = make_args(g);
    a.g = gy; a.w = w; a.out = gx; a.pre = pre;
    set_push(a, push);
    if (g.k == 4 && g.ci == 3 && g.co % 16 == 0 && !pre && use_stem_fwd(a)) {
        // the stem: 48 x 128-pixel tiles on 16 x 16 MFMA blocks (SSCNN_PATCH_STEM=tiled switches them
        // off); a push form copies the edge columns afterwards
        hipLaunchKernelGGL(stem_bwi_kernel, dim3((unsigned)(((int64_t)a.N * a.P + kSiTN - 1) / kSiTN)), dim3(kNT), 0, st,
                           a, a.N * a.P);
        hipError_t e = hipGetLastError();
        if (e == hipSuccess && pushes_any(push))
            e = launch_push_edges(gx, (int64_t)g.n * g.ci, g.h, g.wl, push->hl, push->hr, push->to_left, push->to_right,
                                  push->own, st);
        return e;
    }
    if (g.k == 2 && use_wide(wide_bwi_tiles(a), "SSCNN_PATCH_BWI")) {
        a.tiles_m = (a.Kt + kWideTM - 1) / kWideTM;
        hipLaunchKernelGGL(wide_bwi_kernel, dim3(wide_bwi_tiles(a)), dim3(kNT), 0, st, a, a.N * a.P);
        return hipGetLastError();
    }
    a.tiles_n = (a.P + 127) / 128;
    return launch_rows<BWI>(a, a.Kt, row_tile(a.Kt, a, a.Kt <= kNarrowK), g.k, st);
}

// grad_weight / grad_bias = the sum of n slabs of partials (each Co * Kt
// weights, then Co biases), added in slab order: one pass for n <= 32, else
// groups of 16, then the groups.
static hipError_t sum_slabs(const PArgs& a, float* slabs, int n, float* gw, float* gb, hipStream_t st)
{
    hipError_t e;
    const int64_t slab = (int64_t)a.Co * (a.Kt + 1);
    const int64_t count4 = slab / 4, nw4 = (int64_t)a.Co * a.Kt / 4;
    const unsigned bx = (unsigned)((count4 + 255) / 256);
    float4* dw = reinterpret_cast<float4*>(gw);
    float4* db = reinterpret_cast<float4*>(gb);
    const int groups = split_groups(n);
    if (groups == 0) {
        hipLaunchKernelGGL(slab_sum_kernel, dim3(bx, 1), dim3(256), 0, st, reinterpret_cast<const float4*>(slabs),
                           count4, n, n, nullptr, dw, db, nw4);
        return hipGetLastError();
    }
    float4* mid = reinterpret_cast<float4*>(slabs + n * slab);
    hipLaunchKernelGGL(slab_sum_kernel, dim3(bx, groups), dim3(256), 0, st, reinterpret_cast<const float4*>(slabs),
                       count4, n, kSlabsPerGroup, mid, nullptr, nullptr, nw4);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(slab_sum_kernel, dim3(bx, 1), dim3(256), 0, st, static_cast<const float4*>(mid), count4,
                       groups, groups, nullptr, dw, db, nw4);
    return hipGetLastError();
}

hipError_t launch_patch_bwd_weight(const Geom& g, const float* x, const float* gy, float* gw, float* gb,
                                   void* ws, hipStream_t st)
{
    PArgs a = make_args(g);
    a.x = x; a.g = gy;
    a.chunks = a.N * (a.P / kSub);
    a.with_bias = gb != nullptr;
    float* slabs = static_cast<float*>(ws);
    a.out = slabs;
    hipError_t e;
    if (const int sw = stem_bww_grid(g, a)) {
        hipLaunchKernelGGL(stem_bww_kernel, dim3(sw), dim3(kNT), 0, st, a, slabs);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        return sum_slabs(a, slabs, sw, gw, gb, st);
    }
    const int dma_splits = g.k == 2 ? dma_bww_splits(a) : 0;
    if (dma_splits > 0) {
        a.tiles_m = (a.Co + 127) / 128;
        a.tiles_n = (a.Kt + 127) / 128;
        a.splits = dma_splits;
        a.gw_out = gw;
        a.gb_out = gb;
        hipLaunchKernelGGL(dma_bww_kernel, dim3(a.tiles_m * a.tiles_n * a.splits), dim3(kNT), 0, st, a);
        e = hipGetLastError();
        if (e != hipSuccess || a.splits == 1) return e;
    } else {
        const WgradPlan plan = wgrad_plan(a);
        a.tiles_m = plan.tiles_m;
        a.tiles_n = plan.tiles_n;
        a.splits = plan.splits;
        const int grid = a.tiles_m * a.tiles_n * a.splits;
        e = plan.tn == kNarrowK ? launch<BWW, 128, kNarrowK>(a, g.k, grid, st)
            : plan.tm == 256    ? launch<BWW, 256, 128>(a, g.k, grid, st)
                                : launch<BWW, 128, 128>(a, g.k, grid, st);
        if (e != hipSuccess) return e;
    }

    return sum_slabs(a, slabs, a.splits, gw, gb, st);
}

}  // namespace sscnn
