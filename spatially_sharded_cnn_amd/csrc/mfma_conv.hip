// mfma_conv.hip -- dense (groups == 1) k x k, stride 1, pad k/2 convolution of
// one W-shard as an implicit GEMM on the FP32 matrix cores of gfx950
// (v_mfma_f32_32x32x2_f32), forward and grad_input.  The layer is the pages'
// worked example (NVIDIA blog "Perception Model Training for Autonomous
// Vehicles with Tensor Parallelism", Figure 1: 5x5, padding 2, stride 1) at a
// dense 256 -> 256 channel width.
//
// Per tap t = (kh, kw) the convolution is a matrix product
//     Y[o, px] += sum_c W[o, c, t] * Xext[c, px shifted by t]
// with px the output pixels.  D = A x B with A = weights (rows o, k = c) and
// B = the input patch (k = c, columns px), so the 32 lanes of a D row hold 32
// consecutive output columns and the stores run along W.
//
//  * workgroup tile: 64 output channels x (4 rows x 64 columns) of pixels of
//    one image; each of the 4 waves takes one pixel row: 64 channels x 64
//    pixels (2 x 2 blocks of 32 x 32);
//  * the reduction walks input channels in chunks of 4.  A chunk's weights
//    (4 x k*k x 64) and input patch (4 channels x (4+k-1) rows x (64+k-1)
//    columns: the shard's own columns, halo columns at the shard's edges,
//    zero rows above and below the image) are staged in LDS; the next chunk is
//    fetched into registers while the current one is multiplied;
//  * grad_input is the same kernel on grad_output (and its halo) with the
//    weights read transposed (channels in <-> out) and flipped (tap k*k-1-t).
//
// LDS strides are odd along the lanes of an operand read and put the two
// halves of a wave (k = 0 / 1 of the 32x32x2 operand) in disjoint banks, and
// each thread's k-th staging load sits at a fixed stride from its first, so no
// per-load address has to be kept in registers.
#include "internal.h"
#include "mfma_conv.h"

namespace sscnn {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kNT = 256;    // threads per workgroup (4 waves)
constexpr int kBN = 64;     // output channels per workgroup
constexpr int kTH = 4;      // output rows per workgroup (one per wave)
constexpr int kTW = 64;     // output columns per workgroup
constexpr int kCK = 4;      // reduction channels per chunk

struct MfArgs {
    const float* x;      // GEMM input activation (N, C, H, W): X (forward) or G (grad_input)
    const float* halo;   // (N, C, H + 2 crh, hl + hr); null with hl = hr = 0 when absent
    const float* up;     // rows above / below the slice (height and 2-D sharding), null when absent:
    const float* down;   //   rh rows per plane each, rplane floats between planes
    int64_t rplane;
    int rh, crh;         // row-halo height; rows of the column halo above row 0
    const float* w;      // weight (Co, Ci, k, k) as given
    const float* b;      // bias (O) or null
    float* y;            // (N, O, H, W)
    int N, C, O, H, W, hl, hr;
    int wci;             // Ci of the weight tensor (row length / k*k)
    int tiles_w, tiles_h, tiles_m, tiles_o;
};

template <int K>
struct Shape {
    static constexpr int KK = K * K;
    static constexpr int P = K / 2;
    // Weight chunk in LDS, kept in the weight tensor's own order:
    //   forward      [o][c*k*k + t]  row stride OS (odd: lanes on consecutive o hit distinct banks)
    //   grad_input   [c][o][t]       o stride k*k (odd), channel stride TCS (= 32 mod 64)
    static constexpr int OS = kCK * KK + 1;
    static constexpr int TCS = ((kBN * KK + 31) / 64) * 64 + 32;
    static constexpr int WS_FLOATS = (kBN * OS > kCK * TCS) ? kBN * OS : kCK * TCS;
    static constexpr int XRS = kTW + K - 1;                      // patch row
    static constexpr int XCS = (((kTH + K - 1) * XRS + 31) / 64) * 64 + 32;
    static constexpr int XS_FLOATS = kCK * XCS;
    // forward weight fetch: thread -> (float4 column q of a 4*k*k row, row group), rows step RG
    static constexpr int QROW = KK;                              // float4 per output row (4*KK/4)
    static constexpr int RG = kNT / QROW;                        // row groups per pass
    static constexpr int NWF = (kBN + RG - 1) / RG;
    // grad_input weight fetch: thread -> (channel, float4 index), per channel 64*k*k/4 float4
    static constexpr int QCH = kBN * KK / 4;
    static constexpr int TPC = kNT / kCK;                        // threads per channel
    static constexpr int NWT = (QCH + TPC - 1) / TPC;
    static constexpr int NWV = NWF > NWT ? NWF : NWT;
    static constexpr int NXV = (kCK * (kTH + K - 1) * (kTW / 4) + kNT - 1) / kNT;  // patch float4 per thread
    static constexpr int NXS = (kCK * (kTH + K - 1) * 2 * P + kNT - 1) / kNT;     // patch side floats
};

template <int K>
struct Regs {
    float4 w[Shape<K>::NWV];
    float4 x[Shape<K>::NXV];
    float s[Shape<K>::NXS];
};

// Row r of plane pl over the slice's own columns: the slice for 0 <= r < H,
// the row halos for the rh rows beyond it; null (zeros) elsewhere.
__device__ __forceinline__ const float* row_at(const MfArgs& a, int64_t pl, int r)
{
    if (r >= 0 && r < a.H) return a.x + (pl * a.H + r) * a.W;
    if (r < 0) return (a.up && r >= -a.rh) ? a.up + pl * a.rplane + (int64_t)(r + a.rh) * a.W : nullptr;
    return (a.down && r < a.H + a.rh) ? a.down + pl * a.rplane + (int64_t)(r - a.H) * a.W : nullptr;
}

// Extended-row value: column xcol of the shard (may lie in the column halo),
// zero outside [-hl, W + hr) and outside the rows there are data for.
__device__ __forceinline__ float ext_at(const MfArgs& a, int64_t pl, int r, int xcol)
{
    if (xcol >= 0 && xcol < a.W) {
        const float* p = row_at(a, pl, r);
        return p ? p[xcol] : 0.f;
    }
    if (r < -a.crh || r >= a.H + a.crh) return 0.f;
    const int hw = a.hl + a.hr;
    const float* hp = a.halo + (pl * (a.H + 2 * a.crh) + (r + a.crh)) * hw;
    if (xcol < 0) return xcol >= -a.hl ? hp[a.hl + xcol] : 0.f;
    return xcol < a.W + a.hr ? hp[a.hl + (xcol - a.W)] : 0.f;
}

template <int K, bool TRANS>
__device__ __forceinline__ void fetch(Regs<K>& R, const MfArgs& a, int n, int o0, int i0, int j0, int c0)
{
    using S = Shape<K>;
    constexpr int KK = S::KK, P = S::P;
    const int tid = threadIdx.x;
    // weights: 4 channels x k*k taps x 64 outputs, read along the contiguous
    // direction of the weight tensor; the k-th load of a thread is at a fixed
    // stride from its first, in global memory and in LDS.
    if (!TRANS) {
        // per output o: W[o, c0..c0+3, :] is 4*k*k contiguous floats (KK float4)
        const int q = tid % S::QROW, og = tid / S::QROW;
        const float* src = a.w + ((int64_t)(o0 + og) * a.wci + c0) * KK + 4 * q;
        const int64_t step = (int64_t)S::RG * a.wci * KK;
#pragma unroll
        for (int k = 0; k < S::NWV; ++k) {
            R.w[k] = make_float4(0.f, 0.f, 0.f, 0.f);
            const int ol = og + k * S::RG;
            if (k < S::NWF && og < S::RG && ol < kBN && o0 + ol < a.O)
                R.w[k] = *reinterpret_cast<const float4*>(src + k * step);
        }
    } else {
        // per channel c: W[c, o0..o0+63, :] is 64*k*k contiguous floats
        const int cl = tid / S::TPC, q0 = tid % S::TPC;
        const float* src = a.w + ((int64_t)(c0 + cl) * a.wci + o0) * KK;
#pragma unroll
        for (int k = 0; k < S::NWV; ++k) {
            R.w[k] = make_float4(0.f, 0.f, 0.f, 0.f);
            const int q = q0 + k * S::TPC;
            if (k < S::NWT && q < S::QCH && c0 + cl < a.C) {
                const float* p = src + 4 * q;
                if (o0 + (4 * q + 3) / KK < a.O) {
                    R.w[k] = *reinterpret_cast<const float4*>(p);
                } else {
                    // the float4 crosses the last valid output channel: element-wise
                    if (o0 + (4 * q + 0) / KK < a.O) R.w[k].x = p[0];
                    if (o0 + (4 * q + 1) / KK < a.O) R.w[k].y = p[1];
                    if (o0 + (4 * q + 2) / KK < a.O) R.w[k].z = p[2];
                }
            }
        }
    }
    // input patch: 4 channels x (TH+K-1) rows x (TW+K-1) extended columns
    const int64_t plane0 = (int64_t)n * a.C + c0;
#pragma unroll
    for (int k = 0; k < S::NXV; ++k) {
        const int g = tid + k * kNT;
        R.x[k] = make_float4(0.f, 0.f, 0.f, 0.f);
        constexpr int Q = kTW / 4;
        if (g < kCK * (kTH + K - 1) * Q) {
            const int cl = g / ((kTH + K - 1) * Q);
            const int rem = g - cl * ((kTH + K - 1) * Q);
            const int rr = rem / Q, q = rem - rr * Q;
            const int r = i0 - P + rr, col = j0 + 4 * q;
            if (c0 + cl < a.C) {
                if (col + 3 < a.W) {
                    const float* rp = row_at(a, plane0 + cl, r);
                    if (rp) R.x[k] = *reinterpret_cast<const float4*>(rp + col);
                } else {
                    R.x[k].x = ext_at(a, plane0 + cl, r, col);
                    R.x[k].y = ext_at(a, plane0 + cl, r, col + 1);
                    R.x[k].z = ext_at(a, plane0 + cl, r, col + 2);
                    R.x[k].w = ext_at(a, plane0 + cl, r, col + 3);
                }
            }
        }
    }
#pragma unroll
    for (int k = 0; k < S::NXS; ++k) {
        const int g = tid + k * kNT;
        R.s[k] = 0.f;
        if (g < kCK * (kTH + K - 1) * 2 * P) {
            const int cl = g / ((kTH + K - 1) * 2 * P);
            const int rem = g - cl * ((kTH + K - 1) * 2 * P);
            const int rr = rem / (2 * P), e = rem - rr * (2 * P);
            const int xcol = e < P ? j0 - P + e : j0 + kTW + (e - P);
            if (c0 + cl < a.C) R.s[k] = ext_at(a, plane0 + cl, i0 - P + rr, xcol);
        }
    }
}

template <int K, bool TRANS>
__device__ __forceinline__ void put(const Regs<K>& R, float* __restrict__ ws, float* __restrict__ xs)
{
    using S = Shape<K>;
    constexpr int KK = S::KK, P = S::P;
    const int tid = threadIdx.x;
    if (!TRANS) {
        const int q = tid % S::QROW, og = tid / S::QROW;
        float* d = ws + og * S::OS + 4 * q;
#pragma unroll
        for (int k = 0; k < S::NWF; ++k) {
            const int ol = og + k * S::RG;
            if (og < S::RG && ol < kBN) {
                float* e = d + k * S::RG * S::OS;
                e[0] = R.w[k].x;
                e[1] = R.w[k].y;
                e[2] = R.w[k].z;
                e[3] = R.w[k].w;
            }
        }
    } else {
        const int cl = tid / S::TPC, q0 = tid % S::TPC;
        float* d = ws + cl * S::TCS + 4 * q0;
#pragma unroll
        for (int k = 0; k < S::NWT; ++k)
            if (q0 + k * S::TPC < S::QCH) *reinterpret_cast<float4*>(d + 4 * k * S::TPC) = R.w[k];
    }
    constexpr int Q = kTW / 4;
#pragma unroll
    for (int k = 0; k < S::NXV; ++k) {
        const int g = tid + k * kNT;
        if (g < kCK * (kTH + K - 1) * Q) {
            const int cl = g / ((kTH + K - 1) * Q);
            const int rem = g - cl * ((kTH + K - 1) * Q);
            const int rr = rem / Q, q = rem - rr * Q;
            float* d = xs + cl * S::XCS + rr * S::XRS + P + 4 * q;
            d[0] = R.x[k].x;
            d[1] = R.x[k].y;
            d[2] = R.x[k].z;
            d[3] = R.x[k].w;
        }
    }
#pragma unroll
    for (int k = 0; k < S::NXS; ++k) {
        const int g = tid + k * kNT;
        if (g < kCK * (kTH + K - 1) * 2 * P) {
            const int cl = g / ((kTH + K - 1) * 2 * P);
            const int rem = g - cl * ((kTH + K - 1) * 2 * P);
            const int rr = rem / (2 * P), e = rem - rr * (2 * P);
            xs[cl * S::XCS + rr * S::XRS + (e < P ? e : kTW + e)] = R.s[k];
        }
    }
}

template <int K, bool TRANS>
__global__ void __launch_bounds__(kNT, 2)
mfma_conv_kernel(MfArgs a)
{
    using S = Shape<K>;
    constexpr int KK = S::KK;
    __shared__ __align__(16) float ws[S::WS_FLOATS];
    __shared__ __align__(16) float xs[S::XS_FLOATS];

    // tile -> (output-channel block, image, row block, column block).  Workgroups
    // are dealt round-robin to the 8 XCDs (each with its own L2); when the pixel
    // tiles split evenly, each XCD takes a contiguous range of pixel tiles with
    // all their output-channel blocks, so the input rows a tile shares with its
    // channel blocks and its neighbouring row tiles stay in one L2.
    const int bid = blockIdx.x;
    int ot, mt;
    if (a.tiles_m % 8 == 0) {
        const int xcd = bid % 8, j = bid / 8;
        ot = j % a.tiles_o;
        mt = xcd * (a.tiles_m / 8) + j / a.tiles_o;
    } else {
        ot = bid % a.tiles_o;
        mt = bid / a.tiles_o;
    }
    const int tw = mt % a.tiles_w;
    mt /= a.tiles_w;
    const int th = mt % a.tiles_h;
    const int n = mt / a.tiles_h;
    const int o0 = ot * kBN, i0 = th * kTH, j0 = tw * kTW;

    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wo = 0, wp = wave;   // all 64 output channels, pixel row = wave
    const int lhalf = lane >> 5, l32 = lane & 31;

    // accumulators start at the bias of their output channel
    f32x16 acc[2][2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int o = o0 + wo * 64 + cb * 32 + 8 * (r / 4) + 4 * lhalf + (r % 4);
            const float bv = (a.b && o < a.O) ? a.b[o] : 0.f;
            acc[cb][0][r] = bv;
            acc[cb][1][r] = bv;
        }

    Regs<K> R;
    const int nchunks = (a.C + kCK - 1) / kCK;
    fetch<K, TRANS>(R, a, n, o0, i0, j0, 0);
    for (int ch = 0; ch < nchunks; ++ch) {
        if (ch) lds_barrier();            // everyone is done reading the previous chunk
        put<K, TRANS>(R, ws, xs);
        lds_barrier();
        if (ch + 1 < nchunks) fetch<K, TRANS>(R, a, n, o0, i0, j0, (ch + 1) * kCK);
        // A operand: lane (l32, lhalf) reads output channel wo*64 + l32 (+32), channel 2*cp + lhalf
        const float* wsa = TRANS ? ws + lhalf * S::TCS + (wo * 64 + l32) * KK
                                 : ws + (wo * 64 + l32) * S::OS + lhalf * KK;
        const float* xsb = xs + lhalf * S::XCS + wp * S::XRS + l32;
#pragma unroll 1
        for (int kh = 0; kh < K; ++kh)
#pragma unroll
        for (int kw = 0; kw < K; ++kw) {
            const int t = kh * K + kw;
#pragma unroll
            for (int cp = 0; cp < kCK / 2; ++cp) {
                const float a0 = TRANS ? wsa[2 * cp * S::TCS + (KK - 1 - t)]
                                       : wsa[2 * cp * KK + t];
                const float a1 = TRANS ? wsa[2 * cp * S::TCS + 32 * KK + (KK - 1 - t)]
                                       : wsa[2 * cp * KK + t + 32 * S::OS];
                const float b0 = xsb[2 * cp * S::XCS + kh * S::XRS + kw];
                const float b1 = xsb[2 * cp * S::XCS + kh * S::XRS + kw + 32];
                acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
                acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
                acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
                acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
            }
        }
    }

    // D[o][px]: register r holds output channel 8(r/4) + 4*lhalf + r%4 of the
    // block, lane%32 the pixel column within the 32-column block.
    const int row = i0 + wp;
    if (row < a.H) {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int pb = 0; pb < 2; ++pb) {
                const int col = j0 + pb * 32 + l32;
                if (col < a.W) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int o = o0 + wo * 64 + cb * 32 + 8 * (r / 4) + 4 * lhalf + (r % 4);
                        if (o < a.O) a.y[(((int64_t)n * a.O + o) * a.H + row) * a.W + col] = acc[cb][pb][r];
                    }
                }
            }
    }
}

template <int K, bool TRANS>
hipError_t launch(MfArgs a, hipStream_t st)
{
    a.tiles_w = (a.W + kTW - 1) / kTW;
    a.tiles_h = (a.H + kTH - 1) / kTH;
    a.tiles_m = a.N * a.tiles_h * a.tiles_w;
    a.tiles_o = (a.O + kBN - 1) / kBN;
    const int64_t grid = (int64_t)a.tiles_m * a.tiles_o;
    hipLaunchKernelGGL((mfma_conv_kernel<K, TRANS>), dim3((unsigned)grid), dim3(kNT), 0, st, a);
    return hipGetLastError();
}

template <bool TRANS>
hipError_t launch_k(const MfArgs& a, int k, hipStream_t st)
{
    return k == 3 ? launch<3, TRANS>(a, st) : launch<5, TRANS>(a, st);
}

}  // namespace

bool mfma_conv_supported(const Geom& g)
{
    return g.groups == 1 && g.stride == 1 && (g.k == 3 || g.k == 5) && g.pad == g.k / 2 &&
           g.ci >= 16 && g.co >= 16 && g.ci % 4 == 0 && g.co % 4 == 0 && g.wl % 4 == 0;
}

hipError_t launch_mfma_fwd(const Geom& g, const float* x, const float* xh, const float* w,
                           const float* b, float* y, hipStream_t st)
{
    return launch_mfma_fwd_rows(g, x, xh, RowHalo{}, w, b, y, st);
}

hipError_t launch_mfma_bwd_input(const Geom& g, const float* gy, const float* gyh, const float* w,
                                 float* gx, hipStream_t st)
{
    return launch_mfma_bwd_input_rows(g, gy, gyh, RowHalo{}, w, gx, st);
}

hipError_t launch_mfma_fwd_rows(const Geom& g, const float* x, const float* xh, const RowHalo& rows,
                                const float* w, const float* b, float* y, hipStream_t st)
{
    MfArgs a{};
    a.x = x; a.halo = xh; a.w = w; a.b = b; a.y = y;
    a.up = rows.up; a.down = rows.down; a.rplane = rows.rplane; a.rh = rows.rh; a.crh = xh ? rows.crh : 0;
    a.N = g.n; a.C = g.ci; a.O = g.co; a.H = g.h; a.W = g.wl;
    a.hl = xh ? g.hl : 0; a.hr = xh ? g.hr : 0;     // no halo: ext_at() reads zeros beyond the slice
    a.wci = g.ci;
    return launch_k<false>(a, g.k, st);
}

hipError_t launch_mfma_bwd_input_rows(const Geom& g, const float* gy, const float* gyh, const RowHalo& rows,
                                      const float* w, float* gx, hipStream_t st)
{
    MfArgs a{};
    a.x = gy; a.halo = gyh; a.w = w; a.b = nullptr; a.y = gx;
    a.up = rows.up; a.down = rows.down; a.rplane = rows.rplane; a.rh = rows.rh; a.crh = gyh ? rows.crh : 0;
    a.N = g.n; a.C = g.co; a.O = g.ci; a.H = g.ho; a.W = g.wol;
    a.hl = gyh ? g.ghl : 0; a.hr = gyh ? g.ghr : 0;
    a.wci = g.ci;
    return launch_k<true>(a, g.k, st);
}

}  // namespace sscnn
