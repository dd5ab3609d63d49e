// patchify.hip -- dense convolutions whose kernel equals their stride (k = s,
// pad 0, groups 1) on the FP32 matrix cores of gfx950 (v_mfma_f32_32x32x2_f32):
// the 4x4/4 stem and the 2x2/2 downsamples of the ConvNeXt-style stack that
// the pages shard (NVIDIA blog "Perception Model Training for Autonomous
// Vehicles with Tensor Parallelism", DTensor section: ConvNeXt-XL trained with
// Shard(3) activations).  Such a layer needs no halo (its patches never
// straddle a shard edge), and it is a matrix product after a reshape: with
// K = (ci, kh, kw) and the output pixels p = (i, j) of one image,
//     forward       Y[co][p]   = b[co] + sum_K W[co][K] * Xp[K][p]
//     grad_input    dXp[K][p]  = sum_co W[co][K] * G[co][p]
//     grad_weight   gW[co][K]  = sum_(n,p) G[co][p] * Xp[K][p],  gB[co] = sum G
// where Xp[K][p] = X[ci][i*s + kh][j*s + kw].  The reshape is never
// materialised: operand tiles are gathered from NCHW straight into LDS (s
// consecutive floats per (K group, pixel)), and grad_input's result is
// scattered back to NCHW with one s-wide store per lane.
//
// One kernel template serves the three products: a 256-thread workgroup
// computes a 128 x 128 tile of the result, each of its 4 waves a 64 x 64
// block (2 x 2 MFMA blocks of 32 x 32); the reduction runs in chunks of 16
// staged in LDS (k-major rows), double-buffered with one barrier per chunk,
// the next chunk's global loads in flight while the current one multiplies.
// grad_weight splits the pixel reduction over workgroups (fixed split count,
// partials summed in split order by a second kernel, grad_bias fused into
// the first column tile): no atomics, bitwise reproducible.
#include "internal.h"
#include "patchify.h"

namespace sscnn {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kNT = 256;
constexpr int kBM = 128;         // result rows per workgroup
constexpr int kBN = 128;         // result columns per workgroup
constexpr int kBK = 16;          // reduction per LDS chunk
constexpr int kLD = kBM + 32;    // LDS row pitch: the two half-waves (k rows 2s, 2s+1) fall 32 banks apart

enum Mode { FWD = 0, BWI = 1, BWW = 2 };

struct PArgs {
    const float* x;       // input X (N, Ci, H, W)           FWD, BWW
    const float* g;       // grad_output G (N, Co, Ho, Wo)   BWI, BWW
    const float* w;       // weight (Co, Ci, s, s)           FWD, BWI
    const float* b;       // bias (Co) or null               FWD
    float* out;           // Y (FWD), dX (BWI), partials (splits, Co, Kt) (BWW)
    float* outb;          // bias partials (splits, Co) or null (BWW)
    int N, Ci, Co, H, W, Ho, Wo, P, Kt;
    int tiles_m, tiles_n;             // result tiles (columns: pixels of one image for FWD / BWI)
    int splits, chunks;               // BWW: pixel chunks of kBK, split into `splits` ranges
};

// Global -> registers for one chunk (8 A values and 8 B values per thread),
// then registers -> LDS.  Each mode gathers its own operands.
template <int MODE, int S>
struct Stage {
    static constexpr int GPC = kBK / S;       // K groups (s consecutive K) per chunk   (FWD)
    static constexpr int GPT = kBN / S;       // K groups per column tile               (BWW)
    float ra[8];
    float rb[8];

    // k0: reduction offset of the chunk.  FWD: K; BWI: co; BWW: pixel of image img.
    __device__ void load(const PArgs& a, int img, int m0, int n0, int k0)
    {
        const int t = threadIdx.x;
        if constexpr (MODE == FWD) {
            // A[m][k] = W[m0 + m][k0 + k]: per row 16 contiguous floats, 2 threads a row
            const int m = t >> 1, kh = (t & 1) * 8;
            const bool ok = m0 + m < a.Co;
            const float* src = a.w + (int64_t)(m0 + m) * a.Kt + k0 + kh;
            const float4 v0 = ok ? *reinterpret_cast<const float4*>(src) : make_float4(0.f, 0.f, 0.f, 0.f);
            const float4 v1 = ok ? *reinterpret_cast<const float4*>(src + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
            ra[0] = v0.x; ra[1] = v0.y; ra[2] = v0.z; ra[3] = v0.w;
            ra[4] = v1.x; ra[5] = v1.y; ra[6] = v1.z; ra[7] = v1.w;
            // B[k][p] = X[img][ci][i*s + kh][j*s + kw]: item (group, pixel) = s floats
            const float* xi = a.x + (int64_t)img * a.Ci * a.H * a.W;
#pragma unroll
            for (int r = 0; r < 8 / S; ++r) {
                const int idx = t + kNT * r;
                const int gl = idx / kBN, p = idx % kBN;
                const int gg = k0 / S + gl;                 // global K group = ci * s + kh
                const int ci = gg / S, kh = gg - ci * S;
                const int pp = n0 + p;
                const bool okp = pp < a.P;
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
            for (int r = 0; r < 2; ++r) {
                const int idx = t + kNT * r;
                const int c = idx / 32, m4 = (idx % 32) * 4;
                const bool ok = m0 + m4 < a.Kt;
                const float4 v = ok ? *reinterpret_cast<const float4*>(a.w + (int64_t)(k0 + c) * a.Kt + m0 + m4)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
                ra[4 * r] = v.x; ra[4 * r + 1] = v.y; ra[4 * r + 2] = v.z; ra[4 * r + 3] = v.w;
            }
            // B[c][p] = G[img][k0 + c][n0 + p]: rows along p
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int idx = t + kNT * r;
                const int c = idx / 32, p4 = (idx % 32) * 4;
                const bool ok = n0 + p4 < a.P;
                const float4 v = ok ? *reinterpret_cast<const float4*>(
                                          a.g + ((int64_t)img * a.Co + k0 + c) * a.P + n0 + p4)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
                rb[4 * r] = v.x; rb[4 * r + 1] = v.y; rb[4 * r + 2] = v.z; rb[4 * r + 3] = v.w;
            }
        } else {
            // A[m][q] = G[img][m0 + m][k0 + q]: per row 16 contiguous floats (pixels)
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int idx = t + kNT * r;
                const int m = idx / 4, q4 = (idx % 4) * 4;
                const bool ok = m0 + m < a.Co;
                const float4 v = ok ? *reinterpret_cast<const float4*>(
                                          a.g + ((int64_t)img * a.Co + m0 + m) * a.P + k0 + q4)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
                ra[4 * r] = v.x; ra[4 * r + 1] = v.y; ra[4 * r + 2] = v.z; ra[4 * r + 3] = v.w;
            }
            // B[q][n] = Xp[n0 + n][k0 + q]: the 16 pixels of the chunk lie in one output row
            const int i = k0 / a.Wo, j0 = k0 - i * a.Wo;
            const float* xi = a.x + (int64_t)img * a.Ci * a.H * a.W;
#pragma unroll
            for (int r = 0; r < 8 / S; ++r) {
                const int idx = t + kNT * r;
                const int q = idx % kBK, gl = idx / kBK;
                const int gg = n0 / S + gl;
                const int ci = gg / S, kh = gg - ci * S;
                const bool ok = gg * S < a.Kt;
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

    // LDS chunk: As[k][m], Bs[k][n] (k-major rows of pitch kLD).
    __device__ void put(float* __restrict__ As, float* __restrict__ Bs) const
    {
        const int t = threadIdx.x;
        if constexpr (MODE == FWD) {
            const int m = t >> 1, kh = (t & 1) * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) As[(kh + e) * kLD + m] = ra[e];
#pragma unroll
            for (int r = 0; r < 8 / S; ++r) {
                const int idx = t + kNT * r;
                const int gl = idx / kBN, p = idx % kBN;
#pragma unroll
                for (int kw = 0; kw < S; ++kw) Bs[(gl * S + kw) * kLD + p] = rb[S * r + kw];
            }
        } else if constexpr (MODE == BWI) {
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int idx = t + kNT * r;
                const int c = idx / 32, x4 = (idx % 32) * 4;
                *reinterpret_cast<float4*>(As + c * kLD + x4) = make_float4(ra[4 * r], ra[4 * r + 1], ra[4 * r + 2], ra[4 * r + 3]);
                *reinterpret_cast<float4*>(Bs + c * kLD + x4) = make_float4(rb[4 * r], rb[4 * r + 1], rb[4 * r + 2], rb[4 * r + 3]);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int idx = t + kNT * r;
                const int m = idx / 4, q4 = (idx % 4) * 4;
#pragma unroll
                for (int e = 0; e < 4; ++e) As[(q4 + e) * kLD + m] = ra[4 * r + e];
            }
#pragma unroll
            for (int r = 0; r < 8 / S; ++r) {
                const int idx = t + kNT * r;
                const int q = idx % kBK, gl = idx / kBK;
#pragma unroll
                for (int kw = 0; kw < S; ++kw) Bs[q * kLD + gl * S + kw] = rb[S * r + kw];
            }
        }
    }
};

template <int MODE, int S>
__global__ void __launch_bounds__(kNT, 2)
patch_kernel(PArgs a)
{
    __shared__ __align__(16) float As[2][kBK * kLD];
    __shared__ __align__(16) float Bs[2][kBK * kLD];

    // tile -> (img or split, m tile, n tile); m fastest, so workgroups that
    // share the large operand (the pixels) run side by side
    int bid = blockIdx.x;
    const int mt = bid % a.tiles_m;
    bid /= a.tiles_m;
    const int nt = bid % a.tiles_n;
    const int outer = bid / a.tiles_n;           // image (FWD / BWI) or split (BWW)
    const int m0 = mt * kBM, n0 = nt * kBN;

    // reduction range in chunks of kBK
    int c_beg, c_end;
    if constexpr (MODE == FWD) { c_beg = 0; c_end = a.Kt / kBK; }
    else if constexpr (MODE == BWI) { c_beg = 0; c_end = a.Co / kBK; }
    else {
        c_beg = (int)((int64_t)outer * a.chunks / a.splits);
        c_end = (int)((int64_t)(outer + 1) * a.chunks / a.splits);
    }
    const int cpi = a.P / kBK;                   // BWW: chunks per image
    auto chunk_at = [&](int c, int& img, int& k0) {
        if constexpr (MODE == BWW) { img = c / cpi; k0 = (c - img * cpi) * kBK; }
        else { img = outer; k0 = c * kBK; }
    };

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int hi = lane >> 5, l32 = lane & 31;
    f32x16 acc[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.f;
    float bias_acc = 0.f;
    const bool with_bias = MODE == BWW && a.outb && nt == 0;

    Stage<MODE, S> st;
    if (c_beg < c_end) {
        int img, k0;
        chunk_at(c_beg, img, k0);
        st.load(a, img, m0, n0, k0);
    }
    for (int c = c_beg, it = 0; c < c_end; ++c, ++it) {
        float* as = As[it & 1];
        float* bs = Bs[it & 1];
        st.put(as, bs);
        lds_barrier();
        if (c + 1 < c_end) {
            int img, k0;
            chunk_at(c + 1, img, k0);
            st.load(a, img, m0, n0, k0);
        }
        if (with_bias && threadIdx.x < kBM) {
#pragma unroll
            for (int q = 0; q < kBK; ++q) bias_acc += as[q * kLD + threadIdx.x];
        }
        const float* ap = as + hi * kLD + wm * 64 + l32;
        const float* bp = bs + hi * kLD + wn * 64 + l32;
#pragma unroll
        for (int s2 = 0; s2 < kBK / 2; ++s2) {
            const float a0 = ap[2 * s2 * kLD], a1 = ap[2 * s2 * kLD + 32];
            const float b0 = bp[2 * s2 * kLD], b1 = bp[2 * s2 * kLD + 32];
            acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
        }
        // the buffer just read is rewritten two chunks later, after the next barrier
    }

    // D block (x, y): register 4 q + r holds row 4 hi + 8 q + r, column l32
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) {
            const int rb = m0 + wm * 64 + x * 32;     // block's first row (a multiple of 4)
            const int col = n0 + wn * 64 + y * 32 + l32;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row = rb + 4 * hi + 8 * q;  // rows row .. row + 3 in registers 4q .. 4q + 3
                if constexpr (MODE == FWD) {
                    if (col < a.P) {
                        float* yp = a.out + ((int64_t)outer * a.Co) * a.P + col;
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (row + r < a.Co)
                                yp[(int64_t)(row + r) * a.P] = acc[x][y][4 * q + r] + (a.b ? a.b[row + r] : 0.f);
                    }
                } else if constexpr (MODE == BWI) {
                    // rows = K = (ci, kh, kw), kw fastest: the 4 registers are s-wide runs of kw
                    if (col < a.P && row < a.Kt) {
                        const int i = col / a.Wo, j = col - i * a.Wo;
                        float* dxi = a.out + (int64_t)outer * a.Ci * a.H * a.W;
                        if constexpr (S == 4) {
                            const int ci = row / 16, kh = (row / 4) % 4;
                            *reinterpret_cast<float4*>(dxi + ((int64_t)ci * a.H + i * 4 + kh) * a.W + j * 4) =
                                make_float4(acc[x][y][4 * q], acc[x][y][4 * q + 1], acc[x][y][4 * q + 2],
                                            acc[x][y][4 * q + 3]);
                        } else {
#pragma unroll
                            for (int h = 0; h < 2; ++h) {
                                const int rr = row + 2 * h;
                                const int ci = rr / 4, kh = (rr / 2) % 2;
                                *reinterpret_cast<float2*>(dxi + ((int64_t)ci * a.H + i * 2 + kh) * a.W + j * 2) =
                                    make_float2(acc[x][y][4 * q + 2 * h], acc[x][y][4 * q + 2 * h + 1]);
                            }
                        }
                    }
                } else {
                    if (col < a.Kt) {
                        float* wp = a.out + ((int64_t)outer * a.Co) * a.Kt + col;
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (row + r < a.Co) wp[(int64_t)(row + r) * a.Kt] = acc[x][y][4 * q + r];
                    }
                }
            }
        }
    if (with_bias && threadIdx.x < kBM && m0 + threadIdx.x < a.Co)
        a.outb[(int64_t)outer * a.Co + m0 + threadIdx.x] = bias_acc;
}

// grad_w[co][K] = sum over splits of the partials, in split order (float4 along K).
__global__ void __launch_bounds__(256)
patch_reduce_kernel(const float* __restrict__ ws, const float* __restrict__ wsb, int splits, int Co, int Kt,
                    float* __restrict__ gw, float* __restrict__ gb)
{
    const int64_t n4 = (int64_t)Co * Kt / 4;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx < n4) {
        const float4* p = reinterpret_cast<const float4*>(ws) + idx;
        float4 s = p[0];
        for (int k = 1; k < splits; ++k) {
            const float4 v = p[(int64_t)k * n4];
            s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
        }
        reinterpret_cast<float4*>(gw)[idx] = s;
    } else if (gb && idx < n4 + Co) {
        const int co = (int)(idx - n4);
        float s = wsb[co];
        for (int k = 1; k < splits; ++k) s += wsb[(int64_t)k * Co + co];
        gb[co] = s;
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

int wgrad_splits(const PArgs& a, int tiles)
{
    const int chunks = a.N * (a.P / kBK);
    int s = (1024 + tiles - 1) / tiles;
    if (s > chunks) s = chunks;
    return s < 1 ? 1 : s;
}

template <int MODE>
hipError_t launch(const PArgs& a, int s, int grid, hipStream_t st)
{
    if (s == 2) hipLaunchKernelGGL((patch_kernel<MODE, 2>), dim3(grid), dim3(kNT), 0, st, a);
    else hipLaunchKernelGGL((patch_kernel<MODE, 4>), dim3(grid), dim3(kNT), 0, st, a);
    return hipGetLastError();
}

}  // namespace

bool patch_supported(const Geom& g)
{
    const int64_t p = (int64_t)g.ho * g.wol;
    return g.groups == 1 && g.pad == 0 && g.k == g.stride && (g.k == 2 || g.k == 4) &&
           (g.ci * g.k * g.k) % kBK == 0 && g.co % kBK == 0 && g.wol % kBK == 0 && g.h == g.ho * g.k &&
           g.wl == g.wol * g.k && (int64_t)g.n * g.ci * g.h * g.wl < ((int64_t)1 << 31) &&
           (int64_t)g.n * g.co * p < ((int64_t)1 << 31);
}

size_t patch_wgrad_workspace_bytes(const Geom& g)
{
    const PArgs a = make_args(g);
    const int tiles = ((a.Co + kBM - 1) / kBM) * ((a.Kt + kBN - 1) / kBN);
    const int64_t s = wgrad_splits(a, tiles);
    return (size_t)(s * a.Co * (int64_t)(a.Kt + 1)) * sizeof(float);
}

hipError_t launch_patch_fwd(const Geom& g, const float* x, const float* w, const float* b, float* y,
                            hipStream_t st)
{
    PArgs a = make_args(g);
    a.x = x; a.w = w; a.b = b; a.out = y;
    a.tiles_m = (a.Co + kBM - 1) / kBM;
    a.tiles_n = (a.P + kBN - 1) / kBN;
    return launch<FWD>(a, g.k, a.tiles_m * a.tiles_n * a.N, st);
}

hipError_t launch_patch_bwd_input(const Geom& g, const float* gy, const float* w, float* gx, hipStream_t st)
{
    PArgs a = make_args(g);
    a.g = gy; a.w = w; a.out = gx;
    a.tiles_m = (a.Kt + kBM - 1) / kBM;
    a.tiles_n = (a.P + kBN - 1) / kBN;
    return launch<BWI>(a, g.k, a.tiles_m * a.tiles_n * a.N, st);
}

hipError_t launch_patch_bwd_weight(const Geom& g, const float* x, const float* gy, float* gw, float* gb,
                                   void* ws, hipStream_t st)
{
    PArgs a = make_args(g);
    a.x = x; a.g = gy;
    a.tiles_m = (a.Co + kBM - 1) / kBM;
    a.tiles_n = (a.Kt + kBN - 1) / kBN;
    a.chunks = a.N * (a.P / kBK);
    a.splits = wgrad_splits(a, a.tiles_m * a.tiles_n);
    float* wsf = static_cast<float*>(ws);
    a.out = wsf;
    a.outb = wsf + (int64_t)a.splits * a.Co * a.Kt;
    hipError_t e = launch<BWW>(a, g.k, a.tiles_m * a.tiles_n * a.splits, st);
    if (e != hipSuccess) return e;
    const int64_t total = (int64_t)a.Co * a.Kt / 4 + a.Co;
    hipLaunchKernelGGL(patch_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, a.out, a.outb,
                       a.splits, a.Co, a.Kt, gw, gb);
    return hipGetLastError();
}

}  // namespace sscnn
