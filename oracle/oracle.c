/*
 * oracle.c -- plain CPU oracle for the width-sharded 2-D convolution.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file; only the test-suite, the package smoke check and the
 * benchmark's CPU-baseline leg load it.  It shares no source, header, helper
 * or build flag with the HIP kernels.
 *
 * What it computes.  The sharded convolution of the pages reaches, up to
 * floating-point summation order, exactly the result of the ordinary
 * (unsharded) convolution: NVIDIA blog "Perception Model Training for
 * Autonomous Vehicles with Tensor Parallelism" (DTensor section: the input,
 * activation and output are Shard(3) on W, weight and bias are Replicate, and
 * grad_weight / grad_bias come out of backward as _Partial), and the kwkr.cn
 * retelling of it (section 2.2: halo exchange, concatenate, convolve, crop the
 * columns produced by the invalid padding).  So the oracle is the plain
 * definition of PyTorch's conv2d (cross-correlation with zero padding, square
 * kernel, stride, groups) and of its two gradients, evaluated on the GLOBAL
 * tensors and restricted to one shard's column range.  It never forms a halo,
 * so it checks the halo logic of the product independently.
 *
 * Arithmetic: double inputs (float32 values promoted exactly by the caller),
 * double accumulation, double outputs.  Every output element is computed by
 * one direct nested loop in the order the definition states; OpenMP only
 * spreads different output elements over threads, never one sum.
 *
 * Layouts: activations NCHW, weight OIHW with I = C_in / groups, all
 * contiguous, row-major.
 */
#include <stdint.h>
#include <stddef.h>
#include <omp.h>

/* Output extent of a convolution along one axis. */
int oracle_out_size(int in, int k, int stride, int pad)
{
    return (in + 2 * pad - k) / stride + 1;
}

/* ---------------------------------------------------------------------------
 * Forward.  y[b,o,i,j] = bias[o] + sum over c < Cig, kh < K, kw < K of
 *     wt[o,c,kh,kw] * x[b, g*Cig + c, i*stride + kh - pad, j*stride + kw - pad]
 * with g = o / Cog and x taken as zero outside [0,H) x [0,W).
 * ------------------------------------------------------------------------- */
static double fwd_elem(const double *x, int n, int ci, int h, int w,
                       const double *wt, int co, int k, int stride, int pad,
                       int groups, const double *bias, int b, int o, int i, int j)
{
    int cig = ci / groups, cog = co / groups, g = o / cog;
    double acc = bias ? bias[o] : 0.0;
    (void)n;
    for (int c = 0; c < cig; c++) {
        int cin = g * cig + c;
        for (int kh = 0; kh < k; kh++) {
            int r = i * stride + kh - pad;
            if (r < 0 || r >= h) continue;
            for (int kw = 0; kw < k; kw++) {
                int q = j * stride + kw - pad;
                if (q < 0 || q >= w) continue;
                acc += wt[(((int64_t)o * cig + c) * k + kh) * k + kw] *
                       x[(((int64_t)b * ci + cin) * h + r) * w + q];
            }
        }
    }
    return acc;
}

/* Full forward over output columns [j0, j1): y has shape (N, Co, Ho, j1-j0). */
void oracle_conv_fwd(const double *x, int n, int ci, int h, int w,
                     const double *wt, int co, int k, int stride, int pad,
                     int groups, const double *bias, int j0, int j1, double *y)
{
    int ho = oracle_out_size(h, k, stride, pad);
    int wy = j1 - j0;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < n; b++)
        for (int o = 0; o < co; o++)
            for (int i = 0; i < ho; i++)
                for (int j = j0; j < j1; j++)
                    y[(((int64_t)b * co + o) * ho + i) * wy + (j - j0)] =
                        fwd_elem(x, n, ci, h, w, wt, co, k, stride, pad, groups,
                                 bias, b, o, i, j);
}

/* Forward at listed output positions idx[4*s .. 4*s+3] = (b, o, i, j). */
void oracle_conv_fwd_at(const double *x, int n, int ci, int h, int w,
                        const double *wt, int co, int k, int stride, int pad,
                        int groups, const double *bias, int64_t count,
                        const int64_t *idx, double *out)
{
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t s = 0; s < count; s++)
        out[s] = fwd_elem(x, n, ci, h, w, wt, co, k, stride, pad, groups, bias,
                          (int)idx[4 * s], (int)idx[4 * s + 1],
                          (int)idx[4 * s + 2], (int)idx[4 * s + 3]);
}

/* ---------------------------------------------------------------------------
 * Gradient with respect to the input (the adjoint of the forward map).
 * dx[b,c,y,xx] = sum over o in the group of c, kh, kw such that
 *   y + pad - kh = i*stride and xx + pad - kw = j*stride with 0 <= i < Ho and
 *   0 <= j < Wo, of  wt[o, c mod Cig, kh, kw] * g[b, o, i, j].
 * ------------------------------------------------------------------------- */
static double bwd_input_elem(const double *g, int co, int ho, int wo,
                             const double *wt, int ci, int k, int stride,
                             int pad, int groups, int b, int c, int y, int xx)
{
    int cig = ci / groups, cog = co / groups, grp = c / cig, cl = c % cig;
    double acc = 0.0;
    for (int o = grp * cog; o < (grp + 1) * cog; o++) {
        for (int kh = 0; kh < k; kh++) {
            int t = y + pad - kh;
            if (t < 0 || t % stride != 0) continue;
            int i = t / stride;
            if (i >= ho) continue;
            for (int kw = 0; kw < k; kw++) {
                int u = xx + pad - kw;
                if (u < 0 || u % stride != 0) continue;
                int j = u / stride;
                if (j >= wo) continue;
                acc += wt[(((int64_t)o * cig + cl) * k + kh) * k + kw] *
                       g[(((int64_t)b * co + o) * ho + i) * wo + j];
            }
        }
    }
    return acc;
}

/* Full grad_input over input columns [x0, x1): dx has shape (N, Ci, H, x1-x0).
 * g is the GLOBAL grad_output (N, Co, Ho, Wo). */
void oracle_conv_bwd_input(const double *g, int n, int co, int ho, int wo,
                           const double *wt, int ci, int h, int k, int stride,
                           int pad, int groups, int x0, int x1, double *dx)
{
    int wx = x1 - x0;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < n; b++)
        for (int c = 0; c < ci; c++)
            for (int y = 0; y < h; y++)
                for (int xx = x0; xx < x1; xx++)
                    dx[(((int64_t)b * ci + c) * h + y) * wx + (xx - x0)] =
                        bwd_input_elem(g, co, ho, wo, wt, ci, k, stride, pad,
                                       groups, b, c, y, xx);
}

/* grad_input at listed positions idx[4*s ..] = (b, c, y, x). */
void oracle_conv_bwd_input_at(const double *g, int n, int co, int ho, int wo,
                              const double *wt, int ci, int h, int k,
                              int stride, int pad, int groups, int64_t count,
                              const int64_t *idx, double *out)
{
    (void)n; (void)h;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t s = 0; s < count; s++)
        out[s] = bwd_input_elem(g, co, ho, wo, wt, ci, k, stride, pad, groups,
                                (int)idx[4 * s], (int)idx[4 * s + 1],
                                (int)idx[4 * s + 2], (int)idx[4 * s + 3]);
}

/* ---------------------------------------------------------------------------
 * Gradient with respect to the weight, summed over the output columns
 * [j0, j1) only -- the _Partial a shard owns when [j0, j1) is its own output
 * column range; the full gradient is the same sum over every column.
 * gw[o,c,kh,kw] = sum over b, i < Ho, j in [j0,j1) of
 *     g[b,o,i,j] * x[b, grp*Cig + c, i*stride + kh - pad, j*stride + kw - pad]
 * (x zero outside the image).  gb[o] = sum over b, i, j in [j0,j1) of g[b,o,i,j].
 * ------------------------------------------------------------------------- */
static double bwd_weight_elem(const double *x, const double *g, int n, int ci,
                              int h, int w, int co, int k, int stride, int pad,
                              int groups, int j0, int j1, int o, int c, int kh,
                              int kw)
{
    int cig = ci / groups, cog = co / groups, cin = (o / cog) * cig + c;
    int ho = oracle_out_size(h, k, stride, pad);
    int wo = oracle_out_size(w, k, stride, pad);
    double acc = 0.0;
    for (int b = 0; b < n; b++)
        for (int i = 0; i < ho; i++) {
            int r = i * stride + kh - pad;
            if (r < 0 || r >= h) continue;
            for (int j = j0; j < j1; j++) {
                int q = j * stride + kw - pad;
                if (q < 0 || q >= w) continue;
                acc += g[(((int64_t)b * co + o) * ho + i) * wo + j] *
                       x[(((int64_t)b * ci + cin) * h + r) * w + q];
            }
        }
    return acc;
}

static double bwd_bias_elem(const double *g, int n, int co, int ho, int wo,
                            int j0, int j1, int o)
{
    double acc = 0.0;
    for (int b = 0; b < n; b++)
        for (int i = 0; i < ho; i++)
            for (int j = j0; j < j1; j++)
                acc += g[(((int64_t)b * co + o) * ho + i) * wo + j];
    return acc;
}

/* Full grad_weight (Co, Cig, K, K) and grad_bias (Co) over columns [j0, j1).
 * gb may be NULL. */
void oracle_conv_bwd_weight(const double *x, const double *g, int n, int ci,
                            int h, int w, int co, int k, int stride, int pad,
                            int groups, int j0, int j1, double *gw, double *gb)
{
    int cig = ci / groups;
    int ho = oracle_out_size(h, k, stride, pad);
    int wo = oracle_out_size(w, k, stride, pad);
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int o = 0; o < co; o++)
        for (int c = 0; c < cig; c++)
            for (int kh = 0; kh < k; kh++)
                for (int kw = 0; kw < k; kw++)
                    gw[(((int64_t)o * cig + c) * k + kh) * k + kw] =
                        bwd_weight_elem(x, g, n, ci, h, w, co, k, stride, pad,
                                        groups, j0, j1, o, c, kh, kw);
    if (gb) {
#pragma omp parallel for
        for (int o = 0; o < co; o++)
            gb[o] = bwd_bias_elem(g, n, co, ho, wo, j0, j1, o);
    }
}

/* grad_bias alone (Co) over output columns [j0, j1). */
void oracle_conv_bwd_bias(const double *g, int n, int co, int ho, int wo,
                          int j0, int j1, double *gb)
{
#pragma omp parallel for
    for (int o = 0; o < co; o++)
        gb[o] = bwd_bias_elem(g, n, co, ho, wo, j0, j1, o);
}

/* grad_weight at listed positions idx[4*s ..] = (o, c, kh, kw), summed over
 * output columns [j0, j1). */
void oracle_conv_bwd_weight_at(const double *x, const double *g, int n, int ci,
                               int h, int w, int co, int k, int stride,
                               int pad, int groups, int j0, int j1,
                               int64_t count, const int64_t *idx, double *out)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t s = 0; s < count; s++)
        out[s] = bwd_weight_elem(x, g, n, ci, h, w, co, k, stride, pad, groups,
                                 j0, j1, (int)idx[4 * s], (int)idx[4 * s + 1],
                                 (int)idx[4 * s + 2], (int)idx[4 * s + 3]);
}

/* Number of OpenMP threads the oracle runs on (reported beside its timing). */
int oracle_num_threads(void)
{
    return omp_get_max_threads();
}
