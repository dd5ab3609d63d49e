// api.cpp -- the C ABI of libsscnn (declared in include/sscnn.h): host-side
// validation of every argument, then dispatch to the kernel family that fits
// the layer.  Nothing here allocates device memory.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "blockops.h"
#include "patchify.h"
#include "depthwise.h"
#include "edge.h"
#include "internal.h"
#include "kernels.h"
#include "mfma_conv.h"
#include "rowedge.h"

namespace sscnn {
namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return code;
}

int hip_status(hipError_t e, const char* what)
{
    if (e == hipSuccess) return SSCNN_OK;
    return fail(SSCNN_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Derived fields of a layer; returns a status and fills *out.
int derive(const sscnn_conv_t& c, sscnn_conv_t* out)
{
    if (c.n <= 0 || c.c_in <= 0 || c.c_out <= 0 || c.h <= 0 || c.w_local <= 0 || c.k <= 0 ||
        c.stride <= 0 || c.groups <= 0 || c.num_shards <= 0)
        return fail(SSCNN_EINVAL, "sizes must be positive (n=%d c_in=%d c_out=%d h=%d w_local=%d "
                    "k=%d stride=%d groups=%d num_shards=%d)", c.n, c.c_in, c.c_out, c.h, c.w_local,
                    c.k, c.stride, c.groups, c.num_shards);
    if (c.pad < 0 || c.pad >= c.k) return fail(SSCNN_EINVAL, "pad=%d must satisfy 0 <= pad < k=%d", c.pad, c.k);
    if (c.c_in % c.groups || c.c_out % c.groups)
        return fail(SSCNN_EINVAL, "groups=%d must divide c_in=%d and c_out=%d", c.groups, c.c_in, c.c_out);
    if (c.shard < 0 || c.shard >= c.num_shards)
        return fail(SSCNN_EINVAL, "shard=%d outside [0, %d)", c.shard, c.num_shards);
    if (c.h + 2 * c.pad < c.k) return fail(SSCNN_EINVAL, "h=%d too small for k=%d pad=%d", c.h, c.k, c.pad);
    const int64_t elems_in = (int64_t)c.n * c.c_in * c.h * c.w_local;
    if (elems_in > ((int64_t)1 << 40)) return fail(SSCNN_EINVAL, "tensor too large");
    if (c.w_local % c.stride)
        return fail(SSCNN_EUNSUPPORTED, "w_local=%d is not a multiple of stride=%d", c.w_local, c.stride);
    const int64_t w_global = (int64_t)c.w_local * c.num_shards;
    const int64_t wo_global = (w_global + 2 * c.pad - c.k) / c.stride + 1;
    if (wo_global != w_global / c.stride)
        return fail(SSCNN_EUNSUPPORTED, "global output width %lld != %lld: output columns do not "
                    "split evenly over the shards", (long long)wo_global, (long long)(w_global / c.stride));
    sscnn_conv_t d = c;
    d.h_out = (c.h + 2 * c.pad - c.k) / c.stride + 1;
    d.w_out_local = c.w_local / c.stride;
    d.halo_l = c.pad;
    d.halo_r = c.k - c.stride - c.pad > 0 ? c.k - c.stride - c.pad : 0;
    d.ghalo_l = (c.k - 1 - c.pad) / c.stride;
    d.ghalo_r = (c.pad + c.stride - 1) / c.stride;
    if (d.halo_l > c.w_local || d.halo_r > c.w_local || d.ghalo_l > d.w_out_local ||
        d.ghalo_r > d.w_out_local)
        return fail(SSCNN_EUNSUPPORTED, "halo wider than one slice (halo %d/%d, grad halo %d/%d, "
                    "w_local %d)", d.halo_l, d.halo_r, d.ghalo_l, d.ghalo_r, c.w_local);
    *out = d;
    return SSCNN_OK;
}

// Re-derive and compare, so a descriptor edited after sscnn_conv_init is caught.
int check(const sscnn_conv_t* conv, Geom* g)
{
    if (!conv) return fail(SSCNN_EINVAL, "conv is NULL");
    sscnn_conv_t d;
    int st = derive(*conv, &d);
    if (st) return st;
    if (d.h_out != conv->h_out || d.w_out_local != conv->w_out_local || d.halo_l != conv->halo_l ||
        d.halo_r != conv->halo_r || d.ghalo_l != conv->ghalo_l || d.ghalo_r != conv->ghalo_r)
        return fail(SSCNN_EINVAL, "descriptor not initialised by sscnn_conv_init (or edited since)");
    g->n = d.n; g->ci = d.c_in; g->co = d.c_out; g->h = d.h; g->wl = d.w_local; g->k = d.k;
    g->stride = d.stride; g->pad = d.pad; g->groups = d.groups; g->ho = d.h_out;
    g->wol = d.w_out_local; g->hl = d.halo_l; g->hr = d.halo_r; g->ghl = d.ghalo_l;
    g->ghr = d.ghalo_r; g->cig = d.c_in / d.groups; g->cog = d.c_out / d.groups;
    return SSCNN_OK;
}

// Height sharding: validate an H-shard descriptor and derive its fields.
int derive_h(const sscnn_hconv_t& c, sscnn_hconv_t* out)
{
    if (c.n <= 0 || c.c_in <= 0 || c.c_out <= 0 || c.h_local <= 0 || c.w <= 0 || c.k <= 0 || c.stride <= 0 ||
        c.groups <= 0 || c.num_shards <= 0)
        return fail(SSCNN_EINVAL, "sizes must be positive (n=%d c_in=%d c_out=%d h_local=%d w=%d k=%d "
                    "stride=%d groups=%d num_shards=%d)", c.n, c.c_in, c.c_out, c.h_local, c.w, c.k, c.stride,
                    c.groups, c.num_shards);
    if (c.pad < 0 || c.pad >= c.k) return fail(SSCNN_EINVAL, "pad=%d must satisfy 0 <= pad < k=%d", c.pad, c.k);
    if (c.c_in % c.groups || c.c_out % c.groups)
        return fail(SSCNN_EINVAL, "groups=%d must divide c_in=%d and c_out=%d", c.groups, c.c_in, c.c_out);
    if (c.shard < 0 || c.shard >= c.num_shards)
        return fail(SSCNN_EINVAL, "shard=%d outside [0, %d)", c.shard, c.num_shards);
    if (c.w + 2 * c.pad < c.k) return fail(SSCNN_EINVAL, "w=%d too small for k=%d pad=%d", c.w, c.k, c.pad);
    if ((int64_t)c.n * c.c_in * c.h_local * c.w > ((int64_t)1 << 40)) return fail(SSCNN_EINVAL, "tensor too large");
    if (c.h_local % c.stride || c.w % c.stride)
        return fail(SSCNN_EUNSUPPORTED, "h_local=%d and w=%d must be multiples of stride=%d", c.h_local, c.w,
                    c.stride);
    const int64_t h_global = (int64_t)c.h_local * c.num_shards;
    if ((h_global + 2 * c.pad - c.k) / c.stride + 1 != h_global / c.stride)
        return fail(SSCNN_EUNSUPPORTED, "output rows do not split evenly over the shards");
    if ((c.w + 2 * c.pad - c.k) / c.stride + 1 != c.w / c.stride)
        return fail(SSCNN_EUNSUPPORTED, "output width %d != w / stride = %d", (c.w + 2 * c.pad - c.k) / c.stride + 1,
                    c.w / c.stride);
    sscnn_hconv_t d = c;
    d.h_out_local = c.h_local / c.stride;
    d.w_out = c.w / c.stride;
    d.halo_u = c.pad;
    d.halo_d = c.k - c.stride - c.pad > 0 ? c.k - c.stride - c.pad : 0;
    d.ghalo_u = (c.k - 1 - c.pad) / c.stride;
    d.ghalo_d = (c.pad + c.stride - 1) / c.stride;
    if (d.halo_u > c.h_local || d.halo_d > c.h_local || d.ghalo_u > d.h_out_local || d.ghalo_d > d.h_out_local)
        return fail(SSCNN_EUNSUPPORTED, "row halo taller than one slice (halo %d/%d, grad halo %d/%d, h_local %d)",
                    d.halo_u, d.halo_d, d.ghalo_u, d.ghalo_d, c.h_local);
    *out = d;
    return SSCNN_OK;
}

// The slice as its own image (the interior of an H-shard), for the ordinary
// kernels; its column halos are never passed (read as zeros: the image's
// padding).
int check_h(const sscnn_hconv_t* conv, Geom* g)
{
    if (!conv) return fail(SSCNN_EINVAL, "conv is NULL");
    sscnn_hconv_t d;
    int st = derive_h(*conv, &d);
    if (st) return st;
    if (d.h_out_local != conv->h_out_local || d.w_out != conv->w_out || d.halo_u != conv->halo_u ||
        d.halo_d != conv->halo_d || d.ghalo_u != conv->ghalo_u || d.ghalo_d != conv->ghalo_d)
        return fail(SSCNN_EINVAL, "descriptor not initialised by sscnn_hconv_init (or edited since)");
    g->n = d.n; g->ci = d.c_in; g->co = d.c_out; g->h = d.h_local; g->wl = d.w; g->k = d.k;
    g->stride = d.stride; g->pad = d.pad; g->groups = d.groups; g->ho = d.h_out_local; g->wol = d.w_out;
    g->hl = d.pad; g->hr = d.k - d.stride - d.pad > 0 ? d.k - d.stride - d.pad : 0;
    g->ghl = (d.k - 1 - d.pad) / d.stride; g->ghr = (d.pad + d.stride - 1) / d.stride;
    g->cig = d.c_in / d.groups; g->cog = d.c_out / d.groups;
    return SSCNN_OK;
}

// 2-D shards: the supported layers and their derived fields.
int derive_g(const sscnn_gconv_t& c, sscnn_gconv_t* out)
{
    if (c.n <= 0 || c.c_in <= 0 || c.c_out <= 0 || c.h_local <= 0 || c.w_local <= 0 || c.k <= 0 || c.stride <= 0 ||
        c.groups <= 0 || c.num_h <= 0 || c.num_w <= 0)
        return fail(SSCNN_EINVAL, "sizes must be positive");
    if (c.shard_h < 0 || c.shard_h >= c.num_h || c.shard_w < 0 || c.shard_w >= c.num_w)
        return fail(SSCNN_EINVAL, "shard (%d, %d) outside the %d x %d grid", c.shard_h, c.shard_w, c.num_h, c.num_w);
    if ((int64_t)c.n * c.c_in * c.h_local * c.w_local > ((int64_t)1 << 40)) return fail(SSCNN_EINVAL, "tensor too large");
    sscnn_gconv_t d = c;
    const bool dw = c.groups == c.c_in && c.c_in == c.c_out && c.stride == 1 && (c.k == 3 || c.k == 5 || c.k == 7) &&
                    c.pad == c.k / 2;
    const bool patch = c.k == c.stride && c.pad == 0 && c.groups == 1;
    const bool dense = c.groups == 1 && c.stride == 1 && (c.k == 3 || c.k == 5) && c.pad == c.k / 2;
    if (dw) {
        if (c.w_local % 16 || c.h_local < 16)
            return fail(SSCNN_EUNSUPPORTED, "2-D depthwise blocks need w_local %% 16 == 0 and h_local >= 16 "
                        "(got %d x %d)", c.h_local, c.w_local);
        if ((int64_t)c.n * c.c_in * c.h_local * c.w_local >= ((int64_t)1 << 31))
            return fail(SSCNN_EUNSUPPORTED, "2-D depthwise block of 2^31 elements or more");
        d.h_out_local = c.h_local;
        d.w_out_local = c.w_local;
        d.halo = c.pad;
    } else if (patch) {
        if (c.h_local % c.k || c.w_local % c.k)
            return fail(SSCNN_EUNSUPPORTED, "block %d x %d is not a whole number of %d x %d patches", c.h_local,
                        c.w_local, c.k, c.k);
        d.h_out_local = c.h_local / c.k;
        d.w_out_local = c.w_local / c.k;
        d.halo = 0;
    } else if (dense) {
        if (c.c_in < 16 || c.c_out < 16 || c.c_in % 4 || c.c_out % 4 || c.w_local % 4)
            return fail(SSCNN_EUNSUPPORTED, "2-D dense blocks need c_in, c_out multiples of 4 and at least 16, and "
                        "w_local %% 4 == 0 (got c_in=%d c_out=%d w_local=%d)", c.c_in, c.c_out, c.w_local);
        if (c.h_local < c.pad || c.w_local < c.pad)
            return fail(SSCNN_EUNSUPPORTED, "block %d x %d is smaller than the halo %d", c.h_local, c.w_local, c.pad);
        d.h_out_local = c.h_local;
        d.w_out_local = c.w_local;
        d.halo = c.pad;
    } else {
        return fail(SSCNN_EUNSUPPORTED, "2-D shards take depthwise stride-1 k/2-padded layers, dense stride-1 "
                    "3x3 / 5x5 k/2-padded layers and k = stride layers only (k=%d stride=%d pad=%d groups=%d)",
                    c.k, c.stride, c.pad, c.groups);
    }
    *out = d;
    return SSCNN_OK;
}

int check_g(const sscnn_gconv_t* conv, Geom* g)
{
    if (!conv) return fail(SSCNN_EINVAL, "conv is NULL");
    sscnn_gconv_t d;
    int st = derive_g(*conv, &d);
    if (st) return st;
    if (d.h_out_local != conv->h_out_local || d.w_out_local != conv->w_out_local || d.halo != conv->halo)
        return fail(SSCNN_EINVAL, "descriptor not initialised by sscnn_gconv_init (or edited since)");
    g->n = d.n; g->ci = d.c_in; g->co = d.c_out; g->h = d.h_local; g->wl = d.w_local; g->k = d.k;
    g->stride = d.stride; g->pad = d.pad; g->groups = d.groups; g->ho = d.h_out_local; g->wol = d.w_out_local;
    g->hl = g->hr = g->ghl = g->ghr = d.halo;
    g->cig = d.c_in / d.groups; g->cog = d.c_out / d.groups;
    return SSCNN_OK;
}

// The workspace check shared by the grad_weight calls (rows: also the
// row-edge grad_weight's scratch, used after the interior call is done with
// its own).
int need_workspace(const Geom& g, void* workspace, size_t workspace_bytes, size_t* ws_need, bool rows = false)
{
    *ws_need = kernels_bwd_weight_workspace_bytes(g);
    if (rows && row_edge_workspace_bytes(g) > *ws_need) *ws_need = row_edge_workspace_bytes(g);
    if (*ws_need) {
        if (!workspace || workspace_bytes < *ws_need)
            return fail(SSCNN_EWORKSPACE, "workspace of %zu bytes given, %zu needed",
                        workspace ? workspace_bytes : (size_t)0, *ws_need);
        if (reinterpret_cast<uintptr_t>(workspace) & 15u)
            return fail(SSCNN_EINVAL, "workspace is not 16-byte aligned");
    }
    return SSCNN_OK;
}

int need(const void* p, const char* name)
{
    if (!p) return fail(SSCNN_EINVAL, "%s is NULL", name);
    if (!aligned16(p)) return fail(SSCNN_EINVAL, "%s is not 16-byte aligned", name);
    return SSCNN_OK;
}

int optional(const void* p, const char* name)
{
    if (p && !aligned16(p)) return fail(SSCNN_EINVAL, "%s is not 16-byte aligned", name);
    return SSCNN_OK;
}

#define TRY(expr)                  \
    do {                           \
        int st_ = (expr);          \
        if (st_) return st_;       \
    } while (0)

}  // namespace
}  // namespace sscnn

using namespace sscnn;

extern "C" {

int sscnn_abi_version(void) { return SSCNN_ABI_VERSION; }

const char* sscnn_status_string(int status)
{
    switch (status) {
        case SSCNN_OK: return "ok";
        case SSCNN_EINVAL: return "invalid argument";
        case SSCNN_EUNSUPPORTED: return "unsupported layer for width sharding";
        case SSCNN_EWORKSPACE: return "workspace missing or too small";
        case SSCNN_EHIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* sscnn_last_error(void) { return g_last_error; }

int sscnn_conv_init(sscnn_conv_t* conv)
{
    if (!conv) return fail(SSCNN_EINVAL, "conv is NULL");
    sscnn_conv_t d;
    TRY(derive(*conv, &d));
    *conv = d;
    return SSCNN_OK;
}

int sscnn_halo_gather(const sscnn_conv_t* conv, int32_t which, const float* left_nbr,
                      const float* right_nbr, float* halo, void* stream)
{
    Geom g;
    TRY(check(conv, &g));
    int64_t planes;
    int rows, width, hl, hr;
    if (which == SSCNN_HALO_INPUT) {
        planes = (int64_t)g.n * g.ci; rows = g.h; width = g.wl; hl = g.hl; hr = g.hr;
    } else if (which == SSCNN_HALO_GRAD_OUTPUT) {
        planes = (int64_t)g.n * g.co; rows = g.ho; width = g.wol; hl = g.ghl; hr = g.ghr;
    } else {
        return fail(SSCNN_EINVAL, "which=%d is neither SSCNN_HALO_INPUT nor SSCNN_HALO_GRAD_OUTPUT", which);
    }
    const bool first = conv->shard == 0, last = conv->shard == conv->num_shards - 1;
    if (first != (left_nbr == nullptr))
        return fail(SSCNN_EINVAL, "left_nbr must be NULL exactly for shard 0 (shard=%d)", conv->shard);
    if (last != (right_nbr == nullptr))
        return fail(SSCNN_EINVAL, "right_nbr must be NULL exactly for the last shard (shard=%d)", conv->shard);
    TRY(optional(left_nbr, "left_nbr"));
    TRY(optional(right_nbr, "right_nbr"));
    if (hl + hr == 0) return SSCNN_OK;
    TRY(need(halo, "halo"));
    return hip_status(launch_halo_gather(hl ? left_nbr : nullptr, hr ? right_nbr : nullptr, planes,
                                         rows, width, hl, hr, halo, (hipStream_t)stream),
                      "halo_gather launch");
}

int sscnn_conv_fwd(const sscnn_conv_t* conv, const float* x, const float* x_halo,
                   const float* weight, const float* bias, float* y, void* stream)
{
    Geom g;
    TRY(check(conv, &g));
    TRY(need(x, "x"));
    if (g.hl + g.hr) TRY(need(x_halo, "x_halo")); else TRY(optional(x_halo, "x_halo"));
    TRY(need(weight, "weight"));
    TRY(optional(bias, "bias"));
    TRY(need(y, "y"));
    return hip_status(kernels_conv_fwd(g, x, x_halo, weight, bias, y, (hipStream_t)stream),
                      "conv_fwd launch");
}

int sscnn_conv_bwd_input(const sscnn_conv_t* conv, const float* grad_y, const float* grad_y_halo,
                         const float* weight, float* grad_x, void* stream)
{
    Geom g;
    TRY(check(conv, &g));
    TRY(need(grad_y, "grad_y"));
    if (g.ghl + g.ghr) TRY(need(grad_y_halo, "grad_y_halo")); else TRY(optional(grad_y_halo, "grad_y_halo"));
    TRY(need(weight, "weight"));
    TRY(need(grad_x, "grad_x"));
    return hip_status(kernels_conv_bwd_input(g, grad_y, grad_y_halo, weight, grad_x,
                                             (hipStream_t)stream),
                      "conv_bwd_input launch");
}

size_t sscnn_conv_bwd_weight_workspace_bytes(const sscnn_conv_t* conv)
{
    Geom g;
    if (check(conv, &g)) return 0;
    return kernels_bwd_weight_workspace_bytes(g);
}

int sscnn_conv_bwd_weight_partial(const sscnn_conv_t* conv, const float* x, const float* x_halo,
                                  const float* grad_y, float* grad_w_part, float* grad_b_part,
                                  void* workspace, size_t workspace_bytes, void* stream)
{
    Geom g;
    TRY(check(conv, &g));
    TRY(need(x, "x"));
    if (g.hl + g.hr) TRY(need(x_halo, "x_halo")); else TRY(optional(x_halo, "x_halo"));
    TRY(need(grad_y, "grad_y"));
    TRY(need(grad_w_part, "grad_w_part"));
    TRY(optional(grad_b_part, "grad_b_part"));
    size_t ws_need;
    TRY(need_workspace(g, workspace, workspace_bytes, &ws_need));
    return hip_status(kernels_conv_bwd_weight(g, x, x_halo, grad_y, grad_w_part, grad_b_part,
                                              ws_need ? workspace : nullptr, (hipStream_t)stream),
                      "conv_bwd_weight_partial launch");
}

int sscnn_conv_bwd(const sscnn_conv_t* conv, const float* x, const float* x_halo, const float* grad_y,
                   const float* grad_y_halo, const float* weight, float* grad_x, float* grad_w_part,
                   float* grad_b_part, void* workspace, size_t workspace_bytes, void* stream)
{
    Geom g;
    TRY(check(conv, &g));
    TRY(need(x, "x"));
    if (g.hl + g.hr) TRY(need(x_halo, "x_halo")); else TRY(optional(x_halo, "x_halo"));
    TRY(need(grad_y, "grad_y"));
    if (g.ghl + g.ghr) TRY(need(grad_y_halo, "grad_y_halo")); else TRY(optional(grad_y_halo, "grad_y_halo"));
    TRY(need(weight, "weight"));
    TRY(need(grad_x, "grad_x"));
    TRY(need(grad_w_part, "grad_w_part"));
    TRY(optional(grad_b_part, "grad_b_part"));
    if (grad_x == x || grad_x == x_halo || grad_x == grad_y || grad_x == grad_y_halo)
        return fail(SSCNN_EINVAL, "grad_x aliases an input");
    size_t ws_need;
    TRY(need_workspace(g, workspace, workspace_bytes, &ws_need));
    return hip_status(kernels_conv_bwd(g, x, x_halo, grad_y, grad_y_halo, weight, grad_x, grad_w_part,
                                       grad_b_part, ws_need ? workspace : nullptr, (hipStream_t)stream),
                      "conv_bwd launch");
}

namespace {

// Validates a push descriptor for a producer whose pushed slice is `width`
// columns wide; fills *out and *active (false: nothing to push).
int check_push(const sscnn_conv_t* conv, const Geom& g, const sscnn_push_t* push, int width, const void* const* others,
               int nothers, Push* out, bool* active)
{
    *active = false;
    if (!push) return SSCNN_OK;
    if (push->hl < 0 || push->hr < 0 || push->hl > width || push->hr > width)
        return fail(SSCNN_EINVAL, "push widths hl=%d hr=%d must lie in [0, %d]", push->hl, push->hr, width);
    if (push->hl + push->hr == 0) return SSCNN_OK;
    const bool first = conv->shard == 0, last = conv->shard == conv->num_shards - 1;
    if (first != (push->to_left == nullptr))
        return fail(SSCNN_EINVAL, "push to_left must be NULL exactly for shard 0 (shard=%d)", conv->shard);
    if (last != (push->to_right == nullptr))
        return fail(SSCNN_EINVAL, "push to_right must be NULL exactly for the last shard (shard=%d)", conv->shard);
    if ((first && push->hl > 0) || (last && push->hr > 0)) TRY(need(push->own, "push own"));
    else TRY(optional(push->own, "push own"));
    TRY(optional(push->to_left, "push to_left"));
    TRY(optional(push->to_right, "push to_right"));
    const void* bufs[3] = {push->to_left, push->to_right, push->own};
    for (const void* b : bufs) {
        if (!b) continue;
        for (int k = 0; k < nothers; ++k)
            if (b == others[k]) return fail(SSCNN_EINVAL, "a push halo buffer aliases another argument");
    }
    out->to_left = push->to_left;
    out->to_right = push->to_right;
    out->own = push->own;
    out->hl = push->hl;
    out->hr = push->hr;
    *active = true;
    return SSCNN_OK;
}

}  // namespace

int sscnn_conv_fwd_push(const sscnn_conv_t* conv, const float* x, const float* x_halo, const float* weight,
                        const float* bias, float* y, const sscnn_push_t* push, void* stream)
{
    Geom g;
    TRY(check(conv, &g));
    TRY(need(x, "x"));
    if (g.hl + g.hr) TRY(need(x_halo, "x_halo")); else TRY(optional(x_halo, "x_halo"));
    TRY(need(weight, "weight"));
    TRY(optional(bias, "bias"));
    TRY(need(y, "y"));
    Push P;
    bool active;
    const void* others[5] = {x, x_halo, weight, bias, y};
    TRY(check_push(conv, g, push, g.wol, others, 5, &P, &active));
    const hipStream_t st = (hipStream_t)stream;
    if (active && patch_supported(g))     // pushed from the matrix kernel's epilogue
        return hip_status(launch_patch_fwd(g, x, weight, bias, y, st, nullptr, &P), "conv_fwd_push launch");
    hipError_t e = kernels_conv_fwd(g, x, x_halo, weight, bias, y, st);
    if (e == hipSuccess && active)
        e = launch_push_edges(y, (int64_t)g.n * g.co, g.ho, g.wol, P.hl, P.hr, P.to_left, P.to_right, P.own, st);
    return hip_status(e, "conv_fwd_push launch");
}

int sscnn_conv_bwd_push(const sscnn_conv_t* conv, const float* x, const float* x_halo, const float* grad_y,
                        const float* grad_y_halo, const float* weight, float* grad_x, float* grad_w_part,
                        float* grad_b_part, void* workspace, size_t workspace_bytes, const sscnn_push_t* push,
                        void* stream)
{
    Geom g;
    TRY(check(conv, &g));
    TRY(need(x, "x"));
    if (g.hl + g.hr) TRY(need(x_halo, "x_halo")); else TRY(optional(x_halo, "x_halo"));
    TRY(need(grad_y, "grad_y"));
    if (g.ghl + g.ghr) TRY(need(grad_y_halo, "grad_y_halo")); else TRY(optional(grad_y_halo, "grad_y_halo"));
    TRY(need(weight, "weight"));
    TRY(need(grad_x, "grad_x"));
    TRY(need(grad_w_part, "grad_w_part"));
    TRY(optional(grad_b_part, "grad_b_part"));
    if (grad_x == x || grad_x == x_halo || grad_x == grad_y || grad_x == grad_y_halo)
        return fail(SSCNN_EINVAL, "grad_x aliases an input");
    size_t ws_need;
    TRY(need_workspace(g, workspace, workspace_bytes, &ws_need));
    Push P;
    bool active;
    const void* others[9] = {x, x_halo, grad_y, grad_y_halo, weight, grad_x, grad_w_part, grad_b_part, workspace};
    TRY(check_push(conv, g, push, g.wl, others, 9, &P, &active));
    const hipStream_t st = (hipStream_t)stream;
    void* ws = ws_need ? workspace : nullptr;
    hipError_t e;
    if (active && patch_supported(g)) {   // pushed from the matrix kernel's epilogue
        e = launch_patch_bwd_input(g, grad_y, weight, grad_x, st, nullptr, &P);
        if (e == hipSuccess) e = kernels_conv_bwd_weight(g, x, x_halo, grad_y, grad_w_part, grad_b_part, ws, st);
        return hip_status(e, "conv_bwd_push launch");
    }
    e = kernels_conv_bwd(g, x, x_halo, grad_y, grad_y_halo, weight, grad_x, grad_w_part, grad_b_part, ws, st);
    if (e == hipSuccess && active)
        e = launch_push_edges(grad_x, (int64_t)g.n * g.ci, g.h, g.wl, P.hl, P.hr, P.to_left, P.to_right, P.own, st);
    return hip_status(e, "conv_bwd_push launch");
}

int sscnn_conv_bwd_noalloc(const sscnn_conv_t* conv, const float* x, const float* x_halo,
                           const float* grad_y, const float* grad_y_halo, const float* weight,
                           float* grad_x, float* grad_w_part, float* grad_b_part, void* stream)
{
    Geom g;
    TRY(check(conv, &g));
    TRY(need(x, "x"));
    if (g.hl + g.hr) TRY(need(x_halo, "x_halo")); else TRY(optional(x_halo, "x_halo"));
    TRY(need(grad_y, "grad_y"));
    if (g.ghl + g.ghr) TRY(need(grad_y_halo, "grad_y_halo")); else TRY(optional(grad_y_halo, "grad_y_halo"));
    TRY(need(weight, "weight"));
    TRY(need(grad_x, "grad_x"));
    TRY(need(grad_w_part, "grad_w_part"));
    TRY(optional(grad_b_part, "grad_b_part"));
    if (grad_x == x || grad_x == x_halo || grad_x == grad_y || grad_x == grad_y_halo)
        return fail(SSCNN_EINVAL, "grad_x aliases an input");
    const size_t ws_need = kernels_bwd_weight_workspace_bytes(g);
    if (ws_need > kNoAllocScratchBytes)
        return fail(SSCNN_EWORKSPACE, "conv_bwd_noalloc: this layer needs %zu bytes of scratch, more than the "
                    "library's %zu; use sscnn_conv_bwd with a workspace", ws_need, kNoAllocScratchBytes);
    int dev = -1, sdev = -1;
    TRY(hip_status(hipGetDevice(&dev), "conv_bwd_noalloc: hipGetDevice"));
    TRY(hip_status(hipStreamGetDevice((hipStream_t)stream, &sdev), "conv_bwd_noalloc: hipStreamGetDevice"));
    if (sdev != dev)
        return fail(SSCNN_EINVAL, "conv_bwd_noalloc: stream belongs to device %d, current device is %d", sdev, dev);
    void* scratch = nullptr;
    TRY(hip_status(noalloc_scratch(&scratch), "conv_bwd_noalloc: scratch address"));
    return hip_status(kernels_conv_bwd(g, x, x_halo, grad_y, grad_y_halo, weight, grad_x, grad_w_part,
                                       grad_b_part, ws_need ? scratch : nullptr, (hipStream_t)stream),
                      "conv_bwd_noalloc launch");
}

int sscnn_stream_copy(const float* src, float* dst, int64_t count, void* stream)
{
    if (count < 0) return fail(SSCNN_EINVAL, "count=%lld is negative", (long long)count);
    if (count == 0) return SSCNN_OK;
    TRY(need(src, "src"));
    TRY(need(dst, "dst"));
    const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
    const uintptr_t bytes = (uintptr_t)count * sizeof(float);
    if (a < b + bytes && b < a + bytes) return fail(SSCNN_EINVAL, "src and dst overlap");
    return hip_status(launch_stream_copy(src, dst, count, (hipStream_t)stream), "stream_copy launch");
}

int sscnn_partial_reduce(const float* const* parts, int32_t nparts, int64_t count, float* out,
                         void* stream)
{
    if (!parts) return fail(SSCNN_EINVAL, "parts is NULL");
    if (nparts < 1 || nparts > kMaxParts)
        return fail(SSCNN_EINVAL, "nparts=%d outside [1, %d]", nparts, kMaxParts);
    if (count < 0) return fail(SSCNN_EINVAL, "count=%lld is negative", (long long)count);
    if (!out) return fail(SSCNN_EINVAL, "out is NULL");
    for (int s = 0; s < nparts; ++s) {
        if (!parts[s]) return fail(SSCNN_EINVAL, "parts[%d] is NULL", s);
        if (parts[s] == out) return fail(SSCNN_EINVAL, "out aliases parts[%d]", s);
    }
    return hip_status(launch_partial_reduce(parts, nparts, count, out, (hipStream_t)stream),
                      "partial_reduce launch");
}

// --- the ConvNeXt block's other steps ------------------------------------------

}  // extern "C"

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 38;

int check_dims(int32_t n, int32_t c, int32_t h, int32_t w, bool quads)
{
    if (n < 1 || c < 1 || h < 1 || w < 1)
        return fail(SSCNN_EINVAL, "dims n=%d c=%d h=%d w=%d must all be >= 1", n, c, h, w);
    if ((int64_t)n * c * h * w >= kMaxElems) return fail(SSCNN_EINVAL, "tensor of n*c*h*w elements is too large");
    if (quads && ((int64_t)h * w) % 4) return fail(SSCNN_EINVAL, "h*w=%lld is not a multiple of 4", (long long)h * w);
    return SSCNN_OK;
}

}  // namespace

extern "C" {

int sscnn_layernorm_fwd(int32_t n, int32_t c, int32_t h, int32_t w, float eps, const float* x, const float* gamma,
                        const float* beta, float* y, float* mean, float* rstd, void* stream)
{
    TRY(check_dims(n, c, h, w, false));
    if (!(eps > 0.f) || !std::isfinite(eps)) return fail(SSCNN_EINVAL, "eps must be positive and finite");
    TRY(need(x, "x"));
    TRY(need(gamma, "gamma"));
    TRY(need(beta, "beta"));
    TRY(need(y, "y"));
    TRY(need(mean, "mean"));
    TRY(need(rstd, "rstd"));
    if (mean == rstd || (const float*)mean == x || (const float*)rstd == x || mean == y || rstd == y)
        return fail(SSCNN_EINVAL, "mean / rstd alias each other or a tensor");
    return hip_status(launch_layernorm_fwd(n, c, (int64_t)h * w, eps, x, gamma, beta, y, mean, rstd,
                                           (hipStream_t)stream),
                      "layernorm_fwd launch");
}

int sscnn_layernorm_bwd(int32_t n, int32_t c, int32_t h, int32_t w, const float* x, const float* dy,
                        const float* gamma, const float* mean, const float* rstd, float* dx, float* dgamma,
                        float* dbeta, void* stream)
{
    TRY(check_dims(n, c, h, w, false));
    TRY(need(x, "x"));
    TRY(need(dy, "dy"));
    TRY(need(gamma, "gamma"));
    TRY(need(mean, "mean"));
    TRY(need(rstd, "rstd"));
    TRY(optional(dx, "dx"));
    TRY(optional(dgamma, "dgamma"));
    TRY(optional(dbeta, "dbeta"));
    if (dx && ((const float*)dx == x || (const float*)dx == dy))
        return fail(SSCNN_EINVAL, "dx aliases x or dy");
    if (dgamma && dgamma == dbeta) return fail(SSCNN_EINVAL, "dgamma aliases dbeta");
    return hip_status(launch_layernorm_bwd(n, c, (int64_t)h * w, x, dy, gamma, mean, rstd, dx, dgamma, dbeta,
                                           (hipStream_t)stream),
                      "layernorm_bwd launch");
}

int sscnn_gelu_fwd(int64_t count, const float* x, float* y, void* stream)
{
    if (count < 0 || count >= kMaxElems) return fail(SSCNN_EINVAL, "count=%lld out of range", (long long)count);
    if (count == 0) return SSCNN_OK;
    TRY(need(x, "x"));
    TRY(need(y, "y"));
    return hip_status(launch_gelu_fwd(count, x, y, (hipStream_t)stream), "gelu_fwd launch");
}

int sscnn_gelu_bwd(int64_t count, const float* x, const float* dy, float* dx, void* stream)
{
    if (count < 0 || count >= kMaxElems) return fail(SSCNN_EINVAL, "count=%lld out of range", (long long)count);
    if (count == 0) return SSCNN_OK;
    TRY(need(x, "x"));
    TRY(need(dy, "dy"));
    TRY(need(dx, "dx"));
    return hip_status(launch_gelu_bwd(count, x, dy, dx, (hipStream_t)stream), "gelu_bwd launch");
}

// The fused pointwise calls run the matrix-core kernel of 1x1 layers with its
// GELU epilogue; any other layer is refused rather than run in two passes.
static int check_pointwise(const sscnn_conv_t* conv, Geom* g)
{
    TRY(check(conv, g));
    if (g->k != 1 || g->stride != 1 || g->pad != 0 || g->groups != 1 || !patch_supported(*g))
        return fail(SSCNN_EUNSUPPORTED, "fused GELU needs a pointwise layer on the matrix-core path "
                    "(k=%d stride=%d pad=%d groups=%d)", g->k, g->stride, g->pad, g->groups);
    return SSCNN_OK;
}

int sscnn_pointwise_gelu_fwd(const sscnn_conv_t* conv, const float* x, const float* weight, const float* bias,
                             float* y, float* y_act, void* stream)
{
    Geom g;
    TRY(check_pointwise(conv, &g));
    TRY(need(x, "x"));
    TRY(need(weight, "weight"));
    TRY(optional(bias, "bias"));
    TRY(need(y, "y"));
    TRY(need(y_act, "y_act"));
    if (y_act == y || y == x || y_act == x) return fail(SSCNN_EINVAL, "y or y_act aliases another argument");
    return hip_status(launch_patch_fwd(g, x, weight, bias, y, (hipStream_t)stream, y_act),
                      "pointwise_gelu_fwd launch");
}

int sscnn_pointwise_bwd_input_gelu(const sscnn_conv_t* conv, const float* grad_y, const float* weight,
                                   const float* pre, float* grad_x, void* stream)
{
    Geom g;
    TRY(check_pointwise(conv, &g));
    TRY(need(grad_y, "grad_y"));
    TRY(need(weight, "weight"));
    TRY(need(pre, "pre"));
    TRY(need(grad_x, "grad_x"));
    if (grad_x == grad_y || grad_x == pre || grad_x == weight) return fail(SSCNN_EINVAL, "grad_x aliases an input");
    return hip_status(launch_patch_bwd_input(g, grad_y, weight, grad_x, (hipStream_t)stream, pre),
                      "pointwise_bwd_input_gelu launch");
}

int sscnn_droppath_scales(uint64_t seed, uint64_t offset, int32_t n, double keep_prob, float* scales, void* stream)
{
    if (n < 0) return fail(SSCNN_EINVAL, "n=%d is negative", n);
    if (!(keep_prob > 0.0) || !std::isfinite(keep_prob))
        return fail(SSCNN_EINVAL, "keep_prob must be positive and finite");
    if (n == 0) return SSCNN_OK;
    TRY(need(scales, "scales"));
    const bool draw = keep_prob < 1.0;
    const double t = std::floor(keep_prob * 4294967296.0);
    const uint32_t thr = t >= 4294967295.0 ? 0xFFFFFFFFu : (uint32_t)t;
    const float inv = (float)(1.0 / keep_prob);
    return hip_status(launch_droppath_scales(n, seed, offset, thr, inv, draw, scales, (hipStream_t)stream),
                      "droppath_scales launch");
}

int sscnn_layer_scale_residual_fwd(int32_t n, int32_t c, int32_t h, int32_t w, const float* x, const float* hb,
                                   const float* gamma, const float* scales, float* out, void* stream)
{
    TRY(check_dims(n, c, h, w, true));
    TRY(need(x, "x"));
    TRY(need(hb, "hb"));
    TRY(need(gamma, "gamma"));
    TRY(optional(scales, "scales"));
    TRY(need(out, "out"));
    return hip_status(launch_scale_residual_fwd(n, c, (int64_t)h * w, x, hb, gamma, scales, out, (hipStream_t)stream),
                      "layer_scale_residual_fwd launch");
}

int sscnn_layer_scale_residual_bwd(int32_t n, int32_t c, int32_t h, int32_t w, const float* hb, const float* dout,
                                   const float* gamma, const float* scales, float* dh, float* dgamma, void* stream)
{
    TRY(check_dims(n, c, h, w, true));
    TRY(need(hb, "hb"));
    TRY(need(dout, "dout"));
    TRY(need(gamma, "gamma"));
    TRY(optional(scales, "scales"));
    TRY(optional(dh, "dh"));
    TRY(optional(dgamma, "dgamma"));
    if (dh && dgamma && ((const float*)dh == hb || (const float*)dh == dout))
        return fail(SSCNN_EINVAL, "dh aliases hb or dout while dgamma is requested");
    return hip_status(launch_scale_residual_bwd(n, c, (int64_t)h * w, hb, dout, gamma, scales, dh, dgamma,
                                                (hipStream_t)stream),
                      "layer_scale_residual_bwd launch");
}

// --- split convolution: interior calls (halo read as zeros) and edge calls ---

int sscnn_conv_fwd_interior(const sscnn_conv_t* conv, const float* x, const float* weight,
                            const float* bias, float* y, void* stream)
{
    Geom g;
    TRY(check(conv, &g));
    TRY(need(x, "x"));
    TRY(need(weight, "weight"));
    TRY(optional(bias, "bias"));
    TRY(need(y, "y"));
    return hip_status(kernels_conv_fwd(g, x, nullptr, weight, bias, y, (hipStream_t)stream),
                      "conv_fwd_interior launch");
}

int sscnn_conv_fwd_edge(const sscnn_conv_t* conv, const float* x_halo, const float* weight, float* y,
                        void* stream)
{
    Geom g;
    TRY(check(conv, &g));
    if (g.hl + g.hr == 0) {
        TRY(optional(x_halo, "x_halo"));
        return SSCNN_OK;
    }
    TRY(need(x_halo, "x_halo"));
    TRY(need(weight, "weight"));
    TRY(need(y, "y"));
    if (y == x_halo) return fail(SSCNN_EINVAL, "y aliases x_halo");
    return hip_status(launch_edge_fwd(g, x_halo, weight, y, (hipStream_t)stream), "conv_fwd_edge launch");
}

int sscnn_conv_bwd_input_interior(const sscnn_conv_t* conv, const float* grad_y, const float* weight,
                                  float* grad_x, void* stream)
{
    Geom g;
    TRY(check(conv, &g));
    TRY(need(grad_y, "grad_y"));
    TRY(need(weight, "weight"));
    TRY(need(grad_x, "grad_x"));
    return hip_status(kernels_conv_bwd_input(g, grad_y, nullptr, weight, grad_x, (hipStream_t)stream),
                      "conv_bwd_input_interior launch");
}

int sscnn_conv_bwd_input_edge(const sscnn_conv_t* conv, const float* grad_y_halo, const float* weight,
                              float* grad_x, void* stream)
{
    Geom g;
    TRY(check(conv, &g));
    if (g.ghl + g.ghr == 0) {
        TRY(optional(grad_y_halo, "grad_y_halo"));
        return SSCNN_OK;
    }
    TRY(need(grad_y_halo, "grad_y_halo"));
    TRY(need(weight, "weight"));
    TRY(need(grad_x, "grad_x"));
    if (grad_x == grad_y_halo) return fail(SSCNN_EINVAL, "grad_x aliases grad_y_halo");
    return hip_status(launch_edge_bwd_input(g, grad_y_halo, weight, grad_x, (hipStream_t)stream),
                      "conv_bwd_input_edge launch");
}

int sscnn_conv_bwd_weight_partial_interior(const sscnn_conv_t* conv, const float* x, const float* grad_y,
                                           float* grad_w_part, float* grad_b_part, void* workspace,
                                           size_t workspace_bytes, void* stream)
{
    Geom g;
    TRY(check(conv, &g));
    TRY(need(x, "x"));
    TRY(need(grad_y, "grad_y"));
    TRY(need(grad_w_part, "grad_w_part"));
    TRY(optional(grad_b_part, "grad_b_part"));
    size_t ws_need;
    TRY(need_workspace(g, workspace, workspace_bytes, &ws_need));
    return hip_status(kernels_conv_bwd_weight(g, x, nullptr, grad_y, grad_w_part, grad_b_part,
                                              ws_need ? workspace : nullptr, (hipStream_t)stream),
                      "conv_bwd_weight_partial_interior launch");
}

int sscnn_conv_bwd_weight_edge(const sscnn_conv_t* conv, const float* x_halo, const float* grad_y,
                               float* grad_w_part, void* stream)
{
    Geom g;
    TRY(check(conv, &g));
    if (g.hl + g.hr == 0) {
        TRY(optional(x_halo, "x_halo"));
        return SSCNN_OK;
    }
    TRY(need(x_halo, "x_halo"));
    TRY(need(grad_y, "grad_y"));
    TRY(need(grad_w_part, "grad_w_part"));
    if (grad_w_part == x_halo || grad_w_part == grad_y)
        return fail(SSCNN_EINVAL, "grad_w_part aliases an input");
    return hip_status(launch_edge_bwd_weight(g, x_halo, grad_y, grad_w_part, (hipStream_t)stream),
                      "conv_bwd_weight_edge launch");
}

int sscnn_conv_bwd_interior(const sscnn_conv_t* conv, const float* x, const float* grad_y,
                            const float* weight, float* grad_x, float* grad_w_part, float* grad_b_part,
                            void* workspace, size_t workspace_bytes, void* stream)
{
    Geom g;
    TRY(check(conv, &g));
    TRY(need(x, "x"));
    TRY(need(grad_y, "grad_y"));
    TRY(need(weight, "weight"));
    TRY(need(grad_x, "grad_x"));
    TRY(need(grad_w_part, "grad_w_part"));
    TRY(optional(grad_b_part, "grad_b_part"));
    if (grad_x == x || grad_x == grad_y) return fail(SSCNN_EINVAL, "grad_x aliases an input");
    size_t ws_need;
    TRY(need_workspace(g, workspace, workspace_bytes, &ws_need));
    return hip_status(kernels_conv_bwd(g, x, nullptr, grad_y, nullptr, weight, grad_x, grad_w_part,
                                       grad_b_part, ws_need ? workspace : nullptr, (hipStream_t)stream),
                      "conv_bwd_interior launch");
}

// --- height sharding -----------------------------------------------------

namespace {

// The row halo buffer (planes, up + down, width) of a height or 2-D shard as
// the rows above and below each plane of the slice, for the matrix-core
// kernels; crh = rows of the column halo above row 0 (2-D shards).
RowHalo row_halo(const float* rh, int up, int down, int width, int crh)
{
    RowHalo r;
    r.up = rh;
    r.down = rh ? rh + (int64_t)up * width : nullptr;
    r.rplane = (int64_t)(up + down) * width;
    r.rh = up;
    r.crh = crh;
    return r;
}

// Dense stride-1 layers whose row halo is as tall above as below take the
// matrix-core kernels reading the row halo directly.
bool mfma_rows(const Geom& g, int up, int down) { return mfma_conv_supported(g) && up == down; }

}  // namespace

int sscnn_hconv_init(sscnn_hconv_t* conv)
{
    if (!conv) return fail(SSCNN_EINVAL, "conv is NULL");
    sscnn_hconv_t d;
    TRY(derive_h(*conv, &d));
    *conv = d;
    return SSCNN_OK;
}

int sscnn_row_halo_gather(const sscnn_hconv_t* conv, int32_t which, const float* up_nbr, const float* down_nbr,
                          float* halo, void* stream)
{
    Geom g;
    TRY(check_h(conv, &g));
    int64_t planes;
    int rows, width, hu, hd;
    if (which == SSCNN_HALO_INPUT) {
        planes = (int64_t)g.n * g.ci; rows = g.h; width = g.wl; hu = conv->halo_u; hd = conv->halo_d;
    } else if (which == SSCNN_HALO_GRAD_OUTPUT) {
        planes = (int64_t)g.n * g.co; rows = g.ho; width = g.wol; hu = conv->ghalo_u; hd = conv->ghalo_d;
    } else {
        return fail(SSCNN_EINVAL, "which=%d is neither SSCNN_HALO_INPUT nor SSCNN_HALO_GRAD_OUTPUT", which);
    }
    const bool first = conv->shard == 0, last = conv->shard == conv->num_shards - 1;
    if (first != (up_nbr == nullptr))
        return fail(SSCNN_EINVAL, "up_nbr must be NULL exactly for shard 0 (shard=%d)", conv->shard);
    if (last != (down_nbr == nullptr))
        return fail(SSCNN_EINVAL, "down_nbr must be NULL exactly for the last shard (shard=%d)", conv->shard);
    TRY(optional(up_nbr, "up_nbr"));
    TRY(optional(down_nbr, "down_nbr"));
    if (hu + hd == 0) return SSCNN_OK;
    TRY(need(halo, "halo"));
    return hip_status(launch_row_halo_gather(hu ? up_nbr : nullptr, hd ? down_nbr : nullptr, planes, rows, width,
                                             hu, hd, halo, (hipStream_t)stream),
                      "row_halo_gather launch");
}

int sscnn_hconv_fwd(const sscnn_hconv_t* conv, const float* x, const float* x_halo, const float* weight,
                    const float* bias, float* y, void* stream)
{
    Geom g;
    TRY(check_h(conv, &g));
    TRY(need(x, "x"));
    const int hu = conv->halo_u, hd = conv->halo_d;
    if (hu + hd) TRY(need(x_halo, "x_halo")); else TRY(optional(x_halo, "x_halo"));
    TRY(need(weight, "weight"));
    TRY(optional(bias, "bias"));
    TRY(need(y, "y"));
    const hipStream_t st = (hipStream_t)stream;
    if (dw_supported(g))   // depthwise: the tiles read the row halo themselves
        return hip_status(launch_dw_fwd_rows(g, x, x_halo, hu, hd, weight, bias, y, st), "hconv_fwd launch");
    if (mfma_rows(g, hu, hd))
        return hip_status(launch_mfma_fwd_rows(g, x, nullptr, row_halo(x_halo, hu, hd, g.wl, 0), weight, bias, y, st),
                          "hconv_fwd launch");
    hipError_t e = kernels_conv_fwd(g, x, nullptr, weight, bias, y, st);
    if (e == hipSuccess) e = launch_row_edge_fwd(g, hu, hd, x_halo, weight, y, st);
    return hip_status(e, "hconv_fwd launch");
}

int sscnn_hconv_bwd_input(const sscnn_hconv_t* conv, const float* grad_y, const float* grad_y_halo,
                          const float* weight, float* grad_x, void* stream)
{
    Geom g;
    TRY(check_h(conv, &g));
    TRY(need(grad_y, "grad_y"));
    const int ghu = conv->ghalo_u, ghd = conv->ghalo_d;
    if (ghu + ghd) TRY(need(grad_y_halo, "grad_y_halo")); else TRY(optional(grad_y_halo, "grad_y_halo"));
    TRY(need(weight, "weight"));
    TRY(need(grad_x, "grad_x"));
    const hipStream_t st = (hipStream_t)stream;
    if (dw_supported(g))
        return hip_status(launch_dw_bwd_input_rows(g, grad_y, grad_y_halo, ghu, ghd, weight, grad_x, st),
                          "hconv_bwd_input launch");
    if (mfma_rows(g, ghu, ghd))
        return hip_status(launch_mfma_bwd_input_rows(g, grad_y, nullptr, row_halo(grad_y_halo, ghu, ghd, g.wol, 0),
                                                     weight, grad_x, st),
                          "hconv_bwd_input launch");
    hipError_t e = kernels_conv_bwd_input(g, grad_y, nullptr, weight, grad_x, st);
    if (e == hipSuccess) e = launch_row_edge_bwd_input(g, ghu, ghd, grad_y_halo, weight, grad_x, st);
    return hip_status(e, "hconv_bwd_input launch");
}

size_t sscnn_hconv_bwd_weight_workspace_bytes(const sscnn_hconv_t* conv)
{
    Geom g;
    if (check_h(conv, &g)) return 0;
    const size_t a = kernels_bwd_weight_workspace_bytes(g), b = row_edge_workspace_bytes(g);
    return a > b ? a : b;
}

int sscnn_hconv_bwd_weight_partial(const sscnn_hconv_t* conv, const float* x, const float* x_halo,
                                   const float* grad_y, float* grad_w_part, float* grad_b_part, void* workspace,
                                   size_t workspace_bytes, void* stream)
{
    Geom g;
    TRY(check_h(conv, &g));
    TRY(need(x, "x"));
    const int hu = conv->halo_u, hd = conv->halo_d;
    if (hu + hd) TRY(need(x_halo, "x_halo")); else TRY(optional(x_halo, "x_halo"));
    TRY(need(grad_y, "grad_y"));
    TRY(need(grad_w_part, "grad_w_part"));
    TRY(optional(grad_b_part, "grad_b_part"));
    size_t ws_need;
    TRY(need_workspace(g, workspace, workspace_bytes, &ws_need, true));
    const hipStream_t st = (hipStream_t)stream;
    if (dw_supported(g))
        return hip_status(launch_dw_bwd_weight_rows(g, x, x_halo, hu, hd, grad_y, grad_w_part, grad_b_part,
                                                    workspace, st),
                          "hconv_bwd_weight_partial launch");
    if (mfma_rows(g, hu, hd))
        return hip_status(launch_mfma_bwd_weight_rows(g, x, nullptr, row_halo(x_halo, hu, hd, g.wl, 0), grad_y,
                                                      grad_w_part, grad_b_part, ws_need ? workspace : nullptr, st),
                          "hconv_bwd_weight_partial launch");
    hipError_t e = kernels_conv_bwd_weight(g, x, nullptr, grad_y, grad_w_part, grad_b_part,
                                           ws_need ? workspace : nullptr, st);
    if (e == hipSuccess) e = launch_row_edge_bwd_weight(g, hu, hd, x_halo, grad_y, grad_w_part, workspace, st);
    return hip_status(e, "hconv_bwd_weight_partial launch");
}

int sscnn_hconv_bwd(const sscnn_hconv_t* conv, const float* x, const float* x_halo, const float* grad_y,
                    const float* grad_y_halo, const float* weight, float* grad_x, float* grad_w_part,
                    float* grad_b_part, void* workspace, size_t workspace_bytes, void* stream)
{
    Geom g;
    TRY(check_h(conv, &g));
    TRY(need(x, "x"));
    const int hu = conv->halo_u, hd = conv->halo_d, ghu = conv->ghalo_u, ghd = conv->ghalo_d;
    if (hu + hd) TRY(need(x_halo, "x_halo")); else TRY(optional(x_halo, "x_halo"));
    TRY(need(grad_y, "grad_y"));
    if (ghu + ghd) TRY(need(grad_y_halo, "grad_y_halo")); else TRY(optional(grad_y_halo, "grad_y_halo"));
    TRY(need(weight, "weight"));
    TRY(need(grad_x, "grad_x"));
    TRY(need(grad_w_part, "grad_w_part"));
    TRY(optional(grad_b_part, "grad_b_part"));
    if (grad_x == x || grad_x == x_halo || grad_x == grad_y || grad_x == grad_y_halo)
        return fail(SSCNN_EINVAL, "grad_x aliases an input");
    size_t ws_need;
    TRY(need_workspace(g, workspace, workspace_bytes, &ws_need, true));
    const hipStream_t st = (hipStream_t)stream;
    if (dw_supported(g))
        return hip_status(launch_dw_bwd_rows(g, x, x_halo, hu, hd, grad_y, grad_y_halo, ghu, ghd, weight, grad_x,
                                             grad_w_part, grad_b_part, workspace, st),
                          "hconv_bwd launch");
    if (mfma_rows(g, hu, hd) && ghu == ghd) {
        hipError_t e = launch_mfma_bwd_input_rows(g, grad_y, nullptr, row_halo(grad_y_halo, ghu, ghd, g.wol, 0),
                                                  weight, grad_x, st);
        if (e == hipSuccess)
            e = launch_mfma_bwd_weight_rows(g, x, nullptr, row_halo(x_halo, hu, hd, g.wl, 0), grad_y, grad_w_part,
                                            grad_b_part, ws_need ? workspace : nullptr, st);
        return hip_status(e, "hconv_bwd launch");
    }
    hipError_t e = kernels_conv_bwd(g, x, nullptr, grad_y, nullptr, weight, grad_x, grad_w_part, grad_b_part,
                                    ws_need ? workspace : nullptr, st);
    if (e == hipSuccess) e = launch_row_edge_bwd_input(g, ghu, ghd, grad_y_halo, weight, grad_x, st);
    if (e == hipSuccess) e = launch_row_edge_bwd_weight(g, hu, hd, x_halo, grad_y, grad_w_part, workspace, st);
    return hip_status(e, "hconv_bwd launch");
}

// --- 2-D H x W shards ------------------------------------------------------------

int sscnn_gconv_init(sscnn_gconv_t* conv)
{
    if (!conv) return fail(SSCNN_EINVAL, "conv is NULL");
    sscnn_gconv_t d;
    TRY(derive_g(*conv, &d));
    *conv = d;
    return SSCNN_OK;
}

int sscnn_grid_row_halo_gather(const sscnn_gconv_t* conv, int32_t which, const float* up, const float* down,
                               float* row_halo, void* stream)
{
    Geom g;
    TRY(check_g(conv, &g));
    if (which != SSCNN_HALO_INPUT && which != SSCNN_HALO_GRAD_OUTPUT) return fail(SSCNN_EINVAL, "bad which=%d", which);
    const int hh = conv->halo;
    if (hh == 0) return SSCNN_OK;
    TRY(need(row_halo, "row_halo"));
    if ((conv->shard_h > 0) != (up != nullptr)) return fail(SSCNN_EINVAL, "up must be given exactly when shard_h > 0");
    if ((conv->shard_h < conv->num_h - 1) != (down != nullptr))
        return fail(SSCNN_EINVAL, "down must be given exactly when shard_h < num_h - 1");
    TRY(optional(up, "up"));
    TRY(optional(down, "down"));
    const bool in = which == SSCNN_HALO_INPUT;
    const int64_t planes = (int64_t)g.n * (in ? g.ci : g.co);
    return hip_status(launch_row_halo_gather(up, down, planes, in ? g.h : g.ho, in ? g.wl : g.wol, hh, hh, row_halo,
                                             (hipStream_t)stream),
                      "grid_row_halo_gather launch");
}

int sscnn_grid_col_halo_gather(const sscnn_gconv_t* conv, int32_t which, const float* left, const float* left_row_halo,
                               const float* right, const float* right_row_halo, float* col_halo, void* stream)
{
    Geom g;
    TRY(check_g(conv, &g));
    if (which != SSCNN_HALO_INPUT && which != SSCNN_HALO_GRAD_OUTPUT) return fail(SSCNN_EINVAL, "bad which=%d", which);
    const int hh = conv->halo;
    if (hh == 0) return SSCNN_OK;
    TRY(need(col_halo, "col_halo"));
    if ((conv->shard_w > 0) != (left != nullptr)) return fail(SSCNN_EINVAL, "left must be given exactly when shard_w > 0");
    if ((conv->shard_w < conv->num_w - 1) != (right != nullptr))
        return fail(SSCNN_EINVAL, "right must be given exactly when shard_w < num_w - 1");
    if ((left && !left_row_halo) || (right && !right_row_halo))
        return fail(SSCNN_EINVAL, "a neighbour block needs its phase-1 row halo");
    TRY(optional(left, "left"));
    TRY(optional(right, "right"));
    TRY(optional(left_row_halo, "left_row_halo"));
    TRY(optional(right_row_halo, "right_row_halo"));
    const bool in = which == SSCNN_HALO_INPUT;
    const int64_t planes = (int64_t)g.n * (in ? g.ci : g.co);
    return hip_status(launch_grid_col_halo(left, left_row_halo, right, right_row_halo, planes, in ? g.h : g.ho,
                                           in ? g.wl : g.wol, hh, hh, hh, hh, col_halo, (hipStream_t)stream),
                      "grid_col_halo_gather launch");
}

namespace {

// the row / column halos a call needs (none for k = stride layers)
int need_grid_halos(const sscnn_gconv_t* conv, const float* rh, const float* ch, const char* rn, const char* cn)
{
    if (conv->halo) {
        TRY(need(rh, rn));
        TRY(need(ch, cn));
    } else {
        TRY(optional(rh, rn));
        TRY(optional(ch, cn));
    }
    return SSCNN_OK;
}

}  // namespace

int sscnn_gconv_fwd(const sscnn_gconv_t* conv, const float* x, const float* x_row_halo, const float* x_col_halo,
                    const float* weight, const float* bias, float* y, void* stream)
{
    Geom g;
    TRY(check_g(conv, &g));
    TRY(need(x, "x"));
    TRY(need_grid_halos(conv, x_row_halo, x_col_halo, "x_row_halo", "x_col_halo"));
    TRY(need(weight, "weight"));
    TRY(optional(bias, "bias"));
    TRY(need(y, "y"));
    const hipStream_t st = (hipStream_t)stream;
    const int hh = conv->halo;
    if (!hh) return hip_status(kernels_conv_fwd(g, x, nullptr, weight, bias, y, st), "gconv_fwd launch");
    if (mfma_conv_supported(g))
        return hip_status(launch_mfma_fwd_rows(g, x, x_col_halo, row_halo(x_row_halo, hh, hh, g.wl, hh), weight, bias,
                                               y, st),
                          "gconv_fwd launch");
    return hip_status(launch_dw_fwd_grid(g, x, x_row_halo, x_col_halo, hh, hh, weight, bias, y, st), "gconv_fwd launch");
}

int sscnn_gconv_bwd_input(const sscnn_gconv_t* conv, const float* grad_y, const float* gy_row_halo,
                          const float* gy_col_halo, const float* weight, float* grad_x, void* stream)
{
    Geom g;
    TRY(check_g(conv, &g));
    TRY(need(grad_y, "grad_y"));
    TRY(need_grid_halos(conv, gy_row_halo, gy_col_halo, "gy_row_halo", "gy_col_halo"));
    TRY(need(weight, "weight"));
    TRY(need(grad_x, "grad_x"));
    const hipStream_t st = (hipStream_t)stream;
    const int hh = conv->halo;
    if (!hh) return hip_status(kernels_conv_bwd_input(g, grad_y, nullptr, weight, grad_x, st), "gconv_bwd_input launch");
    if (mfma_conv_supported(g))
        return hip_status(launch_mfma_bwd_input_rows(g, grad_y, gy_col_halo, row_halo(gy_row_halo, hh, hh, g.wol, hh),
                                                     weight, grad_x, st),
                          "gconv_bwd_input launch");
    return hip_status(launch_dw_bwd_input_grid(g, grad_y, gy_row_halo, gy_col_halo, hh, hh, weight, grad_x, st),
                      "gconv_bwd_input launch");
}

size_t sscnn_gconv_bwd_weight_workspace_bytes(const sscnn_gconv_t* conv)
{
    Geom g;
    if (check_g(conv, &g)) return 0;
    return kernels_bwd_weight_workspace_bytes(g);
}

int sscnn_gconv_bwd_weight_partial(const sscnn_gconv_t* conv, const float* x, const float* x_row_halo,
                                   const float* x_col_halo, const float* grad_y, float* grad_w_part, float* grad_b_part,
                                   void* workspace, size_t workspace_bytes, void* stream)
{
    Geom g;
    TRY(check_g(conv, &g));
    TRY(need(x, "x"));
    TRY(need_grid_halos(conv, x_row_halo, x_col_halo, "x_row_halo", "x_col_halo"));
    TRY(need(grad_y, "grad_y"));
    TRY(need(grad_w_part, "grad_w_part"));
    TRY(optional(grad_b_part, "grad_b_part"));
    size_t ws_need;
    TRY(need_workspace(g, workspace, workspace_bytes, &ws_need));
    const hipStream_t st = (hipStream_t)stream;
    const int hh = conv->halo;
    void* ws = ws_need ? workspace : nullptr;
    if (!hh)
        return hip_status(kernels_conv_bwd_weight(g, x, nullptr, grad_y, grad_w_part, grad_b_part, ws, st),
                          "gconv_bwd_weight_partial launch");
    if (mfma_conv_supported(g))
        return hip_status(launch_mfma_bwd_weight_rows(g, x, x_col_halo, row_halo(x_row_halo, hh, hh, g.wl, hh), grad_y,
                                                      grad_w_part, grad_b_part, ws, st),
                          "gconv_bwd_weight_partial launch");
    return hip_status(launch_dw_bwd_weight_grid(g, x, x_row_halo, x_col_halo, hh, hh, grad_y, grad_w_part,
                                                grad_b_part, ws, st),
                      "gconv_bwd_weight_partial launch");
}

int sscnn_gconv_bwd(const sscnn_gconv_t* conv, const float* x, const float* x_row_halo, const float* x_col_halo,
                    const float* grad_y, const float* gy_row_halo, const float* gy_col_halo, const float* weight,
                    float* grad_x, float* grad_w_part, float* grad_b_part, void* workspace, size_t workspace_bytes,
                    void* stream)
{
    Geom g;
    TRY(check_g(conv, &g));
    TRY(need(x, "x"));
    TRY(need_grid_halos(conv, x_row_halo, x_col_halo, "x_row_halo", "x_col_halo"));
    TRY(need(grad_y, "grad_y"));
    TRY(need_grid_halos(conv, gy_row_halo, gy_col_halo, "gy_row_halo", "gy_col_halo"));
    TRY(need(weight, "weight"));
    TRY(need(grad_x, "grad_x"));
    TRY(need(grad_w_part, "grad_w_part"));
    TRY(optional(grad_b_part, "grad_b_part"));
    if (grad_x == x || grad_x == grad_y) return fail(SSCNN_EINVAL, "grad_x aliases an input");
    size_t ws_need;
    TRY(need_workspace(g, workspace, workspace_bytes, &ws_need));
    const hipStream_t st = (hipStream_t)stream;
    const int hh = conv->halo;
    void* ws = ws_need ? workspace : nullptr;
    if (!hh)
        return hip_status(kernels_conv_bwd(g, x, nullptr, grad_y, nullptr, weight, grad_x, grad_w_part, grad_b_part,
                                           ws, st),
                          "gconv_bwd launch");
    if (mfma_conv_supported(g)) {
        hipError_t e = launch_mfma_bwd_input_rows(g, grad_y, gy_col_halo, row_halo(gy_row_halo, hh, hh, g.wol, hh),
                                                  weight, grad_x, st);
        if (e == hipSuccess)
            e = launch_mfma_bwd_weight_rows(g, x, x_col_halo, row_halo(x_row_halo, hh, hh, g.wl, hh), grad_y,
                                            grad_w_part, grad_b_part, ws, st);
        return hip_status(e, "gconv_bwd launch");
    }
    return hip_status(launch_dw_bwd_grid(g, x, x_row_halo, x_col_halo, hh, hh, grad_y, gy_row_halo, gy_col_halo, hh,
                                         hh, weight, grad_x, grad_w_part, grad_b_part, ws, st),
                      "gconv_bwd launch");
}

}  // extern "C"
