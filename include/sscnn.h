/*
 * sscnn.h -- C ABI of the width-sharded 2-D convolution library (libsscnn.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * The method.  A convolution's activations are split along W into S equal
 * slices, one per shard; weight and bias are replicated on every shard (NVIDIA
 * blog "Perception Model Training for Autonomous Vehicles with Tensor
 * Parallelism", DTensor section: input and output Shard(3), weight and bias
 * Replicate).  Each shard fetches the edge columns its outputs need from its
 * two W-neighbours (the halo; same blog, Figure 1: a 5x5 kernel, padding 2,
 * stride 1 needs 2 columns from each side), convolves its slice extended by
 * those columns, and keeps only the columns it owns (kwkr.cn retelling,
 * section 2.2: exchange, concatenate, convolve, crop).  In backward the
 * grad_output is exchanged the same way, grad_input comes out sharded like the
 * input, and grad_weight / grad_bias come out as per-shard partial sums that a
 * reduction turns into the replicated gradient (blog, DTensor section:
 * convolution_backward rule with _Partial grad_weight and grad_bias).
 *
 * This library computes ONE shard's share on one GPU.  The neighbours' slices
 * are ordinary device buffers; halo_gather reads their edge columns where a
 * multi-GPU run would receive them over the fabric, and partial_reduce sums
 * the shards' partial gradients where a multi-GPU run would all-reduce them.
 *
 * Conventions for every call below.
 *  - Tensors are float32, contiguous, row-major: activations NCHW, weights
 *    OIHW with I = c_in / groups.  All tensor pointers are DEVICE pointers to
 *    memory the caller allocated and owns; the library allocates nothing and
 *    keeps no pointer after a call returns.  Pointers must be 16-byte aligned.
 *  - Outputs are overwritten, never accumulated into.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL means
 *    the default stream).  A call returns after launching; results are ready
 *    when the stream is synchronised.  Faults inside a kernel surface at that
 *    synchronisation.
 *  - Every call validates its arguments on the host before launching anything.
 *    It returns SSCNN_OK (0) or a negative status; on error nothing has been
 *    launched and no output was touched.  sscnn_last_error() gives a message
 *    for the calling thread's most recent failure.
 *  - No global mutable state apart from the per-thread error message: calls
 *    may be made concurrently from several threads on different streams.
 *  - All reductions run in a fixed order: results are bitwise reproducible
 *    from run to run on the same device.
 */
#ifndef SSCNN_H
#define SSCNN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSCNN_ABI_VERSION 10

/* Status codes. */
#define SSCNN_OK 0
#define SSCNN_EINVAL (-1)        /* bad argument: NULL pointer, inconsistent shape, misalignment */
#define SSCNN_EUNSUPPORTED (-2)  /* a shape the sharding method cannot express (see sscnn_conv_init) */
#define SSCNN_EWORKSPACE (-3)    /* workspace missing or smaller than the query returned */
#define SSCNN_EHIP (-4)          /* the HIP runtime reported an error while launching */

/* Which tensor a halo is gathered for. */
#define SSCNN_HALO_INPUT 0        /* forward input X: slices (N, c_in, h, w_local) */
#define SSCNN_HALO_GRAD_OUTPUT 1  /* grad_output G: slices (N, c_out, h_out, w_out_local) */

/*
 * One convolution layer as seen by one shard.
 *
 * Caller sets the first block; sscnn_conv_init validates it and fills the
 * derived block.  The layer is the PyTorch conv2d (cross-correlation, zero
 * padding `pad` on all four sides of the GLOBAL image, square kernel k,
 * stride, groups, no dilation) applied to a global input of width
 * w_local * num_shards, whose output columns are split into num_shards equal
 * slices of w_out_local = w_local / stride columns.
 */
typedef struct sscnn_conv {
    /* set by the caller */
    int32_t n;            /* batch */
    int32_t c_in;         /* input channels */
    int32_t c_out;        /* output channels */
    int32_t h;            /* input height (never sharded) */
    int32_t w_local;      /* input columns held by this shard */
    int32_t k;            /* kernel size (k x k) */
    int32_t stride;       /* stride on both axes */
    int32_t pad;          /* zero padding on both axes */
    int32_t groups;       /* channel groups (groups == c_in == c_out: depthwise) */
    int32_t shard;        /* this shard's index s, 0 <= s < num_shards */
    int32_t num_shards;   /* S */
    /* filled by sscnn_conv_init */
    int32_t h_out;        /* (h + 2*pad - k) / stride + 1 */
    int32_t w_out_local;  /* w_local / stride: output columns owned by this shard */
    int32_t halo_l;       /* input columns needed from the left neighbour:  pad */
    int32_t halo_r;       /* input columns needed from the right neighbour: max(0, k - stride - pad) */
    int32_t ghalo_l;      /* grad_output columns needed from the left:  (k - 1 - pad) / stride */
    int32_t ghalo_r;      /* grad_output columns needed from the right: ceil(pad / stride) */
} sscnn_conv_t;

/*
 * Validate a layer description and fill its derived fields.
 * Requirements (else SSCNN_EINVAL): all sizes positive, 0 <= pad < k,
 * c_in % groups == 0, c_out % groups == 0, 0 <= shard < num_shards,
 * h + 2*pad >= k.  Requirements of the sharding itself (else
 * SSCNN_EUNSUPPORTED): w_local % stride == 0; the global output width
 * (S*w_local + 2*pad - k)/stride + 1 equals S * w_local / stride, so that
 * output columns split evenly; every halo is no wider than one slice
 * (halo_l, halo_r <= w_local and ghalo_l, ghalo_r <= w_out_local), since a
 * shard only talks to its two nearest neighbours.
 */
int sscnn_conv_init(sscnn_conv_t *conv);

/*
 * Halo exchange, single-GPU form (blog, Figure 1 and Figure 2 text; kwkr.cn
 * retelling, section 2.2).
 *
 * For which == SSCNN_HALO_INPUT the slices are (n, c_in, h, w_local) and the
 * widths (hl, hr) = (halo_l, halo_r); for SSCNN_HALO_GRAD_OUTPUT the slices
 * are (n, c_out, h_out, w_out_local) and the widths (ghalo_l, ghalo_r).
 * Writes halo, shape (n, C, rows, hl + hr): per row, first the LAST hl columns
 * of the left neighbour's slice, then the FIRST hr columns of the right
 * neighbour's slice.  At the global edges there is no neighbour and the
 * columns are zeros (the original zero padding): left_nbr must be NULL exactly
 * when shard == 0 and right_nbr exactly when shard == num_shards - 1
 * (SSCNN_EINVAL otherwise).  If hl + hr == 0 nothing is launched and halo may
 * be NULL.
 */
int sscnn_halo_gather(const sscnn_conv_t *conv, int32_t which,
                      const float *left_nbr, const float *right_nbr,
                      float *halo, void *stream);

/*
 * Forward of this shard (blog, DTensor section: aten.convolution with input
 * and output Shard(3); kwkr.cn retelling, sections 2.2 and 3.2).
 *   x      (n, c_in, h, w_local)            this shard's input slice
 *   x_halo (n, c_in, h, halo_l + halo_r)    from sscnn_halo_gather(INPUT);
 *                                           may be NULL when both widths are 0
 *   weight (c_out, c_in/groups, k, k)       replicated
 *   bias   (c_out) or NULL for no bias      replicated
 *   y      (n, c_out, h_out, w_out_local)   output: the global output's
 *                                           columns [s*w_out_local, (s+1)*w_out_local)
 */
int sscnn_conv_fwd(const sscnn_conv_t *conv, const float *x, const float *x_halo,
                   const float *weight, const float *bias, float *y, void *stream);

/*
 * grad_input of this shard (blog, DTensor section: convolution_backward with
 * grad_output and grad_input Shard(3); kwkr.cn retelling, section 2.2).  The
 * grad_output halo is pulled from the neighbours, so every grad_input column
 * is finished locally and nothing is sent back.
 *   grad_y      (n, c_out, h_out, w_out_local)        this shard's grad_output
 *   grad_y_halo (n, c_out, h_out, ghalo_l + ghalo_r)  from sscnn_halo_gather(GRAD_OUTPUT);
 *                                                     may be NULL when both widths are 0
 *   weight      (c_out, c_in/groups, k, k)
 *   grad_x      (n, c_in, h, w_local)                 output: columns
 *                                                     [s*w_local, (s+1)*w_local) of the global grad_input
 */
int sscnn_conv_bwd_input(const sscnn_conv_t *conv, const float *grad_y,
                         const float *grad_y_halo, const float *weight,
                         float *grad_x, void *stream);

/*
 * Workspace, in bytes, that sscnn_conv_bwd_weight_partial needs for this
 * layer (split reductions).  0 means none.  Returns 0 as well for an invalid
 * descriptor; the call itself then reports the error.
 */
size_t sscnn_conv_bwd_weight_workspace_bytes(const sscnn_conv_t *conv);

/*
 * _Partial grad_weight and grad_bias of this shard (blog, DTensor section:
 * grad_weight and grad_bias placed _Partial; kwkr.cn retelling, section 2.2):
 * the sums over this shard's OWN output columns only, so that the partials of
 * all shards add up to the full gradients.
 *   x           (n, c_in, h, w_local)                   forward input slice
 *   x_halo      (n, c_in, h, halo_l + halo_r)           the forward's input halo, reused
 *   grad_y      (n, c_out, h_out, w_out_local)          this shard's grad_output
 *   grad_w_part (c_out, c_in/groups, k, k)              output
 *   grad_b_part (c_out) or NULL to skip the bias gradient  output
 *   workspace   device scratch of workspace_bytes >= sscnn_conv_bwd_weight_workspace_bytes()
 *               (may be NULL when that is 0); contents are scratch on return
 */
int sscnn_conv_bwd_weight_partial(const sscnn_conv_t *conv, const float *x,
                                  const float *x_halo, const float *grad_y,
                                  float *grad_w_part, float *grad_b_part,
                                  void *workspace, size_t workspace_bytes,
                                  void *stream);

/*
 * The whole backward of this shard in one call: grad_input as
 * sscnn_conv_bwd_input and the _Partial grad_weight / grad_bias as
 * sscnn_conv_bwd_weight_partial (blog, DTensor section: one
 * convolution_backward produces grad_input, grad_weight and grad_bias from
 * the same grad_output; kwkr.cn retelling, section 2.2).  Results equal the
 * two separate calls up to float32 summation order (grad_input is
 * bitwise equal); for depthwise layers one kernel reads each grad_output tile
 * once for both gradients.
 *   x, x_halo             as for sscnn_conv_bwd_weight_partial
 *   grad_y, grad_y_halo   as for sscnn_conv_bwd_input
 *   weight                (c_out, c_in/groups, k, k)
 *   grad_x                output, as for sscnn_conv_bwd_input
 *   grad_w_part, grad_b_part (nullable), workspace, workspace_bytes
 *                         as for sscnn_conv_bwd_weight_partial (same workspace size)
 * grad_x must not alias any input.
 */
int sscnn_conv_bwd(const sscnn_conv_t *conv, const float *x, const float *x_halo,
                   const float *grad_y, const float *grad_y_halo, const float *weight,
                   float *grad_x, float *grad_w_part, float *grad_b_part,
                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * Push form of the halo exchange, for a layer whose output (or grad_input)
 * the next layer convolves with a halo: the producing call writes, besides
 * its own slice, its first hr columns into the left neighbour's halo buffer
 * and its last hl columns into the right neighbour's -- the columns the
 * neighbours' halos need (blog, Figure 1 text; kwkr.cn retelling, section
 * 2.2) -- from the registers that hold them, instead of the consumer
 * gathering them from the neighbours' slices afterwards (one 128-byte line
 * fetched per few-byte row piece).  On several GPUs these are the stores a
 * shard makes into its neighbours' memory over the fabric.
 *   hl, hr     the NEXT layer's halo widths (its sscnn_conv_t halo_l / halo_r
 *              for a forward, ghalo_l / ghalo_r for a grad_input), each at
 *              most the pushed slice's width
 *   to_left    the left neighbour's halo buffer (n, c, rows, hl + hr): this
 *              slice's columns [0, hr) land in its columns [hl, hl + hr);
 *              NULL exactly when shard == 0
 *   to_right   the right neighbour's halo buffer: this slice's last hl
 *              columns land in its columns [0, hl); NULL exactly when
 *              shard == num_shards - 1
 *   own        this shard's own halo buffer, whose side without a neighbour
 *              (left at shard 0, right at the last shard) is zeroed; may be
 *              NULL when both neighbours exist
 * After every shard's producing call, each shard's halo equals what
 * sscnn_halo_gather would have written.  The halo buffers are written, never
 * read; they may not alias any other argument.
 */
typedef struct sscnn_push {
    int32_t hl, hr;
    float *to_left;
    float *to_right;
    float *own;
} sscnn_push_t;

/* sscnn_conv_fwd that also pushes y's edge columns.  Layers on the
 * matrix-core patchify path (k == stride, pad 0, groups 1: the stem and the
 * downsamples) push from the kernel's epilogue; any other layer runs
 * sscnn_conv_fwd and then copies its edge columns (at the cost of a gather).
 * push may be NULL (then it is sscnn_conv_fwd). */
int sscnn_conv_fwd_push(const sscnn_conv_t *conv, const float *x, const float *x_halo,
                        const float *weight, const float *bias, float *y,
                        const sscnn_push_t *push, void *stream);

/* sscnn_conv_bwd that also pushes grad_x's edge columns (same paths). */
int sscnn_conv_bwd_push(const sscnn_conv_t *conv, const float *x, const float *x_halo,
                        const float *grad_y, const float *grad_y_halo, const float *weight,
                        float *grad_x, float *grad_w_part, float *grad_b_part,
                        void *workspace, size_t workspace_bytes, const sscnn_push_t *push,
                        void *stream);

/*
 * sscnn_conv_bwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The call itself allocates nothing (no
 * hipMalloc, no hipFree, no allocating library routine).  Its split-reduction
 * scratch is a device array inside the library of
 * SSCNN_NOALLOC_SCRATCH_BYTES (8 MiB): every GPU the library runs on holds
 * one copy from module load until the process ends.
 *   arguments   as for sscnn_conv_bwd, minus workspace / workspace_bytes;
 *               results are the same, bitwise
 *   device      the scratch of the CURRENT device is used, so `stream` must
 *               belong to the current device (SSCNN_EINVAL otherwise)
 * Errors: as sscnn_conv_bwd, plus SSCNN_EWORKSPACE (nothing launched) when
 * the layer needs more scratch than that,
 * sscnn_conv_bwd_weight_workspace_bytes(conv) > SSCNN_NOALLOC_SCRATCH_BYTES
 * (every depthwise layer of the ConvNeXt-XL shards fits; the dense and
 * patchify layers' split-K reductions do not).
 * Every call on one GPU shares that GPU's scratch, and the scratch keeps the
 * last call's contents (no kernel relies on it being zero).  Calls that
 * overlap in time on one GPU -- on two streams, or from two threads -- race
 * on the scratch and give wrong results: order them on one stream.
 */
#define SSCNN_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int sscnn_conv_bwd_noalloc(const sscnn_conv_t *conv, const float *x, const float *x_halo,
                           const float *grad_y, const float *grad_y_halo, const float *weight,
                           float *grad_x, float *grad_w_part, float *grad_b_part, void *stream);

/*
 * Split convolution: interior and edge halves (kwkr.cn retelling, section
 * 5.2: the computation that does not depend on the halo overlaps its
 * exchange).  The halo is needed only by the few output columns next to the
 * shard's edges, so a layer can be computed in two steps ordered on the
 * caller's streams:
 *
 *   1. an INTERIOR call, which needs no halo and may run while the halo is
 *      being exchanged: the matching monolithic call with every halo column
 *      read as zero.  Columns away from the edges are then final; the edge
 *      columns lack the terms that involve halo columns;
 *   2. after the exchange, an EDGE call, which ADDS exactly those terms in
 *      place.
 *
 * interior + edge equals the monolithic call up to float32 rounding (the edge
 * sums are added once, to the interior results), and is bitwise reproducible.
 * For layers whose halo has zero width (k == stride, pad 0) the edge calls
 * launch nothing and the interior calls are the monolithic ones.  Arguments,
 * shapes and workspace rules are those of the monolithic calls above; the
 * edge calls' outputs must hold the interior results (they are read and
 * updated, so they must not alias an input).
 */

/* sscnn_conv_fwd with x_halo read as zeros. */
int sscnn_conv_fwd_interior(const sscnn_conv_t *conv, const float *x, const float *weight,
                            const float *bias, float *y, void *stream);

/* y += the forward's terms that read x_halo (n, c_in, h, halo_l + halo_r).
 * Touches only the output columns [0, ceil(halo_l/stride)) and those whose
 * last tap reaches the right halo.  x_halo may be NULL when both widths are 0. */
int sscnn_conv_fwd_edge(const sscnn_conv_t *conv, const float *x_halo, const float *weight,
                        float *y, void *stream);

/* sscnn_conv_bwd_input with grad_y_halo read as zeros. */
int sscnn_conv_bwd_input_interior(const sscnn_conv_t *conv, const float *grad_y,
                                  const float *weight, float *grad_x, void *stream);

/* grad_x += grad_input's terms that read grad_y_halo (n, c_out, h_out,
 * ghalo_l + ghalo_r): at most k - 1 - pad columns on the left and pad on the
 * right.  grad_y_halo may be NULL when both widths are 0. */
int sscnn_conv_bwd_input_edge(const sscnn_conv_t *conv, const float *grad_y_halo,
                              const float *weight, float *grad_x, void *stream);

/* sscnn_conv_bwd_weight_partial with x_halo read as zeros (grad_b_part is
 * already complete: the bias gradient needs no halo). */
int sscnn_conv_bwd_weight_partial_interior(const sscnn_conv_t *conv, const float *x,
                                           const float *grad_y, float *grad_w_part,
                                           float *grad_b_part, void *workspace,
                                           size_t workspace_bytes, void *stream);

/* grad_w_part += the products, over this shard's own output columns, of
 * grad_y with the x_halo columns their taps read.  x_halo may be NULL when both
 * widths are 0. */
int sscnn_conv_bwd_weight_edge(const sscnn_conv_t *conv, const float *x_halo,
                               const float *grad_y, float *grad_w_part, void *stream);

/* sscnn_conv_bwd with both halos read as zeros; finish it with
 * sscnn_conv_bwd_input_edge and sscnn_conv_bwd_weight_edge. */
int sscnn_conv_bwd_interior(const sscnn_conv_t *conv, const float *x, const float *grad_y,
                            const float *weight, float *grad_x, float *grad_w_part,
                            float *grad_b_part, void *workspace, size_t workspace_bytes,
                            void *stream);

/*
 * Height sharding (kwkr.cn retelling, section 5.2: for very high input
 * resolutions the sharded dimension becomes the height, Shard(2)).  The
 * activation's rows are split into num_shards equal slices of full width;
 * weight and bias stay replicated; a shard exchanges ROWS with the shards
 * above and below it: the row halo.  Rows are contiguous in memory, so the
 * exchange moves whole rows.  Depthwise layers, and dense stride-1 3x3 /
 * 5x5 k/2-padded layers on the matrix cores, read the row halo inside their
 * tiles; any other layer convolves the local slice as its own image (the
 * interior) and then adds the terms that read a row halo.  Results equal the
 * unsharded layer's rows [s*h_out_local, (s+1)*h_out_local) up to float32
 * rounding, and the grad_weight / grad_bias partials sum, over the shards, to
 * the full gradients.  Conventions are those of the calls above.
 */
typedef struct sscnn_hconv {
    /* set by the caller */
    int32_t n;            /* batch */
    int32_t c_in;         /* input channels */
    int32_t c_out;        /* output channels */
    int32_t h_local;      /* input rows held by this shard */
    int32_t w;            /* input width (not sharded) */
    int32_t k;            /* kernel size (k x k) */
    int32_t stride;       /* stride on both axes */
    int32_t pad;          /* zero padding on both axes of the GLOBAL image */
    int32_t groups;       /* channel groups */
    int32_t shard;        /* this shard's index s, 0 <= s < num_shards (top to bottom) */
    int32_t num_shards;   /* S */
    /* filled by sscnn_hconv_init */
    int32_t h_out_local;  /* h_local / stride: output rows owned by this shard */
    int32_t w_out;        /* w / stride */
    int32_t halo_u;       /* input rows needed from the shard above: pad */
    int32_t halo_d;       /* input rows needed from the shard below: max(0, k - stride - pad) */
    int32_t ghalo_u;      /* grad_output rows needed from above: (k - 1 - pad) / stride */
    int32_t ghalo_d;      /* grad_output rows needed from below: ceil(pad / stride) */
} sscnn_hconv_t;

/*
 * Validate and fill the derived fields.  Requirements as for
 * sscnn_conv_init with the roles of rows and columns exchanged, plus
 * (SSCNN_EUNSUPPORTED otherwise) w % stride == 0 and (w + 2*pad - k)/stride
 * + 1 == w / stride, the output width the kernels produce.
 */
int sscnn_hconv_init(sscnn_hconv_t *conv);

/*
 * Row halo exchange, single-GPU form.  For which == SSCNN_HALO_INPUT the
 * slices are (n, c_in, h_local, w) and the heights (halo_u, halo_d); for
 * SSCNN_HALO_GRAD_OUTPUT they are (n, c_out, h_out_local, w_out) and
 * (ghalo_u, ghalo_d).  Writes halo, shape (n, C, hu + hd, width): per plane,
 * the LAST hu rows of up_nbr's slice, then the FIRST hd rows of down_nbr's
 * slice; zeros at the global top and bottom.  up_nbr must be NULL exactly
 * when shard == 0 and down_nbr exactly when shard == num_shards - 1.  If
 * hu + hd == 0 nothing is launched and halo may be NULL.
 */
int sscnn_row_halo_gather(const sscnn_hconv_t *conv, int32_t which, const float *up_nbr,
                          const float *down_nbr, float *halo, void *stream);

/* Forward of an H-shard: x (n, c_in, h_local, w), x_halo from
 * sscnn_row_halo_gather(INPUT) (may be NULL when both heights are 0),
 * y (n, c_out, h_out_local, w_out). */
int sscnn_hconv_fwd(const sscnn_hconv_t *conv, const float *x, const float *x_halo,
                    const float *weight, const float *bias, float *y, void *stream);

/* grad_input of an H-shard: grad_y (n, c_out, h_out_local, w_out),
 * grad_y_halo from sscnn_row_halo_gather(GRAD_OUTPUT), grad_x (n, c_in, h_local, w). */
int sscnn_hconv_bwd_input(const sscnn_hconv_t *conv, const float *grad_y,
                          const float *grad_y_halo, const float *weight, float *grad_x,
                          void *stream);

/* Workspace bytes for sscnn_hconv_bwd_weight_partial and sscnn_hconv_bwd. */
size_t sscnn_hconv_bwd_weight_workspace_bytes(const sscnn_hconv_t *conv);

/* _Partial grad_weight / grad_bias of an H-shard: sums over its OWN output rows. */
int sscnn_hconv_bwd_weight_partial(const sscnn_hconv_t *conv, const float *x,
                                   const float *x_halo, const float *grad_y,
                                   float *grad_w_part, float *grad_b_part,
                                   void *workspace, size_t workspace_bytes, void *stream);

/* grad_input and the partials in one call (one pass over grad_output for depthwise layers). */
int sscnn_hconv_bwd(const sscnn_hconv_t *conv, const float *x, const float *x_halo,
                    const float *grad_y, const float *grad_y_halo, const float *weight,
                    float *grad_x, float *grad_w_part, float *grad_b_part,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * 2-D H x W sharding: a grid of num_h x num_w shards, shard (shard_h,
 * shard_w) holding rows [shard_h*h_local, ...) and columns
 * [shard_w*w_local, ...) of every plane (the two splits of kwkr.cn retelling,
 * section 5.2, combined).  The halo arrives in two phases, as on a 2-D mesh:
 *   1. sscnn_grid_row_halo_gather: the `halo` rows above and below the block,
 *      over its own columns, from the blocks above and below;
 *   2. sscnn_grid_col_halo_gather: the `halo` columns left and right of the
 *      block over its EXTENDED rows (halo above, the block's rows, halo below),
 *      from the blocks left and right of it and the row halos THEY gathered
 *      in phase 1 -- which is how the corners arrive from the diagonal blocks.
 * Layers: depthwise (groups = c_in = c_out) stride-1 k in {3,5,7} pad k/2 with
 * w_local % 16 == 0 and h_local >= 16; dense (groups 1) stride-1 k in {3,5}
 * pad k/2 -- the pages' 5x5 pad-2 example -- with c_in and c_out multiples
 * of 4 (at least 16), w_local % 4 == 0 and a block at least pad wide and
 * tall (both on the matrix cores: their tiles read the row halo and the
 * column halo over the extended rows directly); halo = pad on every side for
 * both.  And layers with k = stride, pad 0, groups 1 (no halo: the block is
 * convolved as is).  Anything else is SSCNN_EUNSUPPORTED.  Results equal the unsharded layer's
 * output block, the partials sum to the full gradients.
 */
typedef struct sscnn_gconv {
    /* set by the caller */
    int32_t n, c_in, c_out;
    int32_t h_local, w_local;     /* the block's input rows and columns */
    int32_t k, stride, pad, groups;
    int32_t shard_h, num_h;       /* block row index (top to bottom) and grid rows */
    int32_t shard_w, num_w;       /* block column index (left to right) and grid columns */
    /* filled by sscnn_gconv_init */
    int32_t h_out_local, w_out_local;
    int32_t halo;                 /* rows above/below and columns left/right needed (input and grad_output) */
} sscnn_gconv_t;

int sscnn_gconv_init(sscnn_gconv_t *conv);

/* Phase 1: row_halo (n, c, 2*halo, w) receives the last `halo` rows of `up`
 * then the first `halo` rows of `down` (blocks of the same shape, NULL at the
 * image's top / bottom edge: zeros).  which = SSCNN_HALO_INPUT (c = c_in,
 * the input block) or SSCNN_HALO_GRAD_OUTPUT (c = c_out, the output block). */
int sscnn_grid_row_halo_gather(const sscnn_gconv_t *conv, int32_t which, const float *up,
                               const float *down, float *row_halo, void *stream);

/* Phase 2: col_halo (n, c, halo + h + halo, 2*halo) receives, for each
 * extended row, the last `halo` columns of the left block then the first
 * `halo` columns of the right block; rows beyond a neighbour's block come
 * from that neighbour's phase-1 row halo.  NULL left / right (image edge):
 * zeros; a non-NULL block needs its row halo. */
int sscnn_grid_col_halo_gather(const sscnn_gconv_t *conv, int32_t which, const float *left,
                               const float *left_row_halo, const float *right,
                               const float *right_row_halo, float *col_halo, void *stream);

int sscnn_gconv_fwd(const sscnn_gconv_t *conv, const float *x, const float *x_row_halo,
                    const float *x_col_halo, const float *weight, const float *bias, float *y,
                    void *stream);
int sscnn_gconv_bwd_input(const sscnn_gconv_t *conv, const float *grad_y, const float *gy_row_halo,
                          const float *gy_col_halo, const float *weight, float *grad_x,
                          void *stream);
size_t sscnn_gconv_bwd_weight_workspace_bytes(const sscnn_gconv_t *conv);
/* _Partial grad_weight / grad_bias: sums over this block's own outputs. */
int sscnn_gconv_bwd_weight_partial(const sscnn_gconv_t *conv, const float *x, const float *x_row_halo,
                                   const float *x_col_halo, const float *grad_y, float *grad_w_part,
                                   float *grad_b_part, void *workspace, size_t workspace_bytes,
                                   void *stream);
int sscnn_gconv_bwd(const sscnn_gconv_t *conv, const float *x, const float *x_row_halo,
                    const float *x_col_halo, const float *grad_y, const float *gy_row_halo,
                    const float *gy_col_halo, const float *weight, float *grad_x,
                    float *grad_w_part, float *grad_b_part, void *workspace,
                    size_t workspace_bytes, void *stream);

/*
 * Reduction of partial gradients into the replicated gradient (blog, DTensor
 * section: _Partial reduced to Replicate; kwkr.cn retelling, section 2.2):
 *   out[i] = parts[0][i] + parts[1][i] + ... + parts[nparts-1][i]
 * summed left to right in float32, for 0 <= i < count.
 *   parts   HOST array of nparts DEVICE pointers, 1 <= nparts <= 64
 *   out     device, count floats; may alias none of the parts
 */
int sscnn_partial_reduce(const float *const *parts, int32_t nparts, int64_t count,
                         float *out, void *stream);

/*
 * A plain streaming copy, dst[i] = src[i] for 0 <= i < count: one read and
 * one write of every element with nothing else in the kernel.  Its rate is
 * the practical HBM ceiling of this device for the bandwidth-bound steps
 * (the depthwise layers, the halo gathers, the reductions), measured beside
 * the published peak.
 *   src, dst  device, count floats each, 16-byte aligned, not overlapping
 *             (SSCNN_EINVAL otherwise); count >= 0 (0 launches nothing)
 */
int sscnn_stream_copy(const float *src, float *dst, int64_t count, void *stream);

/*
 * The ConvNeXt block's other steps, on one shard's activations.  They look at
 * one pixel (or one sample) at a time, so a shard runs them on its own slice
 * with no halo; their weight gradients are per-shard partial sums, reduced
 * with sscnn_partial_reduce like the convolutions'.  The distributed DropPath
 * layer keeps its random draws consistent across shards (kwkr.cn retelling,
 * sections 3.1 and 6.1; NVIDIA blog, ConvNeXt-XL paragraph: DropPath's
 * Bernoulli draws must agree on every GPU).  Shapes: x, y, dy, dx and h are
 * (n, c, h, w) slices; the calls need n, c, h, w >= 1, and the two layer-scale
 * calls also h * w % 4 == 0.
 */

/* LayerNorm over channels (each pixel normalised over its c values):
 *   y = (x - mean) * rstd * gamma[c] + beta[c],  rstd = 1 / sqrt(var + eps),
 * with the population variance.  mean and rstd (n, h, w) are written for the
 * backward.  gamma, beta: (c). */
int sscnn_layernorm_fwd(int32_t n, int32_t c, int32_t h, int32_t w, float eps, const float *x,
                        const float *gamma, const float *beta, float *y, float *mean, float *rstd,
                        void *stream);

/* Its gradients from the saved mean / rstd: dx (nullable: skipped), and the
 * partial sums over this slice's pixels dgamma = sum dy * xhat and
 * dbeta = sum dy (each nullable). */
int sscnn_layernorm_bwd(int32_t n, int32_t c, int32_t h, int32_t w, const float *x, const float *dy,
                        const float *gamma, const float *mean, const float *rstd, float *dx,
                        float *dgamma, float *dbeta, void *stream);

/* GELU, y = x * Phi(x) (the exact form, Phi the standard normal CDF), and its
 * gradient dx = dy * (Phi(x) + x * phi(x)); count elements. */
int sscnn_gelu_fwd(int64_t count, const float *x, float *y, void *stream);
int sscnn_gelu_bwd(int64_t count, const float *x, const float *dy, float *dx, void *stream);

/* The block's 1x1 expansion followed by GELU, in one pass: y = conv_fwd(x)
 * (the pre-activation, kept for the backward) and y_act = GELU(y), both with
 * y's shape.  conv must be pointwise (k 1, stride 1, pad 0, groups 1; it
 * needs no halo, so it serves W-, H- or 2-D shards alike, each described as
 * one whole slice) with c_in, c_out and w_local multiples of 16 and fewer
 * than 2^31 elements per tensor (SSCNN_EUNSUPPORTED otherwise).  y, y_act
 * and x must be distinct (SSCNN_EINVAL).  Equals sscnn_conv_fwd then
 * sscnn_gelu_fwd. */
int sscnn_pointwise_gelu_fwd(const sscnn_conv_t *conv, const float *x, const float *weight,
                             const float *bias, float *y, float *y_act, void *stream);

/* The gradient through the block's 1x1 projection and the GELU before it:
 * grad_x = conv_bwd_input(grad_y) * GELU'(pre), pre (x's shape) being the
 * saved pre-activation.  Same conditions as sscnn_pointwise_gelu_fwd, and
 * grad_x distinct from every input; equals sscnn_conv_bwd_input then
 * sscnn_gelu_bwd. */
int sscnn_pointwise_bwd_input_gelu(const sscnn_conv_t *conv, const float *grad_y, const float *weight,
                                   const float *pre, float *grad_x, void *stream);

/* DropPath (stochastic depth) factors for n samples: scales[i] = 1 / keep_prob
 * if sample i is kept, else 0; keep_prob >= 1 gives all ones.  Sample i is
 * kept when the first word of Philox4x32-10 (Salmon et al., SC'11) of the
 * counter (i, offset low, offset high, 0) under the key (seed low, seed high)
 * is below floor(keep_prob * 2^32) (at most 2^32 - 1).  The factors depend on
 * (seed, offset, i) only, so every shard computes the same ones; a caller
 * gives each DropPath call a distinct offset.  0 < keep_prob required. */
int sscnn_droppath_scales(uint64_t seed, uint64_t offset, int32_t n, double keep_prob,
                          float *scales, void *stream);

/* The block's tail: out = x + scales[n] * (gamma[c] * hb) (layer scale, then
 * DropPath, then the residual).  scales (n) nullable: all ones. */
int sscnn_layer_scale_residual_fwd(int32_t n, int32_t c, int32_t h, int32_t w, const float *x,
                                   const float *hb, const float *gamma, const float *scales,
                                   float *out, void *stream);

/* Its gradients: dh = (scales[n] * dout) * gamma[c] (nullable: skipped) and
 * the partial dgamma = sum over this slice of (scales[n] * dout) * hb
 * (nullable); the gradient of x is dout itself. */
int sscnn_layer_scale_residual_bwd(int32_t n, int32_t c, int32_t h, int32_t w, const float *hb,
                                   const float *dout, const float *gamma, const float *scales,
                                   float *dh, float *dgamma, void *stream);

/* Static text for a status code. */
const char *sscnn_status_string(int status);

/* Message describing the calling thread's most recent failed call ("" if none). */
const char *sscnn_last_error(void);

/* SSCNN_ABI_VERSION of the built library. */
int sscnn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSCNN_H */
