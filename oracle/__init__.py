"""CPU oracle for the width-sharded convolution -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does, and this
package imports nothing from the product: the two share no code.  Inputs come
from the seeded generators in ``spatially_sharded_cnn_amd.workloads`` (which
hold no convolution arithmetic) or from the tests themselves.

What is computed, and where it is defined:

* ``conv_fwd`` / ``conv_bwd_input`` / ``conv_bwd_weight`` -- the plain
  definitions of PyTorch ``conv2d`` and its two gradients (cross-correlation,
  zero padding, square kernel, stride, groups), in double precision, on the
  GLOBAL unsharded tensors, restricted to a column range.  NVIDIA blog
  "Perception Model Training for Autonomous Vehicles with Tensor Parallelism",
  DTensor section (placement rules of aten.convolution and
  aten.convolution_backward): the sharded result equals the unsharded one
  column-for-column, and grad_weight / grad_bias are partial sums.
* ``halo_columns`` -- what the halo exchange delivers to a shard: the
  neighbours' edge columns, zeros beyond the global edge (same blog, Figure 1:
  a 5x5 kernel with padding 2 and stride 1 needs 2 columns from each
  neighbour; kwkr.cn retelling, section 2.2).
* ``shard_rows`` / ``halo_rows`` / ``conv_bwd_weight_rows`` -- the same for
  a split along H (kwkr.cn retelling, section 5.2: Shard(2) for very high
  resolutions): the row slices, the neighbours' edge rows, and the partial
  gradients summed over a shard's own output rows.
* ``shard_block`` / ``block_halos`` / ``conv_bwd_weight_block`` -- a grid of
  both (2-D H x W sharding): a shard's block, the rows above and below it over
  its own columns, the columns beside it over its rows extended by the row
  halo (corners included), and the partial gradients over its own outputs.
* ``reduce_partials`` -- the sum that turns _Partial gradients into
  Replicate ones (blog, DTensor section; kwkr.cn retelling, section 2.2).
* ``stack_forward`` / ``stack_backward`` -- a chain of the above for a
  ConvNeXt-style convolution stack.
* ``patchify_fwd`` / ``patchify_bwd_input`` / ``patchify_bwd_weight`` -- the
  same three definitions for a kernel equal to its stride with no padding
  (the stem and the downsamples), where each output reads one disjoint
  k x k patch, with the sum over (c, kh, kw) done by one numpy matrix
  product.
* ``stack_shard`` -- one W-shard's share of that chain (its outputs,
  grad_inputs and partial gradients per layer), from the global tensors,
  evaluating only the columns those results read.

The C part (``oracle.c``) is built with plain ``gcc -O2 -fopenmp``; ``build()``
compiles it, and the loaders compile it once if it is missing.
"""
from __future__ import annotations

import ctypes
import os
import pathlib
import subprocess

import numpy as np

_HERE = pathlib.Path(__file__).resolve().parent
_SRC = _HERE / "oracle.c"
_LIB_PATH = _HERE / "liboracle.so"
_lib = None


def build(force: bool = True) -> pathlib.Path:
    """Compile oracle.c into liboracle.so (plain gcc, OpenMP)."""
    if force or not _LIB_PATH.exists() or _LIB_PATH.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB_PATH.with_suffix(".so.tmp%d" % os.getpid())
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-Wextra", "-o", str(tmp), str(_SRC)]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_D = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.POINTER(ctypes.c_int64)
_i = ctypes.c_int
_l = ctypes.c_int64


def bind(path) -> ctypes.CDLL:
    """Load a compiled oracle library from path and declare its signatures."""
    lib = ctypes.CDLL(str(path))
    lib.oracle_out_size.argtypes = [_i, _i, _i, _i]
    lib.oracle_out_size.restype = _i
    lib.oracle_conv_fwd.argtypes = [_D, _i, _i, _i, _i, _D, _i, _i, _i, _i, _i, _D, _i, _i, _D]
    lib.oracle_conv_fwd_at.argtypes = [_D, _i, _i, _i, _i, _D, _i, _i, _i, _i, _i, _D, _l, _I64, _D]
    lib.oracle_conv_bwd_input.argtypes = [_D, _i, _i, _i, _i, _D, _i, _i, _i, _i, _i, _i, _i, _i, _D]
    lib.oracle_conv_bwd_input_at.argtypes = [_D, _i, _i, _i, _i, _D, _i, _i, _i, _i, _i, _i, _l, _I64, _D]
    lib.oracle_conv_bwd_weight.argtypes = [_D, _D, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _D, _D]
    lib.oracle_conv_bwd_weight_at.argtypes = [_D, _D, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _l, _I64, _D]
    for f in (lib.oracle_conv_fwd, lib.oracle_conv_fwd_at, lib.oracle_conv_bwd_input,
              lib.oracle_conv_bwd_input_at, lib.oracle_conv_bwd_weight,
              lib.oracle_conv_bwd_weight_at):
        f.restype = None
    lib.oracle_conv_bwd_bias.argtypes = [_D, _i, _i, _i, _i, _i, _i, _D]
    lib.oracle_conv_bwd_bias.restype = None
    lib.oracle_num_threads.restype = _i
    return lib


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        _lib = bind(_LIB_PATH)
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a):
    return None if a is None else a.ctypes.data_as(_D)


def out_size(n_in: int, k: int, stride: int, pad: int) -> int:
    """Output extent along one axis: floor((n_in + 2*pad - k) / stride) + 1."""
    return (n_in + 2 * pad - k) // stride + 1


def num_threads() -> int:
    """Threads the C oracle runs on (OpenMP)."""
    return int(_load().oracle_num_threads())


def _idx(idx) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(idx, dtype=np.int64).reshape(-1, 4))
    return a


def conv_fwd(x, wt, bias, stride: int, pad: int, groups: int, cols=None) -> np.ndarray:
    """Forward conv on the global input x (N, Ci, H, W); returns float64
    (N, Co, Ho, j1 - j0) for output columns cols = (j0, j1) (default: all)."""
    x, wt = _f64(x), _f64(wt)
    b = None if bias is None else _f64(bias)
    n, ci, h, w = x.shape
    co, cig, k, k2 = wt.shape
    assert k == k2 and cig * groups == ci and co % groups == 0
    ho, wo = out_size(h, k, stride, pad), out_size(w, k, stride, pad)
    j0, j1 = (0, wo) if cols is None else cols
    y = np.empty((n, co, ho, j1 - j0), dtype=np.float64)
    _load().oracle_conv_fwd(_p(x), n, ci, h, w, _p(wt), co, k, stride, pad, groups,
                            _p(b), j0, j1, _p(y))
    return y


def conv_fwd_at(x, wt, bias, stride: int, pad: int, groups: int, idx) -> np.ndarray:
    """Forward outputs at global positions idx (rows of (n, o, i, j))."""
    x, wt = _f64(x), _f64(wt)
    b = None if bias is None else _f64(bias)
    n, ci, h, w = x.shape
    co, _, k, _ = wt.shape
    ix = _idx(idx)
    out = np.empty(len(ix), dtype=np.float64)
    _load().oracle_conv_fwd_at(_p(x), n, ci, h, w, _p(wt), co, k, stride, pad, groups,
                               _p(b), len(ix), ix.ctypes.data_as(_I64), _p(out))
    return out


def conv_bwd_input(g, wt, in_shape, stride: int, pad: int, groups: int, cols=None) -> np.ndarray:
    """grad_input from the global grad_output g (N, Co, Ho, Wo) for an input of
    shape in_shape = (N, Ci, H, W), over input columns cols = (x0, x1)."""
    g, wt = _f64(g), _f64(wt)
    n, co, ho, wo = g.shape
    _, ci, h, w = in_shape
    k = wt.shape[2]
    assert wt.shape[0] == co and wt.shape[1] * groups == ci
    assert ho == out_size(h, k, stride, pad) and wo == out_size(w, k, stride, pad)
    x0, x1 = (0, w) if cols is None else cols
    dx = np.empty((n, ci, h, x1 - x0), dtype=np.float64)
    _load().oracle_conv_bwd_input(_p(g), n, co, ho, wo, _p(wt), ci, h, k, stride, pad,
                                  groups, x0, x1, _p(dx))
    return dx


def conv_bwd_input_at(g, wt, in_shape, stride: int, pad: int, groups: int, idx) -> np.ndarray:
    """grad_input at global positions idx (rows of (n, c, y, x))."""
    g, wt = _f64(g), _f64(wt)
    n, co, ho, wo = g.shape
    _, ci, h, w = in_shape
    k = wt.shape[2]
    ix = _idx(idx)
    out = np.empty(len(ix), dtype=np.float64)
    _load().oracle_conv_bwd_input_at(_p(g), n, co, ho, wo, _p(wt), ci, h, k, stride, pad,
                                     groups, len(ix), ix.ctypes.data_as(_I64), _p(out))
    return out


def conv_bwd_weight(x, g, k: int, stride: int, pad: int, groups: int, cols=None):
    """(grad_weight, grad_bias) summed over output columns cols = (j0, j1)
    (default: all, i.e. the full gradient)."""
    x, g = _f64(x), _f64(g)
    n, ci, h, w = x.shape
    co = g.shape[1]
    ho, wo = out_size(h, k, stride, pad), out_size(w, k, stride, pad)
    assert g.shape == (n, co, ho, wo)
    j0, j1 = (0, wo) if cols is None else cols
    gw = np.empty((co, ci // groups, k, k), dtype=np.float64)
    gb = np.empty((co,), dtype=np.float64)
    _load().oracle_conv_bwd_weight(_p(x), _p(g), n, ci, h, w, co, k, stride, pad, groups,
                                   j0, j1, _p(gw), _p(gb))
    return gw, gb


def conv_bwd_bias(g, cols=None) -> np.ndarray:
    """grad_bias over output columns cols = (j0, j1) of the global grad_output g."""
    g = _f64(g)
    n, co, ho, wo = g.shape
    j0, j1 = (0, wo) if cols is None else cols
    gb = np.empty((co,), dtype=np.float64)
    _load().oracle_conv_bwd_bias(_p(g), n, co, ho, wo, j0, j1, _p(gb))
    return gb


def conv_bwd_weight_at(x, g, k: int, stride: int, pad: int, groups: int, idx, cols=None) -> np.ndarray:
    """grad_weight at positions idx (rows of (o, c, kh, kw)) over columns cols."""
    x, g = _f64(x), _f64(g)
    n, ci, h, w = x.shape
    co = g.shape[1]
    wo = out_size(w, k, stride, pad)
    j0, j1 = (0, wo) if cols is None else cols
    ix = _idx(idx)
    out = np.empty(len(ix), dtype=np.float64)
    _load().oracle_conv_bwd_weight_at(_p(x), _p(g), n, ci, h, w, co, k, stride, pad, groups,
                                      j0, j1, len(ix), ix.ctypes.data_as(_I64), _p(out))
    return out


def shard_columns(t, num_shards: int, shard: int) -> np.ndarray:
    """Shard(3): the shard-th of num_shards equal slices of t along W."""
    w = t.shape[3]
    assert w % num_shards == 0
    wl = w // num_shards
    return t[:, :, :, shard * wl:(shard + 1) * wl]


def halo_columns(t, num_shards: int, shard: int, hl: int, hr: int) -> np.ndarray:
    """The halo a shard receives: columns [s*Wl - hl, s*Wl) then
    [(s+1)*Wl, (s+1)*Wl + hr) of the global tensor t, zero where they fall
    outside [0, W).  Returned in the compact layout (N, C, H, hl + hr)."""
    n, c, h, w = t.shape
    wl = w // num_shards
    out = np.zeros((n, c, h, hl + hr), dtype=t.dtype)
    for e in range(hl):
        q = shard * wl - hl + e
        if 0 <= q < w:
            out[:, :, :, e] = t[:, :, :, q]
    for e in range(hr):
        q = (shard + 1) * wl + e
        if 0 <= q < w:
            out[:, :, :, hl + e] = t[:, :, :, q]
    return out


def shard_rows(t, num_shards: int, shard: int) -> np.ndarray:
    """Shard(2): the shard-th of num_shards equal slices of t along H (the
    height split of kwkr.cn retelling, section 5.2)."""
    h = t.shape[2]
    assert h % num_shards == 0
    hl = h // num_shards
    return t[:, :, shard * hl:(shard + 1) * hl, :]


def halo_rows(t, num_shards: int, shard: int, hu: int, hd: int) -> np.ndarray:
    """The row halo an H-shard receives: rows [s*Hl - hu, s*Hl) then
    [(s+1)*Hl, (s+1)*Hl + hd) of the global tensor t, zero where they fall
    outside [0, H).  Returned as (N, C, hu + hd, W)."""
    n, c, h, w = t.shape
    hl = h // num_shards
    out = np.zeros((n, c, hu + hd, w), dtype=t.dtype)
    for e in range(hu):
        q = shard * hl - hu + e
        if 0 <= q < h:
            out[:, :, e, :] = t[:, :, q, :]
    for e in range(hd):
        q = (shard + 1) * hl + e
        if 0 <= q < h:
            out[:, :, hu + e, :] = t[:, :, q, :]
    return out


def conv_bwd_weight_rows(x, g, k: int, stride: int, pad: int, groups: int, rows):
    """grad_weight / grad_bias summed over the output rows [rows[0], rows[1])
    only: an H-shard's _Partial gradients.  The sum over a subset of the
    outputs is the gradient with grad_output zero elsewhere."""
    gm = np.zeros_like(np.asarray(g, dtype=np.float64))
    gm[:, :, rows[0]:rows[1], :] = np.asarray(g, dtype=np.float64)[:, :, rows[0]:rows[1], :]
    return conv_bwd_weight(x, gm, k, stride, pad, groups)


def shard_block(t, num_h: int, num_w: int, sh: int, sw: int) -> np.ndarray:
    """2-D H x W sharding: the (sh, sw) block of an num_h x num_w grid of equal
    blocks of t (kwkr.cn retelling, section 5.2 splits H or W; a grid of both
    is the two-dimensional case of the same method)."""
    n, c, h, w = t.shape
    assert h % num_h == 0 and w % num_w == 0
    bh, bw = h // num_h, w // num_w
    return t[:, :, sh * bh:(sh + 1) * bh, sw * bw:(sw + 1) * bw]


def block_halos(t, num_h: int, num_w: int, sh: int, sw: int, hu: int, hd: int, hl: int, hr: int):
    """What a 2-D shard receives, straight from the global tensor: the rows
    above and below its block over its own columns, (N, C, hu + hd, bw); and
    the columns left and right of it over its extended rows (the block's rows
    plus hu above and hd below, so the four corners are included),
    (N, C, hu + bh + hd, hl + hr).  Zeros outside the image."""
    n, c, h, w = t.shape
    bh, bw = h // num_h, w // num_w
    r0, c0 = sh * bh, sw * bw
    pad = np.zeros((n, c, h + hu + hd, w + hl + hr), dtype=t.dtype)
    pad[:, :, hu:hu + h, hl:hl + w] = t
    rows = np.concatenate([pad[:, :, r0:r0 + hu, hl + c0:hl + c0 + bw],
                           pad[:, :, hu + r0 + bh:hu + r0 + bh + hd, hl + c0:hl + c0 + bw]], axis=2)
    cols = np.concatenate([pad[:, :, r0:r0 + hu + bh + hd, c0:c0 + hl],
                           pad[:, :, r0:r0 + hu + bh + hd, hl + c0 + bw:hl + c0 + bw + hr]], axis=3)
    return rows, cols


def conv_bwd_weight_block(x, g, k: int, stride: int, pad: int, groups: int, rows, cols):
    """grad_weight / grad_bias summed over the output block rows x cols only:
    a 2-D shard's _Partial gradients (grad_output zero elsewhere)."""
    g64 = np.asarray(g, dtype=np.float64)
    gm = np.zeros_like(g64)
    gm[:, :, rows[0]:rows[1], cols[0]:cols[1]] = g64[:, :, rows[0]:rows[1], cols[0]:cols[1]]
    return conv_bwd_weight(x, gm, k, stride, pad, groups)


def reduce_partials(parts) -> np.ndarray:
    """Sum of the per-shard partial gradients, in shard order, in double."""
    acc = np.zeros(np.asarray(parts[0]).shape, dtype=np.float64)
    for p in parts:
        acc = acc + np.asarray(p, dtype=np.float64)
    return acc


# --- convolution stack (chain of the definitions above) -------------------

def stack_forward(x, layers):
    """Run a chain of convolutions on the global input.  layers is a list of
    dicts with keys wt, b, k, stride, pad, groups.  Returns the list of layer
    inputs acts[0..L] (acts[0] = x, acts[l+1] = output of layer l), float64."""
    acts = [_f64(x)]
    for L in layers:
        acts.append(conv_fwd(acts[-1], L["wt"], L["b"], L["stride"], L["pad"], L["groups"]))
    return acts


def stack_backward(acts, layers, g_final):
    """Backward through the chain seeded with g_final (grad of the last
    output).  Returns, per layer l, (g_out_l, dx_l, gw_l, gb_l) in float64,
    where g_out_l is the gradient arriving at layer l's output and dx_l the
    gradient it passes to its input (dx_l == g_out_{l-1})."""
    out = [None] * len(layers)
    g = _f64(g_final)
    for l in range(len(layers) - 1, -1, -1):
        L = layers[l]
        x = acts[l]
        dx = conv_bwd_input(g, L["wt"], x.shape, L["stride"], L["pad"], L["groups"])
        gw, gb = conv_bwd_weight(x, g, L["k"], L["stride"], L["pad"], L["groups"])
        out[l] = (g, dx, gw, gb)
        g = dx
    return out


# --- patchify layers (kernel = stride, no padding) as a product of matrices --

def _is_patchify(k: int, stride: int, pad: int, groups: int) -> bool:
    return k == stride and pad == 0 and groups == 1


def patchify_fwd(x, wt, bias, k: int, cols=None) -> np.ndarray:
    """Forward of a k x k / stride k / pad 0 convolution written as the sum of
    its definition over (c, kh, kw) done by one matrix product: the patches of
    output columns cols = (j0, j1) laid out as rows (n, i, j) x (c, kh, kw),
    times the weight laid out as (o) x (c, kh, kw).  The same numbers as
    ``conv_fwd`` (each output reads exactly the k x k block at (i*k, j*k)),
    up to summation order."""
    x, wt = _f64(x), _f64(wt)
    n, ci, h, w = x.shape
    co = wt.shape[0]
    ho, wo = h // k, w // k
    j0, j1 = (0, wo) if cols is None else cols
    xs = x[:, :, :ho * k, j0 * k:j1 * k].reshape(n, ci, ho, k, j1 - j0, k)
    patches = xs.transpose(0, 2, 4, 1, 3, 5).reshape(n * ho * (j1 - j0), ci * k * k)
    y = patches @ wt.reshape(co, ci * k * k).T
    if bias is not None:
        y = y + _f64(bias)[None, :]
    return np.ascontiguousarray(y.reshape(n, ho, j1 - j0, co).transpose(0, 3, 1, 2))


def patchify_bwd_input(g, wt, in_shape, k: int, cols=None) -> np.ndarray:
    """grad_input of the same layer over input columns cols = (x0, x1): input
    column q gets the gradient of output column q // k through tap q % k (and
    none when it lies beyond the last whole patch, as do rows beyond the last
    whole patch row).  The sum over output channels is one matrix product."""
    g, wt = _f64(g), _f64(wt)
    n, co, ho, wo = g.shape
    _, ci, h, w = in_shape
    x0, x1 = (0, w) if cols is None else cols
    dx = np.zeros((n, ci, h, x1 - x0), dtype=np.float64)
    p0, p1 = x0 // k, min(wo, -(-x1 // k))
    if p1 > p0:
        gm = g[:, :, :, p0:p1].transpose(0, 2, 3, 1).reshape(n * ho * (p1 - p0), co)
        dp = gm @ wt.reshape(co, ci * k * k)
        blk = dp.reshape(n, ho, p1 - p0, ci, k, k).transpose(0, 3, 1, 4, 2, 5).reshape(n, ci, ho * k, (p1 - p0) * k)
        q0 = x0 - p0 * k
        q1 = min(x1 - p0 * k, (p1 - p0) * k)
        dx[:, :, :ho * k, 0:q1 - q0] = blk[:, :, :, q0:q1]
    return dx


def patchify_bwd_weight(x, g, k: int, cols=None):
    """(grad_weight, grad_bias) of the same layer summed over output columns
    cols = (j0, j1): the sum over (n, i, j) of grad_output times the patch,
    as one matrix product; grad_bias is the sum of grad_output."""
    x, g = _f64(x), _f64(g)
    n, ci, h, w = x.shape
    _, co, ho, wo = g.shape
    j0, j1 = (0, wo) if cols is None else cols
    xs = x[:, :, :ho * k, j0 * k:j1 * k].reshape(n, ci, ho, k, j1 - j0, k)
    patches = xs.transpose(0, 2, 4, 1, 3, 5).reshape(n * ho * (j1 - j0), ci * k * k)
    gm = g[:, :, :, j0:j1].transpose(0, 2, 3, 1).reshape(n * ho * (j1 - j0), co)
    gw = (gm.T @ patches).reshape(co, ci, k, k)
    gb = gm.sum(axis=0)
    return gw, gb


# --- one shard's share of a convolution stack, from the global tensors -------

def _shard_range(width: int, num_shards: int, shard: int):
    """Shard(3) column range [s*W/S, (s+1)*W/S) of a width-W tensor."""
    assert width % num_shards == 0
    wl = width // num_shards
    return shard * wl, (shard + 1) * wl


def _hull(a, b):
    return min(a[0], b[0]), max(a[1], b[1])


def input_columns_read(out_cols, k: int, stride: int, pad: int, w: int):
    """Input columns that the output columns [j0, j1) read: output j reads
    j*stride - pad + kw for kw < k, clipped to the image [0, w)."""
    j0, j1 = out_cols
    return max(0, j0 * stride - pad), min(w, (j1 - 1) * stride - pad + k)


def output_columns_reaching(in_cols, k: int, stride: int, pad: int, wo: int):
    """Output columns whose receptive field meets the input columns
    [x0, x1): output j reads input j*stride - pad + kw, so it meets [x0, x1)
    when j*stride is in (x0 + pad - k, x1 - 1 + pad]; clipped to [0, wo)."""
    x0, x1 = in_cols
    lo = -((-(x0 + pad - k + 1)) // stride)     # ceil((x0 + pad - k + 1) / stride)
    hi = (x1 - 1 + pad) // stride + 1
    return max(0, lo), min(wo, hi)


def stack_shard(x, layers, g_final, num_shards: int, shard: int, gw_at=None):
    """One W-shard's share of a convolution chain, computed from the GLOBAL
    input x and the global gradient g_final of the last output, exactly as
    ``stack_forward`` / ``stack_backward`` would give it but without
    evaluating columns the shard's results never read.

    Layer l's output is evaluated only on the columns needed for (a) the
    shard's own output columns and (b) the columns the next layer reads;
    every other column stays zero and is never read (the sums of the
    definitions above reach only the receptive field).  Backward likewise
    evaluates each layer's grad_input only on the shard's input columns plus
    those the layer below reads.  The chain's placements are those of the
    pages: every activation and gradient Shard(3), weights replicated,
    weight / bias gradients partial over the shard's own output columns
    (NVIDIA blog "Perception Model Training for Autonomous Vehicles with
    Tensor Parallelism", DTensor section).  Patchify layers (kernel = stride,
    no padding) use the matrix-product form of the same definitions
    (``patchify_*``); every other layer uses the direct loops.

    layers: dicts with keys wt, b, k, stride, pad, groups (as for
    stack_forward).  gw_at: optional per-layer list; where entry l is an
    index array (rows of (o, c, kh, kw)), grad_weight is evaluated only there
    (returned as a flat array), otherwise in full.

    Returns per layer a dict with float64 arrays:
      y   -- the layer's output on the shard's output columns (N, Co, Ho, Wo/S)
      dx  -- grad of the layer's input on the shard's input columns (N, Ci, H, W/S)
      gw  -- grad_weight partial over the shard's output columns (full or at gw_at[l])
      gb  -- grad_bias partial over the shard's output columns (Co,)
    """
    nl = len(layers)
    x = _f64(x)
    widths, owidths = [], []
    w = x.shape[3]
    for L in layers:
        widths.append(w)
        w = out_size(w, L["k"], L["stride"], L["pad"])
        owidths.append(w)
    own_in = [_shard_range(widths[l], num_shards, shard) for l in range(nl)]
    own_out = [_shard_range(owidths[l], num_shards, shard) for l in range(nl)]

    # forward: the output columns each layer must produce, from the top down
    need_out = [None] * nl
    need_out[nl - 1] = own_out[nl - 1]
    for l in range(nl - 1, 0, -1):
        L = layers[l]
        reads = input_columns_read(need_out[l], L["k"], L["stride"], L["pad"], widths[l])
        need_out[l - 1] = _hull(own_out[l - 1], reads)

    # backward: the input columns each layer's grad_input must cover, from the bottom up
    need_dx = [None] * nl
    need_dx[0] = own_in[0]
    for l in range(nl - 1):
        L = layers[l]
        gcols = output_columns_reaching(need_dx[l], L["k"], L["stride"], L["pad"], owidths[l])
        need_dx[l + 1] = _hull(own_in[l + 1], _hull(own_out[l], gcols))

    patch = [_is_patchify(L["k"], L["stride"], L["pad"], L["groups"]) for L in layers]
    res = [dict() for _ in range(nl)]
    acts = [x]
    for l, L in enumerate(layers):
        j0, j1 = need_out[l]
        if patch[l]:
            yw = patchify_fwd(acts[l], L["wt"], L["b"], L["k"], cols=(j0, j1))
        else:
            yw = conv_fwd(acts[l], L["wt"], L["b"], L["stride"], L["pad"], L["groups"], cols=(j0, j1))
        full = np.zeros(yw.shape[:3] + (owidths[l],), dtype=np.float64)
        full[:, :, :, j0:j1] = yw
        o0, o1 = own_out[l]
        res[l]["y"] = full[:, :, :, o0:o1].copy()
        acts.append(full)

    g = _f64(g_final)
    for l in range(nl - 1, -1, -1):
        L = layers[l]
        xin = acts[l]
        x0, x1 = need_dx[l]
        if patch[l]:
            dxw = patchify_bwd_input(g, L["wt"], xin.shape, L["k"], cols=(x0, x1))
        else:
            dxw = conv_bwd_input(g, L["wt"], xin.shape, L["stride"], L["pad"], L["groups"], cols=(x0, x1))
        full = np.zeros(xin.shape, dtype=np.float64)
        full[:, :, :, x0:x1] = dxw
        i0, i1 = own_in[l]
        res[l]["dx"] = full[:, :, :, i0:i1].copy()
        cols = own_out[l]
        if patch[l]:
            gw, res[l]["gb"] = patchify_bwd_weight(xin, g, L["k"], cols=cols)
            if gw_at is not None and gw_at[l] is not None:
                ix = _idx(gw_at[l])
                gw = gw[ix[:, 0], ix[:, 1], ix[:, 2], ix[:, 3]]
            res[l]["gw"] = gw
        elif gw_at is not None and gw_at[l] is not None:
            res[l]["gw"] = conv_bwd_weight_at(xin, g, L["k"], L["stride"], L["pad"], L["groups"],
                                              gw_at[l], cols=cols)
            res[l]["gb"] = conv_bwd_bias(g, cols=cols)
        else:
            res[l]["gw"], res[l]["gb"] = conv_bwd_weight(xin, g, L["k"], L["stride"], L["pad"],
                                                         L["groups"], cols=cols)
        acts[l + 1] = None            # the output of layer l is no longer needed
        g = full
    return res
