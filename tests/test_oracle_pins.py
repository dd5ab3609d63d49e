"""Pins of the CPU oracle to things other than itself (CPU only, no GPU).

Each pin is chosen so that a plausible mistake in the oracle (a flipped or
transposed kernel, a wrong padding sign, a dropped bias, a wrong group index,
a missing stride test, a wrong column range) fails at least one of them; the
last test plants such mistakes in copies of oracle.c and checks exactly that.

* torch's CPU conv2d and autograd in float64 (an independent library routine);
* scipy's correlate2d for the depthwise case (a textbook routine);
* the patchify case as a reshape plus a numpy matmul (closed form);
* delta kernels (a pure shift) and constant inputs (sums of kernel slices);
* adjoint identities and central finite differences (exact for a bilinear map);
* the method's own pipeline -- halo exchange, concatenate, convolve, crop --
  written with torch on the extended tensor (NVIDIA blog "Perception Model
  Training for Autonomous Vehicles with Tensor Parallelism", DTensor section
  and Figure 1; kwkr.cn retelling, sections 2.2 and 3.2);
* the printed facts in tests/golden/page_facts.json.
"""
import json
import os
import pathlib
import subprocess
import tempfile

import numpy as np
import pytest
import scipy.signal
import torch
import torch.nn.functional as F

import oracle

GOLDEN = pathlib.Path(__file__).parent / "golden" / "page_facts.json"

# (n, ci, co, h, w, k, stride, pad, groups)
CASES = [
    (1, 3, 8, 8, 12, 5, 1, 2, 1),   # the pages' 5x5 / pad 2 / stride 1 example
    (2, 4, 6, 7, 9, 3, 1, 1, 2),    # grouped
    (2, 5, 5, 9, 8, 7, 1, 3, 5),    # depthwise 7x7 pad 3 (ConvNeXt)
    (1, 3, 4, 8, 8, 4, 4, 0, 1),    # patchify stem 4x4 / 4
    (2, 4, 6, 6, 10, 2, 2, 0, 1),   # downsample 2x2 / 2
    (1, 2, 3, 7, 9, 3, 2, 1, 1),    # strided with padding, odd extents
    (1, 2, 2, 5, 6, 1, 1, 0, 1),    # 1x1
    (1, 6, 4, 6, 7, 5, 2, 2, 2),    # grouped, strided, 5x5
]


def _rand(rng, shape):
    return rng.standard_normal(shape)


def _case_tensors(case, seed=0):
    n, ci, co, h, w, k, s, p, g = case
    rng = np.random.default_rng(seed)
    x = _rand(rng, (n, ci, h, w))
    wt = _rand(rng, (co, ci // g, k, k))
    b = _rand(rng, (co,))
    ho, wo = (h + 2 * p - k) // s + 1, (w + 2 * p - k) // s + 1
    gy = _rand(rng, (n, co, ho, wo))
    return x, wt, b, gy


def _close(a, b, tol=1e-11):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, (a.shape, b.shape)
    scale = max(1.0, float(np.max(np.abs(b))))
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, f"max abs err {err} (scale {scale})"


def _torch_ref(case, x, wt, b, gy):
    n, ci, co, h, w, k, s, p, g = case
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    wtt = torch.tensor(wt, dtype=torch.float64, requires_grad=True)
    bt = torch.tensor(b, dtype=torch.float64, requires_grad=True)
    y = F.conv2d(xt, wtt, bt, stride=s, padding=p, groups=g)
    y.backward(torch.tensor(gy, dtype=torch.float64))
    return y.detach().numpy(), xt.grad.numpy(), wtt.grad.numpy(), bt.grad.numpy()


# --- pin checks (reused by the mutation test) ------------------------------

def check_forward_vs_torch(case):
    x, wt, b, gy = _case_tensors(case)
    n, ci, co, h, w, k, s, p, g = case
    y_ref, _, _, _ = _torch_ref(case, x, wt, b, gy)
    _close(oracle.conv_fwd(x, wt, b, s, p, g), y_ref)


def check_gradients_vs_torch(case):
    x, wt, b, gy = _case_tensors(case, seed=1)
    n, ci, co, h, w, k, s, p, g = case
    _, dx_ref, gw_ref, gb_ref = _torch_ref(case, x, wt, b, gy)
    _close(oracle.conv_bwd_input(gy, wt, x.shape, s, p, g), dx_ref)
    gw, gb = oracle.conv_bwd_weight(x, gy, k, s, p, g)
    _close(gw, gw_ref)
    _close(gb, gb_ref)


def check_column_partition(case, parts=3):
    """Shard(3) outputs concatenate to the full result; _Partial gradients
    over disjoint output-column ranges sum to the full gradient."""
    x, wt, b, gy = _case_tensors(case, seed=2)
    n, ci, co, h, w, k, s, p, g = case
    wo = gy.shape[3]
    cuts = np.linspace(0, wo, parts + 1).astype(int)
    ys = [oracle.conv_fwd(x, wt, b, s, p, g, cols=(cuts[i], cuts[i + 1])) for i in range(parts)]
    _close(np.concatenate(ys, axis=3), oracle.conv_fwd(x, wt, b, s, p, g))
    xcuts = np.linspace(0, w, parts + 1).astype(int)
    dxs = [oracle.conv_bwd_input(gy, wt, x.shape, s, p, g, cols=(xcuts[i], xcuts[i + 1]))
           for i in range(parts)]
    _close(np.concatenate(dxs, axis=3), oracle.conv_bwd_input(gy, wt, x.shape, s, p, g))
    gws = [oracle.conv_bwd_weight(x, gy, k, s, p, g, cols=(cuts[i], cuts[i + 1])) for i in range(parts)]
    gw, gb = oracle.conv_bwd_weight(x, gy, k, s, p, g)
    _close(oracle.reduce_partials([t[0] for t in gws]), gw)
    _close(oracle.reduce_partials([t[1] for t in gws]), gb)


def check_sampled_equal_full(case):
    x, wt, b, gy = _case_tensors(case, seed=3)
    n, ci, co, h, w, k, s, p, g = case
    rng = np.random.default_rng(5)
    y = oracle.conv_fwd(x, wt, b, s, p, g)
    idx = np.stack([rng.integers(0, d, 20) for d in y.shape], axis=1)
    _close(oracle.conv_fwd_at(x, wt, b, s, p, g, idx), y[tuple(idx.T)])
    dx = oracle.conv_bwd_input(gy, wt, x.shape, s, p, g)
    idx = np.stack([rng.integers(0, d, 20) for d in dx.shape], axis=1)
    _close(oracle.conv_bwd_input_at(gy, wt, x.shape, s, p, g, idx), dx[tuple(idx.T)])
    wo = gy.shape[3]
    cols = (wo // 3, wo)
    gw, _ = oracle.conv_bwd_weight(x, gy, k, s, p, g, cols=cols)
    idx = np.stack([rng.integers(0, d, 20) for d in gw.shape], axis=1)
    _close(oracle.conv_bwd_weight_at(x, gy, k, s, p, g, idx, cols=cols), gw[tuple(idx.T)])


def check_adjoint(case):
    """<conv(X; V), G> = <V, gW(X, G)> = <X, dX(G; V)> and <b, gB> = <1 b, G>."""
    x, wt, b, gy = _case_tensors(case, seed=4)
    n, ci, co, h, w, k, s, p, g = case
    y0 = oracle.conv_fwd(x, wt, None, s, p, g)
    lhs = float(np.sum(y0 * gy))
    gw, gb = oracle.conv_bwd_weight(x, gy, k, s, p, g)
    dx = oracle.conv_bwd_input(gy, wt, x.shape, s, p, g)
    scale = float(np.sum(np.abs(y0 * gy))) + 1.0
    assert abs(lhs - float(np.sum(wt * gw))) <= 1e-12 * scale
    assert abs(lhs - float(np.sum(x * dx))) <= 1e-12 * scale
    yb = oracle.conv_fwd(x, wt, b, s, p, g) - y0
    assert abs(float(np.sum(yb * gy)) - float(np.sum(b * gb))) <= 1e-11 * (float(np.sum(np.abs(yb * gy))) + 1)


def check_finite_differences(case):
    """L = <conv(X, W, b), G> is linear in each argument, so a central
    difference equals the gradient up to rounding."""
    x, wt, b, gy = _case_tensors(case, seed=6)
    n, ci, co, h, w, k, s, p, g = case

    def loss(xx, ww, bb):
        return float(np.sum(oracle.conv_fwd(xx, ww, bb, s, p, g) * gy))

    gw, gb = oracle.conv_bwd_weight(x, gy, k, s, p, g)
    dx = oracle.conv_bwd_input(gy, wt, x.shape, s, p, g)
    rng = np.random.default_rng(9)
    eps = 0.5
    for _ in range(4):
        e = tuple(rng.integers(0, d) for d in wt.shape)
        wp, wm = wt.copy(), wt.copy()
        wp[e] += eps
        wm[e] -= eps
        fd = (loss(x, wp, b) - loss(x, wm, b)) / (2 * eps)
        assert abs(fd - gw[e]) <= 1e-9 * (1 + abs(gw[e])), (e, fd, gw[e])
        e = tuple(rng.integers(0, d) for d in x.shape)
        xp, xm = x.copy(), x.copy()
        xp[e] += eps
        xm[e] -= eps
        fd = (loss(xp, wt, b) - loss(xm, wt, b)) / (2 * eps)
        assert abs(fd - dx[e]) <= 1e-9 * (1 + abs(dx[e])), (e, fd, dx[e])
    o = int(rng.integers(0, co))
    bp, bm = b.copy(), b.copy()
    bp[o] += eps
    bm[o] -= eps
    fd = (loss(x, wt, bp) - loss(x, wt, bm)) / (2 * eps)
    assert abs(fd - gb[o]) <= 1e-9 * (1 + abs(gb[o]))


# --- tests ------------------------------------------------------------------

@pytest.mark.parametrize("case", CASES)
def test_forward_matches_torch_conv2d(case):
    check_forward_vs_torch(case)


@pytest.mark.parametrize("case", CASES)
def test_gradients_match_torch_autograd(case):
    check_gradients_vs_torch(case)


@pytest.mark.parametrize("case", CASES)
def test_column_ranges_partition_the_result(case):
    check_column_partition(case)


@pytest.mark.parametrize("case", CASES[:4])
def test_sampled_outputs_equal_full_outputs(case):
    check_sampled_equal_full(case)


@pytest.mark.parametrize("case", CASES)
def test_adjoint_identities(case):
    check_adjoint(case)


@pytest.mark.parametrize("case", [CASES[0], CASES[2], CASES[3], CASES[5]])
def test_finite_differences(case):
    check_finite_differences(case)


@pytest.mark.parametrize("case", CASES)
def test_bias_grad_closed_form(case):
    x, wt, b, gy = _case_tensors(case, seed=7)
    n, ci, co, h, w, k, s, p, g = case
    _, gb = oracle.conv_bwd_weight(x, gy, k, s, p, g)
    _close(gb, gy.sum(axis=(0, 2, 3)))
    wo = gy.shape[3]
    _close(oracle.conv_bwd_bias(gy), gb)
    _close(oracle.conv_bwd_bias(gy, cols=(1, wo)), gy[..., 1:].sum(axis=(0, 2, 3)))


@pytest.mark.parametrize("d", [-2, -1, 0, 1, 2])
def test_delta_kernel_is_a_shift(d):
    """W = delta(o = c, kh = P, kw = P + d) gives Y[..., j] = X[..., j + d] + b,
    zero beyond the global edge: pins the correlation direction and padding."""
    n, c, h, w, k, p = 2, 3, 5, 12, 5, 2
    rng = np.random.default_rng(11)
    x = rng.standard_normal((n, c, h, w))
    b = rng.standard_normal(c)
    wt = np.zeros((c, c, k, k))
    for o in range(c):
        wt[o, o, p, p + d] = 1.0
    y = oracle.conv_fwd(x, wt, b, 1, p, 1)
    exp = np.zeros_like(x)
    for j in range(w):
        if 0 <= j + d < w:
            exp[..., j] = x[..., j + d]
    _close(y, exp + b[None, :, None, None])


def test_constant_input_sums_kernel_slices():
    """X = 1: interior outputs are sum(W) + b; border outputs see only the taps
    that land inside the image (zero padding), e.g. the top-left corner of a
    5x5 pad-2 conv sums W[:, :, 2:, 2:]."""
    n, ci, co, h, w, k, p = 1, 2, 3, 9, 10, 5, 2
    rng = np.random.default_rng(12)
    x = np.ones((n, ci, h, w))
    wt = rng.standard_normal((co, ci, k, k))
    b = rng.standard_normal(co)
    y = oracle.conv_fwd(x, wt, b, 1, p, 1)
    full = wt.sum(axis=(1, 2, 3)) + b
    _close(y[0, :, 2:h - 2, 2:w - 2], np.broadcast_to(full[:, None, None], (co, h - 4, w - 4)))
    _close(y[0, :, 0, 0], wt[:, :, 2:, 2:].sum(axis=(1, 2, 3)) + b)
    _close(y[0, :, 0, w - 1], wt[:, :, 2:, :3].sum(axis=(1, 2, 3)) + b)
    _close(y[0, :, 1, 1], wt[:, :, 1:, 1:].sum(axis=(1, 2, 3)) + b)
    _close(y[0, :, h - 1, 4], wt[:, :, :3, :].sum(axis=(1, 2, 3)) + b)


def test_depthwise_equals_scipy_correlate2d():
    n, c, h, w, k = 2, 4, 9, 11, 7
    p = k // 2
    rng = np.random.default_rng(13)
    x = rng.standard_normal((n, c, h, w))
    wt = rng.standard_normal((c, 1, k, k))
    b = rng.standard_normal(c)
    y = oracle.conv_fwd(x, wt, b, 1, p, c)
    for bi in range(n):
        for ch in range(c):
            ref = scipy.signal.correlate2d(x[bi, ch], wt[ch, 0], mode="same", boundary="fill")
            _close(y[bi, ch], ref + b[ch])


@pytest.mark.parametrize("stride", [2, 4])
def test_patchify_is_reshape_and_matmul(stride):
    """K = stride, pad 0: non-overlapping patches, so conv = patches @ W^T."""
    n, ci, co, h, w = 2, 3, 5, 8, 12
    s = stride
    rng = np.random.default_rng(14)
    x = rng.standard_normal((n, ci, h, w))
    wt = rng.standard_normal((co, ci, s, s))
    b = rng.standard_normal(co)
    ho, wo = h // s, w // s
    gy = rng.standard_normal((n, co, ho, wo))
    patches = x.reshape(n, ci, ho, s, wo, s).transpose(0, 2, 4, 1, 3, 5).reshape(n * ho * wo, ci * s * s)
    wm = wt.reshape(co, -1)
    y_ref = (patches @ wm.T + b).reshape(n, ho, wo, co).transpose(0, 3, 1, 2)
    _close(oracle.conv_fwd(x, wt, b, s, 0, 1), y_ref)
    gm = gy.transpose(0, 2, 3, 1).reshape(-1, co)
    gw_ref = (gm.T @ patches).reshape(co, ci, s, s)
    dpatch = gm @ wm
    dx_ref = dpatch.reshape(n, ho, wo, ci, s, s).transpose(0, 3, 1, 4, 2, 5).reshape(n, ci, h, w)
    gw, gb = oracle.conv_bwd_weight(x, gy, s, s, 0, 1)
    _close(gw, gw_ref)
    _close(gb, gm.sum(axis=0))
    _close(oracle.conv_bwd_input(gy, wt, x.shape, s, 0, 1), dx_ref)


def test_golden_halo_width_and_shard_shapes():
    facts = json.loads(GOLDEN.read_text())
    for ex in facts["halo_examples"]:
        k, s, p = ex["kernel"], ex["stride"], ex["pad"]
        # Input columns a shard's outputs touch beyond its own: left P, right K - s - P.
        assert p == ex["halo_columns_each_side"]
        assert k - s - p == ex["halo_columns_each_side"]
        # The same count, read off the oracle: an output at the shard's first
        # column depends on exactly hl columns left of the shard.
        n, ci, h, w = 1, 1, 4, 8
        x = np.zeros((n, ci, h, w))
        wt = np.ones((1, 1, k, k))
        deps_left = 0
        for q in range(4):           # shard 1 of 2 starts at column 4
            x[:] = 0
            x[..., q] = 1
            if oracle.conv_fwd(x, wt, None, s, p, 1, cols=(4, 5))[0, 0, 1, 0] != 0:
                deps_left += 1
        assert deps_left == ex["halo_columns_each_side"]
    for ex in facts["shard_examples"]:
        t = np.zeros(ex["global_input"][:3] + [ex["global_input"][3]], dtype=np.float32)[:1]
        sl = oracle.shard_columns(t, ex["num_shards"], 1)
        assert list(sl.shape[1:]) == ex["shard_shape"][1:]


@pytest.mark.parametrize("case", [CASES[0], CASES[1], CASES[2], CASES[5]])
@pytest.mark.parametrize("num_shards", [2, 3])
def test_page_pipeline_equals_oracle_columns(case, num_shards):
    """The method as the pages describe it -- gather halos, concatenate with
    the local slice, convolve, keep the shard's columns -- reproduces the
    oracle's column range, forward and backward (pull reading of backward:
    gather grad_output halos, then correlate with the flipped kernel)."""
    n, ci, co, h, w, k, s, p, g = case
    w = w - w % (num_shards * s) + num_shards * s  # make W divisible
    case = (n, ci, co, h, w, k, s, p, g)
    x, wt, b, gy = _case_tensors(case, seed=21)
    wl, wol = w // num_shards, (w // s) // num_shards
    hl, hr = p, max(0, k - s - p)
    ghl, ghr = (k - 1 - p) // s, (p + s - 1) // s
    for sh in range(num_shards):
        xs = oracle.shard_columns(x, num_shards, sh)
        ext = np.concatenate([oracle.halo_columns(x, num_shards, sh, hl, hr)[..., :hl], xs,
                              oracle.halo_columns(x, num_shards, sh, hl, hr)[..., hl:]], axis=3)
        ext_t = torch.tensor(ext, requires_grad=True)
        wt_t = torch.tensor(wt, requires_grad=True)
        b_t = torch.tensor(b, requires_grad=True)
        # Extended tensor convolved "valid" along W, zero-padded along H.
        y = F.conv2d(ext_t, wt_t, b_t, stride=s, padding=(p, 0), groups=g)
        ys = oracle.conv_fwd(x, wt, b, s, p, g, cols=(sh * wol, (sh + 1) * wol))
        _close(y.detach().numpy(), ys, 1e-10)
        if s == 1:
            # Reading of the kwkr.cn snippet (section 3.2): convolve the
            # extended tensor with the original padding on both axes, then
            # crop P columns per side -- identical at stride 1.
            full = F.conv2d(torch.tensor(ext), torch.tensor(wt), torch.tensor(b),
                            stride=1, padding=p, groups=g)
            crop = full[..., p:full.shape[3] - p] if p else full
            _close(crop.numpy(), ys, 1e-10)
        # Backward: _Partial grad_weight of this shard = autograd through the pipeline.
        gs = oracle.shard_columns(gy, num_shards, sh)
        y.backward(torch.tensor(gs))
        gw_s, gb_s = oracle.conv_bwd_weight(x, gy, k, s, p, g, cols=(sh * wol, (sh + 1) * wol))
        _close(wt_t.grad.numpy(), gw_s, 1e-10)
        _close(b_t.grad.numpy(), gb_s, 1e-10)
        if s == 1:
            # grad_input of the shard: gather grad_output halos (K-1-P left, P right),
            # correlate with the flipped, channel-transposed kernel.
            gh = oracle.halo_columns(gy, num_shards, sh, ghl, ghr)
            gext = np.concatenate([gh[..., :ghl], gs, gh[..., ghl:]], axis=3)
            cig, cog = ci // g, co // g
            wflip = np.flip(wt, axis=(2, 3)).reshape(g, cog, cig, k, k).transpose(0, 2, 1, 3, 4)
            wflip = np.ascontiguousarray(wflip.reshape(ci, cog, k, k))
            dx = F.conv2d(torch.tensor(gext), torch.tensor(wflip), None, stride=1,
                          padding=(k - 1 - p, 0), groups=g)
            dxs = oracle.conv_bwd_input(gy, wt, x.shape, s, p, g, cols=(sh * wl, (sh + 1) * wl))
            _close(dx.numpy(), dxs, 1e-10)


@pytest.mark.parametrize("case", [CASES[0], CASES[1], CASES[2], CASES[5]])
@pytest.mark.parametrize("num_shards", [2, 3])
def test_row_pipeline_equals_oracle_rows(case, num_shards):
    """The same method along H (Shard(2), kwkr.cn retelling, section 5.2):
    gather row halos, stack them on the local rows, convolve 'valid' along H
    (zero padding along W) -- torch's conv2d and autograd -- and compare with
    the oracle's unsharded rows and its row-restricted partial gradients."""
    n, ci, co, h, w, k, s, p, g = case
    h = h - h % (num_shards * s) + num_shards * s  # make H divisible
    case = (n, ci, co, h, w, k, s, p, g)
    x, wt, b, gy = _case_tensors(case, seed=22)
    hl, hol = h // num_shards, (h // s) // num_shards
    hu, hd = p, max(0, k - s - p)
    y_full = oracle.conv_fwd(x, wt, b, s, p, g)
    for sh in range(num_shards):
        xs = oracle.shard_rows(x, num_shards, sh)
        rh = oracle.halo_rows(x, num_shards, sh, hu, hd)
        ext_t = torch.tensor(np.concatenate([rh[:, :, :hu], xs, rh[:, :, hu:]], axis=2), requires_grad=True)
        wt_t = torch.tensor(wt, requires_grad=True)
        b_t = torch.tensor(b, requires_grad=True)
        y = F.conv2d(ext_t, wt_t, b_t, stride=s, padding=(0, p), groups=g)
        rows = (sh * hol, (sh + 1) * hol)
        _close(y.detach().numpy(), y_full[:, :, rows[0]:rows[1], :], 1e-10)
        y.backward(torch.tensor(np.ascontiguousarray(gy[:, :, rows[0]:rows[1], :])))
        gw_s, gb_s = oracle.conv_bwd_weight_rows(x, gy, k, s, p, g, rows)
        _close(wt_t.grad.numpy(), gw_s, 1e-10)
        _close(b_t.grad.numpy(), gb_s, 1e-10)
    # the row partials sum to the full gradient
    parts = [oracle.conv_bwd_weight_rows(x, gy, k, s, p, g, (sh * hol, (sh + 1) * hol))[0]
             for sh in range(num_shards)]
    _close(oracle.reduce_partials(parts), oracle.conv_bwd_weight(x, gy, k, s, p, g)[0], 1e-10)


# --- mutation check ---------------------------------------------------------

MUTANTS = {
    "flipped kernel (convolution, not correlation)": (
        "acc += wt[(((int64_t)o * cig + c) * k + kh) * k + kw] *",
        "acc += wt[(((int64_t)o * cig + c) * k + (k - 1 - kh)) * k + (k - 1 - kw)] *", 1),
    "transposed kernel": (
        "acc += wt[(((int64_t)o * cig + c) * k + kh) * k + kw] *",
        "acc += wt[(((int64_t)o * cig + c) * k + kw) * k + kh] *", 1),
    "wrong padding sign in forward rows": (
        "int r = i * stride + kh - pad;", "int r = i * stride + kh + pad;", 1),
    "dropped bias": ("double acc = bias ? bias[o] : 0.0;", "double acc = 0.0;", 1),
    "wrong group index": ("int cin = g * cig + c;", "int cin = c;", 1),
    "missing stride test in grad_input": (
        "if (t < 0 || t % stride != 0) continue;", "if (t < 0) continue;", 1),
    "grad_input with unflipped kernel": (
        "acc += wt[(((int64_t)o * cig + cl) * k + kh) * k + kw] *",
        "acc += wt[(((int64_t)o * cig + cl) * k + (k - 1 - kh)) * k + (k - 1 - kw)] *", 1),
    "grad_weight without column padding": (
        "int q = j * stride + kw - pad;\n                if (q < 0 || q >= w) continue;\n                acc += g[",
        "int q = j * stride + kw;\n                if (q < 0 || q >= w) continue;\n                acc += g[", 1),
    "grad_weight summing one column too many": (
        "for (int j = j0; j < j1; j++) {\n                int q = j * stride + kw - pad;\n                if (q < 0 || q >= w) continue;\n                acc += g[",
        "for (int j = j0; j <= j1 && j < wo; j++) {\n                int q = j * stride + kw - pad;\n                if (q < 0 || q >= w) continue;\n                acc += g[", 1),
    "grad_bias over the wrong channel": (
        "acc += g[(((int64_t)b * co + o) * ho + i) * wo + j];\n    return acc;",
        "acc += g[(((int64_t)b * co + (o + 1) % co) * ho + i) * wo + j];\n    return acc;", 1),
}

PIN_CHECKS = [
    (check_forward_vs_torch, CASES[0]), (check_forward_vs_torch, CASES[1]),
    (check_forward_vs_torch, CASES[5]), (check_gradients_vs_torch, CASES[0]),
    (check_gradients_vs_torch, CASES[1]), (check_gradients_vs_torch, CASES[5]),
    (check_column_partition, CASES[0]),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_oracle_mistakes_fail_a_pin(name, monkeypatch, tmp_path):
    src = (pathlib.Path(oracle.__file__).parent / "oracle.c").read_text()
    old, new, count = MUTANTS[name]
    assert src.count(old) >= count, f"mutation anchor not found: {name}"
    mutated = src.replace(old, new, count)
    c_path = tmp_path / "mut.c"
    so_path = tmp_path / "libmut.so"
    c_path.write_text(mutated)
    subprocess.run(["gcc", "-O1", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-o",
                    str(so_path), str(c_path)], check=True)
    monkeypatch.setattr(oracle, "_lib", oracle.bind(so_path))
    failed = []
    for fn, case in PIN_CHECKS:
        try:
            fn(case)
        except AssertionError:
            failed.append(fn.__name__)
    assert failed, f"no pin caught the planted mistake: {name}"


def test_block_halos_are_the_padded_neighbourhood():
    """2-D shards: the block, its row halo and its extended column halo tile
    exactly the zero-padded neighbourhood of the block (checked by assembling
    them), and the blocks' partial gradients sum to the full gradient."""
    rng = np.random.default_rng(41)
    t = rng.standard_normal((2, 3, 12, 20))
    hu = hd = hl = hr = 2
    pad = np.pad(t, ((0, 0), (0, 0), (hu, hd), (hl, hr)))
    for sh in range(3):
        for sw in range(4):
            blk = oracle.shard_block(t, 3, 4, sh, sw)
            rows, cols = oracle.block_halos(t, 3, 4, sh, sw, hu, hd, hl, hr)
            assert rows.shape == (2, 3, hu + hd, 5) and cols.shape == (2, 3, hu + 4 + hd, hl + hr)
            mid = np.concatenate([rows[:, :, :hu], blk, rows[:, :, hu:]], axis=2)
            ext = np.concatenate([cols[:, :, :, :hl], mid, cols[:, :, :, hl:]], axis=3)
            np.testing.assert_array_equal(ext, pad[:, :, sh * 4:sh * 4 + 4 + hu + hd, sw * 5:sw * 5 + 5 + hl + hr])
            # the same halos from the one-dimensional definitions (pinned above): the row halo of the
            # block's column slice, and the column halo of the image's rows extended around the block
            np.testing.assert_array_equal(rows, oracle.halo_rows(oracle.shard_columns(t, 4, sw), 3, sh, hu, hd))
            band = pad[:, :, sh * 4:sh * 4 + 4 + hu + hd, hl:hl + 20]
            np.testing.assert_array_equal(cols, oracle.halo_columns(band, 4, sw, hl, hr))
    g = rng.standard_normal((2, 3, 12, 20))
    full = oracle.conv_bwd_weight(t, g, 5, 1, 2, 3)
    parts = [oracle.conv_bwd_weight_block(t, g, 5, 1, 2, 3, (sh * 4, sh * 4 + 4), (sw * 5, sw * 5 + 5))
             for sh in range(3) for sw in range(4)]
    np.testing.assert_allclose(oracle.reduce_partials([p[0] for p in parts]), full[0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.reduce_partials([p[1] for p in parts]), full[1], rtol=1e-12, atol=1e-12)
