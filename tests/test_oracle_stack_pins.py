"""Pins of the oracle's convolution chain (CPU only, no GPU).

``oracle.stack_forward`` / ``oracle.stack_backward`` chain the single-layer
definitions, and ``oracle.stack_shard`` gives one W-shard's share of that
chain.  Each is pinned here to something other than itself:

* torch's CPU conv2d and autograd in float64 through a stem -> depthwise ->
  depthwise -> downsample -> depthwise chain (an independent library routine
  doing the whole forward and backward, including the order of the layers and
  which gradient reaches which layer): every activation, every grad_input,
  every grad_weight and grad_bias;
* the shard's share against the full chain's columns, and its partial
  gradients against torch autograd run on the global tensors with the
  grad_output of the other shards' columns zeroed (the pages' _Partial
  placement: NVIDIA blog "Perception Model Training for Autonomous Vehicles
  with Tensor Parallelism", DTensor section);
* the matrix-product form of patchify layers (``oracle.patchify_*``) against
  the direct loops on column ranges with ragged remainders, and against torch;
* planted slips (a layer fed the wrong activation, the wrong gradient passed
  down, the layers walked in the wrong order, a window too narrow, patch taps
  transposed, a dropped bias) each fail one of these.
"""
import inspect
import textwrap

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

# name, ci, co, k, stride, pad, groups: a ConvNeXt-style chain with two
# consecutive same-shape layers, so that a slip between them changes values
# rather than shapes
CHAIN = [
    ("stem", 3, 8, 4, 4, 0, 1),
    ("dw_a", 8, 8, 7, 1, 3, 8),
    ("dw_b", 8, 8, 3, 1, 1, 8),
    ("ds", 8, 12, 2, 2, 0, 1),
    ("dw_c", 12, 12, 7, 1, 3, 12),
]
X_SHAPE = (2, 3, 32, 96)


def _chain(seed=5, x_shape=X_SHAPE, chain=CHAIN):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(x_shape)
    layers = []
    h, w = x_shape[2], x_shape[3]
    for _, ci, co, k, s, p, g in chain:
        layers.append(dict(wt=rng.standard_normal((co, ci // g, k, k)) * 0.3,
                           b=rng.standard_normal((co,)) * 0.1, k=k, stride=s, pad=p, groups=g))
        h, w = (h + 2 * p - k) // s + 1, (w + 2 * p - k) // s + 1
    g_final = rng.standard_normal((x_shape[0], chain[-1][2], h, w))
    return x, layers, g_final


def _torch_chain(x, layers, g_final, gmask=None):
    """The chain in torch float64 with autograd: returns (outputs, grads of
    each layer's input, grad_weights, grad_biases).  gmask, if given, zeroes
    the seeded gradient outside a mask."""
    xt = torch.tensor(x, requires_grad=True)
    ins, outs, wts, bts = [], [], [], []
    cur = xt
    for L in layers:
        ins.append(cur)
        wt = torch.tensor(L["wt"], requires_grad=True)
        bt = torch.tensor(L["b"], requires_grad=True)
        wts.append(wt)
        bts.append(bt)
        cur = F.conv2d(cur, wt, bt, stride=L["stride"], padding=L["pad"], groups=L["groups"])
        cur.retain_grad()
        outs.append(cur)
    for t in ins:
        t.retain_grad()
    seed = torch.tensor(g_final if gmask is None else g_final * gmask)
    outs[-1].backward(seed)
    return ([o.detach().numpy() for o in outs], [t.grad.numpy() for t in ins],
            [w.grad.numpy() for w in wts], [b.grad.numpy() for b in bts])


def _close(a, b, tol=1e-10):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, (a.shape, b.shape)
    scale = max(1.0, float(np.max(np.abs(b))))
    err = float(np.max(np.abs(a - b)))
    assert err <= tol * scale, f"max abs err {err} (scale {scale})"


def check_chain_vs_torch(seed=5):
    x, layers, g_final = _chain(seed)
    acts = oracle.stack_forward(x, layers)
    back = oracle.stack_backward(acts, layers, g_final)
    outs, dins, gws, gbs = _torch_chain(x, layers, g_final)
    assert len(acts) == len(layers) + 1
    _close(acts[0], x, 0.0)
    for l in range(len(layers)):
        _close(acts[l + 1], outs[l])
        g_out, dx, gw, gb = back[l]
        seed_l = g_final if l == len(layers) - 1 else dins[l + 1]
        _close(g_out, seed_l)
        _close(dx, dins[l])
        _close(gw, gws[l])
        _close(gb, gbs[l])


def check_shard_vs_full_chain(num_shards=4, shard=1, seed=6):
    """stack_shard equals the full chain on the shard's columns, and its
    partials equal torch autograd with the seeded gradient of every layer
    restricted to the shard's output columns."""
    x, layers, g_final = _chain(seed)
    acts = oracle.stack_forward(x, layers)
    back = oracle.stack_backward(acts, layers, g_final)
    res = oracle.stack_shard(x, layers, g_final, num_shards, shard)
    for l in range(len(layers)):
        y_full, dx_full = acts[l + 1], back[l][1]
        wo, wi = y_full.shape[3] // num_shards, dx_full.shape[3] // num_shards
        _close(res[l]["y"], y_full[:, :, :, shard * wo:(shard + 1) * wo])
        _close(res[l]["dx"], dx_full[:, :, :, shard * wi:(shard + 1) * wi])
        # the partial of layer l: the same layer's weight gradient with the
        # gradient reaching its output kept on the shard's columns only
        g_out = back[l][0]
        xt = torch.tensor(acts[l])
        wt = torch.tensor(layers[l]["wt"], requires_grad=True)
        bt = torch.tensor(layers[l]["b"], requires_grad=True)
        y = F.conv2d(xt, wt, bt, stride=layers[l]["stride"], padding=layers[l]["pad"], groups=layers[l]["groups"])
        mask = np.zeros_like(g_out)
        mask[:, :, :, shard * wo:(shard + 1) * wo] = 1.0
        y.backward(torch.tensor(g_out * mask))
        _close(res[l]["gw"], wt.grad.numpy())
        _close(res[l]["gb"], bt.grad.numpy())


def test_chain_matches_torch_autograd():
    check_chain_vs_torch()


@pytest.mark.parametrize("num_shards,shard", [(4, 0), (4, 1), (4, 3), (2, 1)])
def test_shard_share_matches_full_chain(num_shards, shard):
    check_shard_vs_full_chain(num_shards, shard)


def test_shard_share_sampled_weight_grad():
    """grad_weight at listed positions equals the full partial there."""
    x, layers, g_final = _chain(8)
    full = oracle.stack_shard(x, layers, g_final, 4, 2)
    rng = np.random.default_rng(3)
    gw_at = []
    for L in layers:
        co, cig, k, _ = L["wt"].shape
        gw_at.append(np.stack([rng.integers(0, co, 40), rng.integers(0, cig, 40),
                               rng.integers(0, k, 40), rng.integers(0, k, 40)], axis=1))
    samp = oracle.stack_shard(x, layers, g_final, 4, 2, gw_at=gw_at)
    for l in range(len(layers)):
        ix = gw_at[l]
        _close(samp[l]["gw"], full[l]["gw"][ix[:, 0], ix[:, 1], ix[:, 2], ix[:, 3]], 1e-12)
        _close(samp[l]["gb"], full[l]["gb"], 1e-12)
        _close(samp[l]["y"], full[l]["y"], 0.0)
        _close(samp[l]["dx"], full[l]["dx"], 0.0)


def test_column_ranges_of_a_receptive_field():
    """input_columns_read / output_columns_reaching against brute force: the
    columns an output range reads, and the outputs that read an input range."""
    for k, s, p in [(7, 1, 3), (5, 1, 2), (4, 4, 0), (2, 2, 0), (3, 2, 1), (1, 1, 0)]:
        w = 37 if s == 1 or p else 36
        wo = oracle.out_size(w, k, s, p)
        reads = [set(q for q in range(j * s - p, j * s - p + k) if 0 <= q < w) for j in range(wo)]
        for j0 in range(wo):
            for j1 in range(j0 + 1, wo + 1):
                cols = set().union(*reads[j0:j1])
                lo, hi = oracle.input_columns_read((j0, j1), k, s, p, w)
                if cols:
                    assert (lo, hi) == (min(cols), max(cols) + 1), (k, s, p, j0, j1)
        for x0 in range(w):
            for x1 in range(x0 + 1, w + 1):
                outs = [j for j in range(wo) if reads[j] & set(range(x0, x1))]
                lo, hi = oracle.output_columns_reaching((x0, x1), k, s, p, wo)
                if outs:
                    assert (lo, hi) == (min(outs), max(outs) + 1), (k, s, p, x0, x1)


# --- planted chain slips ----------------------------------------------------

CHAIN_MUTANTS = {
    "stack_backward: layer input off by one": ("stack_backward", "x = acts[l]", "x = acts[l + 1]"),
    "stack_backward: grad_output passed down instead of grad_input": ("stack_backward", "g = dx", "g = g"),
    "stack_backward: layers walked bottom-up": (
        "stack_backward", "for l in range(len(layers) - 1, -1, -1):", "for l in range(len(layers)):"),
    "stack_forward: every layer fed the chain's input": (
        "stack_forward", "conv_fwd(acts[-1],", "conv_fwd(acts[0],"),
    "stack_shard: forward reads beyond the columns evaluated": (
        "stack_shard", "need_out[l - 1] = _hull(own_out[l - 1], reads)", "need_out[l - 1] = own_out[l - 1]"),
    "stack_shard: grad_input reads beyond the columns evaluated": (
        "stack_shard", "need_dx[l + 1] = _hull(own_in[l + 1], _hull(own_out[l], gcols))",
        "need_dx[l + 1] = own_in[l + 1]"),
    "stack_shard: partials over all columns": (
        "stack_shard", "cols = own_out[l]\n", "cols = (0, owidths[l])\n"),
}


def _mutate(fname, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(oracle, fname)))
    assert src.count(old) == 1, f"mutation anchor not found in {fname}: {old!r}"
    ns = dict(vars(oracle))
    exec(compile(src.replace(old, new), f"<mutant {fname}>", "exec"), ns)
    return ns[fname]


@pytest.mark.parametrize("name", sorted(CHAIN_MUTANTS))
def test_planted_chain_slips_fail_a_pin(name, monkeypatch):
    fname, old, new = CHAIN_MUTANTS[name]
    monkeypatch.setattr(oracle, fname, _mutate(fname, old, new))
    caught = []
    for check in (check_chain_vs_torch, check_shard_vs_full_chain):
        try:
            check()
        except (AssertionError, ValueError, IndexError):
            caught.append(check.__name__)
    assert caught, f"no pin caught the planted slip: {name}"


# --- the matrix-product form of patchify layers -------------------------------

# (n, ci, co, h, w, k): whole patches, and extents that leave a ragged remainder
PATCH_CASES = [(2, 3, 5, 8, 12, 4), (1, 4, 6, 7, 9, 2), (2, 2, 3, 6, 10, 2), (1, 3, 4, 9, 13, 4)]


def check_patchify_vs_loops(case, seed=0):
    n, ci, co, h, w, k = case
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, ci, h, w))
    wt = rng.standard_normal((co, ci, k, k))
    b = rng.standard_normal((co,))
    ho, wo = h // k, w // k
    g = rng.standard_normal((n, co, ho, wo))
    for j0, j1 in [(0, wo), (1, wo), (0, max(1, wo - 1)), (wo // 2, wo // 2 + 1)]:
        _close(oracle.patchify_fwd(x, wt, b, k, cols=(j0, j1)),
               oracle.conv_fwd(x, wt, b, k, 0, 1, cols=(j0, j1)), 1e-12)
        gw, gb = oracle.patchify_bwd_weight(x, g, k, cols=(j0, j1))
        gw_ref, gb_ref = oracle.conv_bwd_weight(x, g, k, k, 0, 1, cols=(j0, j1))
        _close(gw, gw_ref, 1e-12)
        _close(gb, gb_ref, 1e-12)
    for x0, x1 in [(0, w), (1, w), (0, w - 1), (k - 1, k + 1), (w - 3, w), (2, 5)]:
        _close(oracle.patchify_bwd_input(g, wt, x.shape, k, cols=(x0, x1)),
               oracle.conv_bwd_input(g, wt, x.shape, k, 0, 1, cols=(x0, x1)), 1e-12)
    # and against torch, independently of the loops
    y, dx, gw_t, gb_t = _torch_chain(x, [dict(wt=wt, b=b, k=k, stride=k, pad=0, groups=1)], g)
    _close(oracle.patchify_fwd(x, wt, b, k), y[0], 1e-12)
    _close(oracle.patchify_bwd_input(g, wt, x.shape, k), dx[0], 1e-12)
    gw, gb = oracle.patchify_bwd_weight(x, g, k)
    _close(gw, gw_t[0], 1e-12)
    _close(gb, gb_t[0], 1e-12)


@pytest.mark.parametrize("case", PATCH_CASES)
def test_patchify_product_form_matches_loops_and_torch(case):
    check_patchify_vs_loops(case)


PATCH_MUTANTS = {
    "patch taps transposed": ("patchify_fwd", "xs.transpose(0, 2, 4, 1, 3, 5)", "xs.transpose(0, 2, 4, 1, 5, 3)"),
    "dropped bias": ("patchify_fwd", "y = y + _f64(bias)[None, :]", "y = y"),
    "grad_input placed one patch off": ("patchify_bwd_input", "q0 = x0 - p0 * k", "q0 = x0 - p0 * k + k"),
    "grad_input taps transposed": (
        "patchify_bwd_input", ".transpose(0, 3, 1, 4, 2, 5)", ".transpose(0, 3, 1, 5, 2, 4)"),
    "grad_weight over all columns": ("patchify_bwd_weight", "j0, j1 = (0, wo) if cols is None else cols",
                                     "j0, j1 = (0, wo)"),
}


@pytest.mark.parametrize("name", sorted(PATCH_MUTANTS))
def test_planted_patchify_slips_fail_a_pin(name, monkeypatch):
    fname, old, new = PATCH_MUTANTS[name]
    monkeypatch.setattr(oracle, fname, _mutate(fname, old, new))
    caught = 0
    for case in PATCH_CASES:
        try:
            check_patchify_vs_loops(case)
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught, f"no pin caught the planted slip: {name}"
