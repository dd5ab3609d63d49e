"""GPU parity of the autograd layer (needs an MI355X).

`ShardedConv2d` runs on lists of W-shards (or, with dim=2, H-shards); a loss sum_s <y_s, g_s> makes the
gradient arriving at the outputs exactly g, so the input, weight and bias
gradients autograd returns are compared with the oracle's grad_input,
grad_weight and grad_bias of the unsharded layer (or chain), computed on the
global tensors in double precision.
"""
import numpy as np
import pytest
import torch

import oracle
from shard_harness import TOL_DX, TOL_FWD, TOL_GW, assert_close, host, to_dev
from spatially_sharded_cnn_amd import autograd as sa

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _draw(rng, shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float32)


def _layer(ci, co, k, s, p, g, rng):
    layer = sa.ShardedConv2d(ci, co, k, stride=s, padding=p, groups=g)
    w = _draw(rng, tuple(layer.weight.shape), 0.05)
    b = _draw(rng, (co,), 0.05)
    with torch.no_grad():
        layer.weight.copy_(to_dev(w))
        layer.bias.copy_(to_dev(b))
    return layer, dict(wt=w, b=b, k=k, stride=s, pad=p, groups=g)


def _loss(ys, gs):
    return sum((y * g).sum() for y, g in zip(ys, gs))


# (name, global input shape, co, k, stride, pad, groups, S): one layer of each kernel family
LAYERS = [
    ("depthwise7", (2, 12, 20, 4 * 32), 12, 7, 1, 3, 12, 4),
    ("dense3x3", (1, 16, 12, 2 * 48), 24, 3, 1, 1, 1, 2),
    ("patch2x2", (2, 32, 16, 2 * 64), 48, 2, 2, 0, 1, 2),
    ("stem4x4", (1, 3, 32, 4 * 64), 32, 4, 4, 0, 1, 4),
]


@pytest.mark.parametrize("case", LAYERS, ids=[c[0] for c in LAYERS])
def test_layer_gradients_match_oracle(case):
    name, shape, co, k, s, p, g, S = case
    _say(f"  {name}: input {shape} co={co} k={k} s={s} p={p} g={g} S={S}")
    rng = np.random.default_rng(3001)
    x = _draw(rng, shape)
    layer, L = _layer(shape[1], co, k, s, p, g, rng)
    xs = [t.requires_grad_() for t in sa.shard(to_dev(x), S)]
    ys = layer(xs)
    gout = _draw(rng, tuple(sa.unshard(ys).shape))
    _loss(ys, sa.shard(to_dev(gout), S)).backward()
    torch.cuda.synchronize()

    assert_close(host(sa.unshard(ys)), oracle.conv_fwd(x, L["wt"], L["b"], s, p, g), TOL_FWD, f"{name} forward")
    dx_ref = oracle.conv_bwd_input(gout, L["wt"], x.shape, s, p, g)
    assert_close(np.concatenate([host(t.grad) for t in xs], axis=3), dx_ref, TOL_DX, f"{name} grad_input")
    gw_ref, gb_ref = oracle.conv_bwd_weight(x, gout, k, s, p, g)
    assert_close(host(layer.weight.grad), gw_ref, TOL_GW, f"{name} grad_weight")
    assert_close(host(layer.bias.grad), gb_ref, TOL_GW, f"{name} grad_bias")


def _chain(rng):
    specs = [(3, 32, 4, 4, 0, 1), (32, 32, 7, 1, 3, 32), (32, 64, 2, 2, 0, 1)]   # stem, depthwise, downsample
    mods, refs = [], []
    for ci, co, k, s, p, g in specs:
        m, L = _layer(ci, co, k, s, p, g, rng)
        mods.append(m)
        refs.append(L)
    return mods, refs


def test_chain_gradients_match_oracle():
    """Stem 4x4/4 -> depthwise 7x7 -> 2x2/2 downsample on a (1,3,64,256)
    input in two shards: every parameter's gradient and the input gradient
    against the oracle's unsharded chain."""
    S = 2
    rng = np.random.default_rng(3002)
    x = _draw(rng, (1, 3, 64, 256))
    mods, refs = _chain(rng)
    xs = [t.requires_grad_() for t in sa.shard(to_dev(x), S)]
    h = xs
    for m in mods:
        h = m(h)
    gout = _draw(rng, tuple(sa.unshard(h).shape))
    _say(f"  chain: input {x.shape} -> output {tuple(gout.shape)}, S={S}")
    _loss(h, sa.shard(to_dev(gout), S)).backward()
    torch.cuda.synchronize()

    acts = oracle.stack_forward(x, refs)
    grads = oracle.stack_backward(acts, refs, gout)
    assert_close(host(sa.unshard(h)), acts[-1], TOL_FWD, "chain output")
    assert_close(np.concatenate([host(t.grad) for t in xs], axis=3), grads[0][1], TOL_DX, "chain grad_input")
    for l, m in enumerate(mods):
        _, _, gw_ref, gb_ref = grads[l]
        assert_close(host(m.weight.grad), gw_ref, TOL_GW, f"chain layer {l} grad_weight")
        assert_close(host(m.bias.grad), gb_ref, TOL_GW, f"chain layer {l} grad_bias")


def test_weight_only_backward():
    """Inputs that need no gradient take the grad_weight-only call."""
    S = 4
    rng = np.random.default_rng(3003)
    x = _draw(rng, (2, 8, 18, 4 * 16))
    layer, L = _layer(8, 8, 5, 1, 2, 8, rng)
    xs = sa.shard(to_dev(x), S)
    ys = layer(xs)
    gout = _draw(rng, tuple(sa.unshard(ys).shape))
    _loss(ys, sa.shard(to_dev(gout), S)).backward()
    torch.cuda.synchronize()
    assert all(t.grad is None for t in xs)
    gw_ref, gb_ref = oracle.conv_bwd_weight(x, gout, 5, 1, 2, 8)
    assert_close(host(layer.weight.grad), gw_ref, TOL_GW, "weight-only grad_weight")
    assert_close(host(layer.bias.grad), gb_ref, TOL_GW, "weight-only grad_bias")


def test_gradients_are_bitwise_reproducible():
    S = 2
    rng = np.random.default_rng(3004)
    x = _draw(rng, (1, 3, 64, 256))
    mods, _ = _chain(rng)
    gout = None
    results = []
    for _ in range(2):
        for m in mods:
            m.zero_grad(set_to_none=True)
        xs = [t.requires_grad_() for t in sa.shard(to_dev(x), S)]
        h = xs
        for m in mods:
            h = m(h)
        if gout is None:
            gout = _draw(rng, tuple(sa.unshard(h).shape))
        _loss(h, sa.shard(to_dev(gout), S)).backward()
        torch.cuda.synchronize()
        results.append([t.grad.clone() for t in xs] + [m.weight.grad.clone() for m in mods] +
                       [m.bias.grad.clone() for m in mods])
    for a, b in zip(*results):
        assert torch.equal(a, b)


# (name, global input shape, co, k, stride, pad, groups, S): H-shards (dim=2)
HLAYERS = [
    ("depthwise7_rows", (2, 12, 4 * 16, 40), 12, 7, 1, 3, 12, 4),
    ("dense3x3_rows", (1, 16, 2 * 24, 36), 24, 3, 1, 1, 1, 2),
    ("strided3x3_rows", (1, 6, 2 * 16, 22), 10, 3, 2, 1, 1, 2),
]


@pytest.mark.parametrize("case", HLAYERS, ids=[c[0] for c in HLAYERS])
def test_row_sharded_layer_gradients_match_oracle(case):
    """The same check with the activations split along H (Shard(2))."""
    name, shape, co, k, s, p, g, S = case
    _say(f"  {name}: input {shape} co={co} k={k} s={s} p={p} g={g} S={S} (H-shards)")
    rng = np.random.default_rng(3005)
    x = _draw(rng, shape)
    w = _draw(rng, (co, shape[1] // g, k, k), 0.05)
    b = _draw(rng, (co,), 0.05)
    layer = sa.ShardedConv2d(shape[1], co, k, stride=s, padding=p, groups=g, dim=2)
    with torch.no_grad():
        layer.weight.copy_(to_dev(w))
        layer.bias.copy_(to_dev(b))
    xs = [t.requires_grad_() for t in sa.shard(to_dev(x), S, dim=2)]
    ys = layer(xs)
    gout = _draw(rng, tuple(sa.unshard(ys, dim=2).shape))
    _loss(ys, sa.shard(to_dev(gout), S, dim=2)).backward()
    torch.cuda.synchronize()

    assert_close(host(sa.unshard(ys, dim=2)), oracle.conv_fwd(x, w, b, s, p, g), TOL_FWD, f"{name} forward")
    dx_ref = oracle.conv_bwd_input(gout, w, x.shape, s, p, g)
    assert_close(np.concatenate([host(t.grad) for t in xs], axis=2), dx_ref, TOL_DX, f"{name} grad_input")
    gw_ref, gb_ref = oracle.conv_bwd_weight(x, gout, k, s, p, g)
    assert_close(host(layer.weight.grad), gw_ref, TOL_GW, f"{name} grad_weight")
    assert_close(host(layer.bias.grad), gb_ref, TOL_GW, f"{name} grad_bias")
