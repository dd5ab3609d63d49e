"""Pins of the block-operation oracle (oracle/blockops.py), no GPU.

Each function is checked against something other than itself:
* Philox4x32-10 against its published known-answer vectors (tests/golden);
* the DropPath factors against their definition's statistics and edge cases;
* LayerNorm over channels against torch.nn.functional.layer_norm (float64,
  channels moved last) and against its defining invariants;
* GELU against torch.nn.functional.gelu (exact form, float64) and closed values;
* every backward against torch autograd in float64 and central differences.
"""
import math
import pathlib

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import blockops as B

GOLDEN = pathlib.Path(__file__).resolve().parent / "golden" / "philox4x32_10_kat.txt"


def _kat():
    rows = []
    for line in GOLDEN.read_text().splitlines():
        if line.strip() and not line.startswith("#"):
            w = [int(t, 16) for t in line.split()]
            rows.append((w[0:4], w[4:6], w[6:10]))
    return rows


def test_philox_known_answers():
    rows = _kat()
    assert len(rows) == 3
    for ctr, key, out in rows:
        assert B.philox4x32_10(ctr, key) == out


def test_droppath_scales_definition():
    n, keep = 4000, 0.75
    s = B.droppath_scales(seed=1234, offset=7, n=n, keep_prob=keep)
    vals = set(np.unique(s).tolist())
    assert vals <= {0.0, float(np.float32(1.0 / keep))}
    kept = (s > 0).mean()
    assert abs(kept - keep) < 4 * math.sqrt(keep * (1 - keep) / n)       # binomial, 4 sigma
    # the same (seed, offset) gives the same draws; another offset or seed gives others
    assert np.array_equal(s, B.droppath_scales(1234, 7, n, keep))
    assert not np.array_equal(s, B.droppath_scales(1234, 8, n, keep))
    assert not np.array_equal(s, B.droppath_scales(1235, 7, n, keep))
    # a sample's draw does not depend on how many samples are drawn (shard-independent)
    assert np.array_equal(s[:100], B.droppath_scales(1234, 7, 100, keep))
    # the decision is the first Philox word against floor(keep * 2^32)
    w = B.philox4x32_10((5, 7, 0, 0), (1234, 0))[0]
    assert (s[5] > 0) == (w < math.floor(keep * 2 ** 32))
    assert np.array_equal(B.droppath_scales(1, 2, 9, 1.0), np.ones(9, np.float32))


def _rand(shape, seed, scale=1.0, shift=0.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale + shift


def test_layernorm_matches_torch_and_invariants():
    x = _rand((2, 12, 5, 7), 1, 2.0, 0.5)
    g, b = _rand(12, 2), _rand(12, 3)
    y, mean, rstd = B.layernorm_channels_fwd(x, g, b, 1e-6)
    ref = F.layer_norm(torch.from_numpy(x).permute(0, 2, 3, 1), (12,), torch.from_numpy(g), torch.from_numpy(b),
                       1e-6).permute(0, 3, 1, 2).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    # with unit weight and zero bias each pixel has mean 0 and variance var/(var+eps)
    yh, _, _ = B.layernorm_channels_fwd(x, np.ones(12), np.zeros(12), 1e-6)
    np.testing.assert_allclose(yh.mean(axis=1), 0.0, atol=1e-12)
    var = x.var(axis=1)
    np.testing.assert_allclose((yh ** 2).mean(axis=1), var / (var + 1e-6), rtol=1e-12)
    np.testing.assert_allclose(mean, x.mean(axis=1), rtol=1e-12)
    np.testing.assert_allclose(rstd, 1 / np.sqrt(var + 1e-6), rtol=1e-12)


def _torch_grads(fn, inputs, dy):
    ts = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in inputs]
    out = fn(*ts)
    out.backward(torch.from_numpy(np.asarray(dy, dtype=np.float64)))
    return [t.grad.numpy() for t in ts]


def test_layernorm_backward_matches_autograd_and_differences():
    x = _rand((2, 8, 3, 5), 4, 1.5)
    g, b = _rand(8, 5), _rand(8, 6)
    dy = _rand(x.shape, 7)
    dx, dg, db = B.layernorm_channels_bwd(x, dy, g, 1e-6)
    tx, tg, tb = _torch_grads(lambda x_, g_, b_: F.layer_norm(x_.permute(0, 2, 3, 1), (8,), g_, b_, 1e-6)
                              .permute(0, 3, 1, 2), [x, g, b], dy)
    np.testing.assert_allclose(dx, tx, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dg, tg, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(db, tb, rtol=1e-10, atol=1e-12)
    # central differences of L = <y, dy> in a few input coordinates
    L = lambda xx: float((B.layernorm_channels_fwd(xx, g, b, 1e-6)[0] * dy).sum())
    for idx in [(0, 0, 0, 0), (1, 5, 2, 4), (0, 7, 1, 2)]:
        e = np.zeros_like(x)
        e[idx] = 1e-6
        fd = (L(x + e) - L(x - e)) / 2e-6
        assert abs(fd - dx[idx]) < 1e-6 * max(1.0, abs(dx[idx]))


def test_gelu_matches_torch_and_closed_values():
    x = np.linspace(-8, 8, 401)
    np.testing.assert_allclose(B.gelu_fwd(x), F.gelu(torch.from_numpy(x)).numpy(), rtol=1e-13, atol=1e-15)
    assert B.gelu_fwd(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(B.gelu_fwd(np.array([1.0])), [0.5 * (1 + math.erf(1 / math.sqrt(2)))], rtol=1e-15)
    np.testing.assert_allclose(B.gelu_fwd(np.array([-30.0, 30.0])), [0.0, 30.0], atol=1e-12)
    dy = _rand(x.shape, 8)
    (tx,) = _torch_grads(lambda t: F.gelu(t), [x], dy)
    np.testing.assert_allclose(B.gelu_bwd(x, dy), tx, rtol=1e-12, atol=1e-14)
    for v in (-2.5, -0.3, 0.0, 0.7, 3.1):
        fd = (B.gelu_fwd(np.array([v + 1e-6]))[0] - B.gelu_fwd(np.array([v - 1e-6]))[0]) / 2e-6
        assert abs(fd - B.gelu_bwd(np.array([v]), np.array([1.0]))[0]) < 1e-8


def test_layer_scale_residual_matches_autograd():
    x, h = _rand((3, 6, 4, 5), 9), _rand((3, 6, 4, 5), 10)
    gamma, s = _rand(6, 11), np.array([2.0, 0.0, 2.0])
    out = B.layer_scale_residual_fwd(x, h, gamma, s)
    np.testing.assert_allclose(out[1], x[1])                       # a dropped sample passes through
    np.testing.assert_allclose(out[0], x[0] + 2.0 * gamma[:, None, None] * h[0], rtol=1e-14)
    dout = _rand(x.shape, 12)
    dh, dg = B.layer_scale_residual_bwd(h, dout, gamma, s)
    th, tg = _torch_grads(lambda h_, g_: torch.from_numpy(x) + torch.from_numpy(s)[:, None, None, None] *
                          (g_[None, :, None, None] * h_), [h, gamma], dout)
    np.testing.assert_allclose(dh, th, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(dg, tg, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(B.layer_scale_residual_fwd(x, h, gamma), x + gamma[None, :, None, None] * h)
