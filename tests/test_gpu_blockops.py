"""GPU parity of the ConvNeXt block's other steps (needs an MI355X).

LayerNorm over channels, GELU, layer scale with DropPath and the residual add,
and the DropPath factors, each through the C ABI on seeded inputs, against the
float64 oracle in oracle/blockops.py:
* outputs and grad_inputs within 1e-5, weight gradients within 1e-4
  (normwise, relative to max |ref|);
* DropPath factors bit-exact (an integer decision on a Philox word, then
  1/keep in float32 on both sides);
* the shard invariants: the ops on W-shards concatenate to the op on the
  whole tensor, and the shards' partial weight gradients sum to the whole one.
"""
import numpy as np
import pytest
import torch

from oracle import blockops as B
from shard_harness import TOL_DX, TOL_FWD, TOL_GW, assert_close, host, to_dev
from spatially_sharded_cnn_amd import sscnn

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _rand(shape, seed, scale=1.0, shift=0.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale + shift).astype(np.float32)


# (name, (n, c, h, w)): the c2 block's shard shape, a ragged one, a single channel, a single pixel row,
# and channel counts that reach each register-held kernel (up to 1024 forward, 512 backward) and the
# loop kernels beyond them, full and ragged
LN_SHAPES = [("c256_shard", (2, 256, 16, 64)), ("ragged", (3, 37, 5, 7)), ("one_channel", (2, 1, 4, 4)),
             ("wide_c", (1, 1024, 2, 8)), ("c100_ragged", (2, 100, 3, 5)), ("c512", (1, 512, 3, 8)),
             ("c768", (1, 768, 2, 5)), ("c2048", (1, 2048, 2, 4)), ("c1100_ragged", (1, 1100, 1, 7))]


def _ln(x, gamma, beta, eps=1e-6):
    n, c, h, w = x.shape
    y = torch.empty_like(x)
    mean = torch.empty((n, h, w), device="cuda")
    rstd = torch.empty((n, h, w), device="cuda")
    sscnn.layernorm_fwd(x, gamma, beta, y, mean, rstd, eps)
    return y, mean, rstd


@pytest.mark.parametrize("case", LN_SHAPES, ids=[c[0] for c in LN_SHAPES])
def test_layernorm_matches_oracle(case):
    name, shape = case
    _say(f"  layernorm {name} {shape}")
    x, dy = _rand(shape, 1, 2.0, 0.3), _rand(shape, 2)
    gamma, beta = _rand(shape[1], 3, 0.5, 1.0), _rand(shape[1], 4, 0.1)
    xd, dyd, gd, bd = to_dev(x), to_dev(dy), to_dev(gamma), to_dev(beta)
    y, mean, rstd = _ln(xd, gd, bd)
    dx = torch.empty_like(xd)
    dg = torch.empty(shape[1], device="cuda")
    db = torch.empty(shape[1], device="cuda")
    sscnn.layernorm_bwd(xd, dyd, gd, mean, rstd, dx, dg, db)
    torch.cuda.synchronize()
    y_ref, mean_ref, rstd_ref = B.layernorm_channels_fwd(x, gamma, beta, 1e-6)
    assert_close(host(y), y_ref, TOL_FWD, f"{name} y")
    assert_close(host(mean), mean_ref, TOL_FWD, f"{name} mean")
    assert_close(host(rstd), rstd_ref, TOL_FWD, f"{name} rstd")
    dx_ref, dg_ref, db_ref = B.layernorm_channels_bwd(x, dy, gamma, 1e-6)
    assert_close(host(dx), dx_ref, TOL_DX, f"{name} dx")
    assert_close(host(dg), dg_ref, TOL_GW, f"{name} dgamma")
    assert_close(host(db), db_ref, TOL_GW, f"{name} dbeta")
    # the optional outputs are independent: dx alone, the parameter gradients alone
    dx2 = torch.empty_like(xd)
    sscnn.layernorm_bwd(xd, dyd, gd, mean, rstd, dx2, None, None)
    dg2 = torch.empty_like(dg)
    sscnn.layernorm_bwd(xd, dyd, gd, mean, rstd, None, dg2, None)
    torch.cuda.synchronize()
    assert torch.equal(dx2, dx) and torch.equal(dg2, dg)


def test_layernorm_shards_compose():
    """Per-pixel ops need no halo: W-shards give the whole tensor's result, and
    the shards' partial dgamma / dbeta sum to the whole ones."""
    S, shape = 4, (2, 64, 8, 4 * 16)
    x, dy = _rand(shape, 5), _rand(shape, 6)
    gamma, beta = _rand(64, 7, 0.5, 1.0), _rand(64, 8, 0.1)
    gd, bd = to_dev(gamma), to_dev(beta)
    ys, parts = [], []
    for s in range(S):
        xs, dys = to_dev(x[..., s * 16:(s + 1) * 16]), to_dev(dy[..., s * 16:(s + 1) * 16])
        y, mean, rstd = _ln(xs, gd, bd)
        part = torch.empty(128, device="cuda")
        sscnn.layernorm_bwd(xs, dys, gd, mean, rstd, None, part[:64], part[64:])
        ys.append(y)
        parts.append(part)
    red = torch.empty(128, device="cuda")
    sscnn.partial_reduce(parts, red)
    torch.cuda.synchronize()
    assert_close(np.concatenate([host(t) for t in ys], axis=3), B.layernorm_channels_fwd(x, gamma, beta, 1e-6)[0],
                 TOL_FWD, "concatenated shards")
    _, dg_ref, db_ref = B.layernorm_channels_bwd(x, dy, gamma, 1e-6)
    assert_close(host(red[:64]), dg_ref, TOL_GW, "reduced dgamma")
    assert_close(host(red[64:]), db_ref, TOL_GW, "reduced dbeta")


@pytest.mark.parametrize("count", [4 * 16384, 1001, 3, 1])
def test_gelu_matches_oracle(count):
    _say(f"  gelu count={count}")
    x = _rand(count, 9, 3.0)
    x[:min(count, 3)] = [0.0, -12.0, 9.5][:min(count, 3)]
    dy = _rand(count, 10)
    xd = to_dev(x)
    y, dx = torch.empty_like(xd), torch.empty_like(xd)
    sscnn.gelu_fwd(xd, y)
    sscnn.gelu_bwd(xd, to_dev(dy), dx)
    torch.cuda.synchronize()
    assert_close(host(y), B.gelu_fwd(x), TOL_FWD, "gelu")
    assert_close(host(dx), B.gelu_bwd(x, dy), TOL_DX, "gelu grad")


@pytest.mark.parametrize("seed,offset,n,keep", [(1234, 7, 4096, 0.75), (2 ** 40 + 3, 2 ** 33 + 5, 97, 0.9),
                                                (0, 0, 8, 0.5), (5, 1, 33, 1.0), (9, 2, 64, 1e-3)])
def test_droppath_scales_bit_exact(seed, offset, n, keep):
    s = torch.empty(n, device="cuda")
    sscnn.droppath_scales(seed, offset, keep, s)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(s), B.droppath_scales(seed, offset, n, keep))


@pytest.mark.parametrize("with_scales", [True, False])
def test_layer_scale_residual_matches_oracle(with_scales):
    shape = (4, 48, 6, 10)
    x, h, dout = _rand(shape, 11), _rand(shape, 12), _rand(shape, 13)
    gamma = _rand(48, 14, 1e-2)
    scales = np.array([1.25, 0.0, 1.25, 1.25], np.float32) if with_scales else None
    sd = to_dev(scales) if with_scales else None
    xd, hd, dod, gd = to_dev(x), to_dev(h), to_dev(dout), to_dev(gamma)
    out, dh = torch.empty_like(xd), torch.empty_like(xd)
    dg = torch.empty(48, device="cuda")
    sscnn.layer_scale_residual_fwd(xd, hd, gd, sd, out)
    sscnn.layer_scale_residual_bwd(hd, dod, gd, sd, dh, dg)
    torch.cuda.synchronize()
    assert_close(host(out), B.layer_scale_residual_fwd(x, h, gamma, scales), TOL_FWD, "out")
    dh_ref, dg_ref = B.layer_scale_residual_bwd(h, dout, gamma, scales)
    assert_close(host(dh), dh_ref, TOL_DX, "dh")
    assert_close(host(dg), dg_ref, TOL_GW, "dgamma")
    if with_scales:
        assert torch.equal(out[1], xd[1]) and not dh[1].any()      # the dropped sample


# (name, (n, c_in, c_out, h, w)): the block's expansion and projection on a c2-style shard slice, a
# ragged pixel count (h * w not a multiple of 128) and a one-image slice
PW_SHAPES = [("expand", (2, 64, 256, 8, 32)), ("project", (2, 256, 64, 8, 32)), ("ragged", (3, 32, 48, 5, 16)),
             ("one_image", (1, 16, 16, 3, 16))]


@pytest.mark.parametrize("case", PW_SHAPES, ids=[c[0] for c in PW_SHAPES])
def test_pointwise_gelu_matches_oracle(case):
    """The fused 1x1 + GELU forward and the fused projection grad_input times
    GELU'(pre), against the oracle's conv and GELU in float64, and bit for bit
    against the same steps as separate calls."""
    from oracle import conv_bwd_input, conv_fwd
    name, (n, ci, co, h, w) = case
    _say(f"  pointwise gelu {name} {(n, ci, co, h, w)}")
    x, g = _rand((n, ci, h, w), 21), _rand((n, co, h, w), 22)
    pre = _rand((n, ci, h, w), 23, 2.0)
    wt, b = _rand((co, ci, 1, 1), 24, 0.1), _rand(co, 25, 0.1)
    c = sscnn.conv_init(n, ci, co, h, w, 1, 1, 0, 1, 0, 1)
    xd, gd, pd, wd, bd = to_dev(x), to_dev(g), to_dev(pre), to_dev(wt), to_dev(b)
    y, ya = torch.empty(c.y_shape, device="cuda"), torch.empty(c.y_shape, device="cuda")
    dx = torch.empty(c.x_shape, device="cuda")
    sscnn.pointwise_gelu_fwd(c, xd, wd, bd, y, ya)
    sscnn.pointwise_bwd_input_gelu(c, gd, wd, pd, dx)
    # the unfused steps
    y2, ya2 = torch.empty_like(y), torch.empty_like(y)
    dxa, dx2 = torch.empty_like(dx), torch.empty_like(dx)
    sscnn.conv_fwd(c, xd, None, wd, bd, y2)
    sscnn.gelu_fwd(y2, ya2)
    sscnn.conv_bwd_input(c, gd, None, wd, dxa)
    sscnn.gelu_bwd(pd, dxa, dx2)
    torch.cuda.synchronize()
    y_ref = conv_fwd(x, wt, b, 1, 0, 1)
    assert_close(host(y), y_ref, TOL_FWD, f"{name} y")
    assert_close(host(ya), B.gelu_fwd(y_ref), TOL_FWD, f"{name} gelu(y)")
    assert_close(host(dx), B.gelu_bwd(pre, conv_bwd_input(g, wt, x.shape, 1, 0, 1)), TOL_DX, f"{name} dx")
    assert torch.equal(y, y2) and torch.equal(ya, ya2) and torch.equal(dx, dx2)
