"""GPU parity of the ConvNeXt block over shards (needs an MI355X).

ShardedConvNeXtBlock runs the depthwise 7x7 convolution, LayerNorm over
channels, the two 1x1 convolutions, GELU, layer scale, DropPath and the
residual add on lists of W- (or H-) shards, all through the library.  The
reference is the same block in float64 on the CPU built from the oracle's
pinned definitions alone: ``oracle.conv_*`` for the depthwise convolution,
the matrix-product form ``oracle.patchify_*`` for the 1x1 convolutions, and
``oracle.blockops`` for LayerNorm, GELU, layer scale with the DropPath
factors of its Philox4x32-10, and the residual; the backward chains their
gradients by hand.  Forward within 1e-5 and every gradient (input, each
weight) within 1e-4, normwise: five float32 stages in a chain, and weight
gradients summed over every pixel.  One case runs at C = 256 on the
(7,256,128,256) map split into four (7,256,128,64) shards.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import blockops as B
from shard_harness import TOL_FWD, TOL_GW, assert_close, host, to_dev
from spatially_sharded_cnn_amd import autograd as sa

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _init(block, rng):
    """Random parameters of a visible size (layer scale O(1) so the branch matters)."""
    vals = {}
    with torch.no_grad():
        for name, p in block.named_parameters():
            scale = 0.3 if "weight" in name and p.dim() == 4 else 0.5
            shift = 1.0 if name in ("norm_weight", "gamma") else 0.0
            v = (rng.standard_normal(tuple(p.shape)) * scale + shift).astype(np.float32)
            p.copy_(to_dev(v))
            vals[name] = v
    return vals


def _oracle_block(x, P, scales, dim, gout):
    """Forward and backward of the block from the oracle's definitions:
    returns (out, grad of x, {parameter name: grad})."""
    eps = 1e-6
    h1 = oracle.conv_fwd(x, P["dwconv.weight"], P["dwconv.bias"], 1, 3, dim)
    h2, _, _ = B.layernorm_channels_fwd(h1, P["norm_weight"], P["norm_bias"], eps)
    h3 = oracle.patchify_fwd(h2, P["pwconv1.weight"], P["pwconv1.bias"], 1)
    h4 = B.gelu_fwd(h3)
    h5 = oracle.patchify_fwd(h4, P["pwconv2.weight"], P["pwconv2.bias"], 1)
    out = B.layer_scale_residual_fwd(x, h5, P["gamma"], scales)
    g = {}
    dh5, g["gamma"] = B.layer_scale_residual_bwd(h5, gout, P["gamma"], scales)
    g["pwconv2.weight"], g["pwconv2.bias"] = oracle.patchify_bwd_weight(h4, dh5, 1)
    dh4 = oracle.patchify_bwd_input(dh5, P["pwconv2.weight"], h4.shape, 1)
    del h4, h5, dh5
    dh3 = B.gelu_bwd(h3, dh4)
    del h3, dh4
    g["pwconv1.weight"], g["pwconv1.bias"] = oracle.patchify_bwd_weight(h2, dh3, 1)
    dh2 = oracle.patchify_bwd_input(dh3, P["pwconv1.weight"], h2.shape, 1)
    del dh3
    dh1, g["norm_weight"], g["norm_bias"] = B.layernorm_channels_bwd(h1, dh2, P["norm_weight"], eps)
    g["dwconv.weight"], g["dwconv.bias"] = oracle.conv_bwd_weight(x, dh1, 7, 1, 3, dim)
    dx = np.asarray(gout, dtype=np.float64) + oracle.conv_bwd_input(dh1, P["dwconv.weight"], x.shape, 1, 3, dim)
    return out, dx, g


# (name, input shape, S, shard dim, drop_path)
CASES = [
    ("w_shards_droppath", (4, 32, 12, 4 * 16), 4, 3, 0.5),
    ("w_shards_no_droppath_tiled", (2, 16, 32, 2 * 64), 2, 3, 0.0),
    ("h_shards_droppath", (3, 24, 2 * 10, 16), 2, 2, 0.25),     # 24 channels: GELU as a pass of its own
    ("h_shards_fused_gelu", (2, 32, 2 * 8, 32), 2, 2, 0.25),
    ("w_shards_c256_full_shard", (7, 256, 128, 4 * 64), 4, 3, 0.1),   # the (7,256,128,64) shard of the block bench
]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_block_matches_oracle(case):
    name, shape, S, sdim, dp = case
    _say(f"  block {name}: input {shape}, {S} shards along dim {sdim}, drop_path {dp}")
    dim = shape[1]
    rng = np.random.default_rng(3100 + CASES.index(case))
    block = sa.ShardedConvNeXtBlock(dim, drop_path=dp, seed=77, shard_dim=sdim)
    block.train()
    P = _init(block, rng)
    x = rng.standard_normal(shape).astype(np.float32)
    gout = rng.standard_normal(shape).astype(np.float32)
    xs = [t.requires_grad_() for t in sa.shard(to_dev(x), S, dim=sdim)]
    outs = block(xs)
    sum((o * g).sum() for o, g in zip(outs, sa.shard(to_dev(gout), S, dim=sdim))).backward()
    torch.cuda.synchronize()
    assert block.calls == (1 if dp > 0 else 0)

    got_out = host(sa.unshard(outs, dim=sdim))
    got_dx = np.concatenate([host(v.grad) for v in xs], axis=sdim)
    got_g = {pname: host(p.grad) for pname, p in block.named_parameters()}
    del outs, xs
    torch.cuda.empty_cache()
    scales = B.droppath_scales(77, 0, shape[0], 1.0 - dp) if dp > 0 else None
    ref, ref_dx, ref_g = _oracle_block(x, P, scales, dim, gout)
    assert_close(got_out, ref, TOL_FWD, f"{name} output")
    assert_close(got_dx, ref_dx, TOL_GW, f"{name} grad x")
    for pname, gv in got_g.items():
        assert_close(gv, ref_g[pname].reshape(gv.shape), TOL_GW, f"{name} grad {pname}")


def test_block_droppath_counter_and_eval():
    """Each training call draws new factors (the counter advances); eval mode
    and drop_path 0 skip DropPath."""
    dim, shape = 8, (16, 8, 4, 64)
    block = sa.ShardedConvNeXtBlock(dim, drop_path=0.5, seed=5)
    _init(block, np.random.default_rng(3200))
    x = to_dev(np.random.default_rng(3201).standard_normal(shape).astype(np.float32))
    xs = sa.shard(x, 1)
    with torch.no_grad():
        a = sa.unshard(block(xs))
        b = sa.unshard(block(xs))
        block.eval()
        c = sa.unshard(block(xs))
    torch.cuda.synchronize()
    assert block.calls == 2
    kept = lambda out: [bool((out[i] != x[i]).any()) for i in range(shape[0])]
    assert kept(a) != kept(b)                                 # different draws on the two calls
    assert kept(a) == [bool(v) for v in B.droppath_scales(5, 0, shape[0], 0.5)]
    assert all(kept(c))                                       # eval: every sample keeps its branch
