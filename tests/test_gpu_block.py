"""GPU parity of the ConvNeXt block over shards (needs an MI355X).

ShardedConvNeXtBlock runs the depthwise 7x7 convolution, LayerNorm over
channels, the two 1x1 convolutions, GELU, layer scale, DropPath and the
residual add on lists of W- (or H-) shards, all through the library.  The
reference is the same block in float64 on the CPU with plain torch ops
(conv2d, layer_norm, gelu) and torch autograd, given the DropPath factors of
the oracle's Philox4x32-10.  Forward within 1e-5 and every gradient (input,
each weight) within 1e-4, normwise: five float32 stages in a chain, and
weight gradients summed over every pixel.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

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


def _reference(x, P, scales, dim):
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in P.items()}
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    h = F.conv2d(xt, t["dwconv.weight"], t["dwconv.bias"], padding=3, groups=dim)
    h = F.layer_norm(h.permute(0, 2, 3, 1), (dim,), t["norm_weight"], t["norm_bias"], 1e-6).permute(0, 3, 1, 2)
    h = F.conv2d(h, t["pwconv1.weight"], t["pwconv1.bias"])
    h = F.gelu(h)
    h = F.conv2d(h, t["pwconv2.weight"], t["pwconv2.bias"])
    s = torch.ones(x.shape[0], dtype=torch.float64) if scales is None else torch.tensor(scales, dtype=torch.float64)
    out = xt + s[:, None, None, None] * (t["gamma"][None, :, None, None] * h)
    return out, xt, t


# (name, input shape, S, shard dim, drop_path)
CASES = [
    ("w_shards_droppath", (4, 32, 12, 4 * 16), 4, 3, 0.5),
    ("w_shards_no_droppath_tiled", (2, 16, 32, 2 * 64), 2, 3, 0.0),
    ("h_shards_droppath", (3, 24, 2 * 10, 16), 2, 2, 0.25),     # 24 channels: GELU as a pass of its own
    ("h_shards_fused_gelu", (2, 32, 2 * 8, 32), 2, 2, 0.25),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_block_matches_float64_reference(case):
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

    scales = B.droppath_scales(77, 0, shape[0], 1.0 - dp) if dp > 0 else None
    ref, xt, t = _reference(x, P, scales, dim)
    ref.backward(torch.tensor(gout, dtype=torch.float64))
    assert_close(host(sa.unshard(outs, dim=sdim)), ref.detach().numpy(), TOL_FWD, f"{name} output")
    assert_close(np.concatenate([host(v.grad) for v in xs], axis=sdim), xt.grad.numpy(), TOL_GW, f"{name} grad x")
    for pname, p in block.named_parameters():
        assert_close(host(p.grad), t[pname].grad.numpy(), TOL_GW, f"{name} grad {pname}")


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
