"""GPU tests of the push form of the halo exchange (needs an MI355X).

A stem-like 4x4/4 layer and a 2x2/2 downsample, each followed by a
depthwise 7x7 layer, on four W-shards: every shard's sscnn_conv_fwd_push
(sscnn_conv_bwd_push) writes its edge columns into its neighbours' halo
buffers for the next (previous) layer.  After all shards ran, each shard's
halo must equal, bit for bit, what sscnn_halo_gather writes from the
neighbours' slices (zeros at the global edges: the halo buffers start as NaN
so an unwritten element shows), and the convolution results must equal
sscnn_conv_fwd's / sscnn_conv_bwd's bit for bit.  The forward outputs are
also compared with the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from shard_harness import TOL_FWD, assert_close, host, slices, to_dev
from spatially_sharded_cnn_amd import sscnn

pytestmark = pytest.mark.gpu

S = 4
# (name, n, ci, co, h, w, k): the producer (k = stride, pad 0), followed by a depthwise 7x7 pad 3 on co channels
CASES = [
    ("stem4x4", 2, 3, 32, 64, 4 * 64, 4),
    ("down2x2", 2, 32, 48, 32, 4 * 64, 2),
    ("down2x2_w16", 1, 16, 32, 16, 4 * 32, 2),      # consumer slices 16 wide
    ("down2x2_w8_fallback", 1, 16, 32, 16, 4 * 16, 2),   # 8-column output slices: not on the matrix-core
                                                          # path, pushed by the edge-copy kernel after it
]


def _nan(shape):
    return torch.full(shape, float("nan"), device="cuda")


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_push_forward_and_backward_equal_gather(case):
    name, n, ci, co, h, w, k = case
    print(f"  push {name}: ({n},{ci},{h},{w}) k={k}, then dw7 on {co} channels", flush=True)
    rng = np.random.default_rng(4600 + CASES.index(case))
    x = rng.standard_normal((n, ci, h, w)).astype(np.float32)
    wt = (rng.standard_normal((co, ci, k, k)) * 0.1).astype(np.float32)
    b = (rng.standard_normal(co) * 0.1).astype(np.float32)
    ho, wo = h // k, w // k
    g = rng.standard_normal((n, co, ho, wo)).astype(np.float32)
    prod = [sscnn.conv_init(n, ci, co, h, w // S, k, k, 0, 1, s, S) for s in range(S)]
    cons = [sscnn.conv_init(n, co, co, ho, wo // S, 7, 1, 3, co, s, S) for s in range(S)]
    xs, gs = slices(x, S), slices(g, S)
    wd, bd = to_dev(wt), to_dev(b)
    nb = lambda lst, s: (lst[s - 1] if s > 0 else None, lst[s + 1] if s < S - 1 else None)

    # forward: push into the consumer's input halos
    xh = [_nan(c.halo_shape(sscnn.HALO_INPUT)) for c in cons]
    ys, ys_ref = [], []
    for s in range(S):
        y, y_ref = torch.empty(prod[s].y_shape, device="cuda"), torch.empty(prod[s].y_shape, device="cuda")
        p = sscnn.make_push(cons[s], sscnn.HALO_INPUT, *nb(xh, s), xh[s])
        sscnn.conv_fwd_push(prod[s], xs[s], None, wd, bd, y, p)
        sscnn.conv_fwd(prod[s], xs[s], None, wd, bd, y_ref)
        ys.append(y)
        ys_ref.append(y_ref)
    torch.cuda.synchronize()
    for s in range(S):
        assert torch.equal(ys[s], ys_ref[s]), f"{name} shard {s}: forward differs from conv_fwd"
        gathered = torch.empty(cons[s].halo_shape(sscnn.HALO_INPUT), device="cuda")
        sscnn.halo_gather(cons[s], sscnn.HALO_INPUT, *nb(ys, s), gathered)
        torch.cuda.synchronize()
        assert torch.equal(xh[s], gathered), f"{name} shard {s}: pushed input halo != gathered halo"
    y_full = oracle.conv_fwd(x, wt, b, k, 0, 1)
    assert_close(np.concatenate([host(t) for t in ys], axis=3), y_full, TOL_FWD, f"{name}: forward")

    # backward: push grad_x's edge columns into the grad_output halos of the layer below it --
    # here the producer's own input plays that layer's output (a dw7 on ci channels below it)
    below = [sscnn.conv_init(n, ci, ci, h, w // S, 7, 1, 3, ci, s, S) for s in range(S)]
    gh = [_nan(c.halo_shape(sscnn.HALO_GRAD_OUTPUT)) for c in below]
    outs = []
    for s in range(S):
        ws = sscnn.new_workspace(prod[s])
        dx, dx_ref = torch.empty(prod[s].x_shape, device="cuda"), torch.empty(prod[s].x_shape, device="cuda")
        gw, gw_ref = torch.empty(prod[s].w_shape, device="cuda"), torch.empty(prod[s].w_shape, device="cuda")
        gb, gb_ref = torch.empty(co, device="cuda"), torch.empty(co, device="cuda")
        p = sscnn.make_push(below[s], sscnn.HALO_GRAD_OUTPUT, *nb(gh, s), gh[s])
        sscnn.conv_bwd_push(prod[s], xs[s], None, gs[s], None, wd, dx, gw, gb, p, ws)
        sscnn.conv_bwd(prod[s], xs[s], None, gs[s], None, wd, dx_ref, gw_ref, gb_ref, ws)
        outs.append((dx, dx_ref, gw, gw_ref, gb, gb_ref))
    torch.cuda.synchronize()
    dxs = [o[0] for o in outs]
    for s, (dx, dx_ref, gw, gw_ref, gb, gb_ref) in enumerate(outs):
        assert torch.equal(dx, dx_ref) and torch.equal(gw, gw_ref) and torch.equal(gb, gb_ref), \
            f"{name} shard {s}: conv_bwd_push differs from conv_bwd"
        gathered = torch.empty(below[s].halo_shape(sscnn.HALO_GRAD_OUTPUT), device="cuda")
        sscnn.halo_gather(below[s], sscnn.HALO_GRAD_OUTPUT, *nb(dxs, s), gathered)
        torch.cuda.synchronize()
        assert torch.equal(gh[s], gathered), f"{name} shard {s}: pushed grad_output halo != gathered halo"
