"""GPU parity of height sharding, Shard(2) (needs an MI355X).

The pages switch the sharded dimension to H for very high resolutions
(kwkr.cn retelling, section 5.2).  Each case runs every H-shard of a layer
through row_halo_gather -> hconv_fwd -> row_halo_gather(grad) -> hconv_bwd_input
-> hconv_bwd_weight_partial (and the fused hconv_bwd), and compares with the
oracle on the GLOBAL tensors:

* row halos bit-exact against the neighbours' edge rows (zeros at the top
  and bottom of the image);
* forward and grad_input within 1e-5, grad_weight / grad_bias within 1e-4
  (normwise), the partials being the gradients summed over the shard's own
  output rows;
* concatenated shard rows are the unsharded result, and the reduced partials
  are the full gradients.
"""
import numpy as np
import pytest
import torch

import oracle
from shard_harness import TOL_DX, TOL_FWD, TOL_GW, assert_close, host, to_dev
from spatially_sharded_cnn_amd import sscnn, workloads

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


# (name, n, ci, co, H global, w, k, stride, pad, groups, S): one case per kernel family
CASES = [
    ("dw7", 2, 16, 16, 4 * 16, 64, 7, 1, 3, 16, 4),
    ("dw3", 1, 8, 8, 4 * 8, 48, 3, 1, 1, 8, 4),
    ("dw7_64rows", 1, 4, 4, 2 * 64, 128, 7, 1, 3, 4, 2),    # 64-row slices: 4 rows per thread, 2 column tiles
    ("dw5_w32_rows24", 1, 6, 6, 2 * 24, 32, 5, 1, 2, 6, 2),   # 32 wide: 16-row tiles, the last moved up
    ("dw7_w32_rows40", 1, 5, 5, 2 * 40, 32, 7, 1, 3, 5, 2),   # 32 wide: 32-row tiles, the last moved up
    ("dw5_w40_direct", 1, 6, 6, 3 * 10, 40, 5, 1, 2, 6, 3),
    ("mfma5x5", 1, 24, 32, 2 * 12, 64, 5, 1, 2, 1, 2),
    ("mfma3x3", 1, 16, 20, 3 * 8, 32, 3, 1, 1, 1, 3),
    ("mfma5x5_tiles_ragged", 2, 36, 68, 2 * 22, 100, 5, 1, 2, 1, 2),     # ragged row, column, channel tiles
    ("mfma5x5_c128", 2, 128, 128, 4 * 16, 128, 5, 1, 2, 1, 4),
    ("direct5x5_example", 1, 3, 8, 4 * 8, 64, 5, 1, 2, 1, 4),
    ("grouped3x3", 1, 8, 12, 3 * 10, 12, 3, 1, 1, 4, 3),
    ("strided3x3p1", 1, 6, 10, 2 * 16, 22, 3, 2, 1, 1, 2),
    ("patch2_no_halo", 2, 32, 48, 2 * 16, 64, 2, 2, 0, 1, 2),
]


def _row_slices(a, S):
    h = a.shape[2] // S
    return [to_dev(a[:, :, s * h:(s + 1) * h, :]) for s in range(S)]


def _run_hshard(L, S, s, x_sl, g_sl, wt_d, b_d):
    n, ci, H, w = L.in_shape
    c = sscnn.hconv_init(n, ci, L.co, H // S, w, L.k, L.stride, L.pad, L.groups, s, S)
    up = lambda sl: sl[s - 1] if s > 0 else None
    down = lambda sl: sl[s + 1] if s < S - 1 else None
    xh = torch.empty(c.halo_shape(sscnn.HALO_INPUT), device="cuda")
    gh = torch.empty(c.halo_shape(sscnn.HALO_GRAD_OUTPUT), device="cuda")
    y = torch.empty(c.y_shape, device="cuda")
    dx = torch.empty(c.x_shape, device="cuda")
    gw = torch.empty(c.w_shape, device="cuda")
    gb = torch.empty((c.c_out,), device="cuda")
    dx2, gw2, gb2 = torch.empty_like(dx), torch.empty_like(gw), torch.empty_like(gb)
    ws = sscnn.new_hworkspace(c)
    sscnn.row_halo_gather(c, sscnn.HALO_INPUT, up(x_sl), down(x_sl), xh)
    sscnn.hconv_fwd(c, x_sl[s], xh, wt_d, b_d, y)
    sscnn.row_halo_gather(c, sscnn.HALO_GRAD_OUTPUT, up(g_sl), down(g_sl), gh)
    sscnn.hconv_bwd_input(c, g_sl[s], gh, wt_d, dx)
    sscnn.hconv_bwd_weight_partial(c, x_sl[s], xh, g_sl[s], gw, gb, ws)
    sscnn.hconv_bwd(c, x_sl[s], xh, g_sl[s], gh, wt_d, dx2, gw2, gb2, ws)
    torch.cuda.synchronize()
    return dict(conv=c, xh=xh, gh=gh, y=y, dx=dx, gw=gw, gb=gb, dx2=dx2, gw2=gw2, gb2=gb2)


def _check(wl, t, shards):
    L = wl.layers[0]
    S = wl.num_shards
    x, wt, b, g = t.x, t.weights[0], t.biases[0], t.g
    x_sl, g_sl = _row_slices(x, S), _row_slices(g, S)
    wt_d, b_d = to_dev(wt), to_dev(b)
    hl, hol = L.in_shape[2] // S, L.out_shape[2] // S
    y_full = oracle.conv_fwd(x, wt, b, L.stride, L.pad, L.groups)
    dx_full = oracle.conv_bwd_input(g, wt, x.shape, L.stride, L.pad, L.groups)
    outs = []
    for s in shards:
        _say(f"  {wl.name}: H-shard {s}/{S} in={L.in_shape} k={L.k} s={L.stride} p={L.pad} g={L.groups}")
        r = _run_hshard(L, S, s, x_sl, g_sl, wt_d, b_d)
        c = r["conv"]
        np.testing.assert_array_equal(host(r["xh"]), oracle.halo_rows(x, S, s, c.halo_u, c.halo_d))
        np.testing.assert_array_equal(host(r["gh"]), oracle.halo_rows(g, S, s, c.ghalo_u, c.ghalo_d))
        rows = (s * hol, (s + 1) * hol)
        assert_close(host(r["y"]), y_full[:, :, rows[0]:rows[1]], TOL_FWD, f"{wl.name} H-shard {s} forward")
        assert_close(host(r["dx"]), dx_full[:, :, s * hl:(s + 1) * hl], TOL_DX, f"{wl.name} H-shard {s} grad_input")
        gw_ref, gb_ref = oracle.conv_bwd_weight_rows(x, g, L.k, L.stride, L.pad, L.groups, rows)
        assert_close(host(r["gw"]), gw_ref, TOL_GW, f"{wl.name} H-shard {s} grad_weight partial")
        assert_close(host(r["gb"]), gb_ref, TOL_GW, f"{wl.name} H-shard {s} grad_bias partial")
        assert torch.equal(r["dx2"], r["dx"]), f"{wl.name} H-shard {s}: hconv_bwd grad_input != hconv_bwd_input"
        assert_close(host(r["gw2"]), gw_ref, TOL_GW, f"{wl.name} H-shard {s} hconv_bwd grad_weight")
        assert_close(host(r["gb2"]), gb_ref, TOL_GW, f"{wl.name} H-shard {s} hconv_bwd grad_bias")
        outs.append(r)
    return outs


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_hshard_matches_oracle(case):
    name, n, ci, co, H, w, k, s, p, g, S = case
    ho, wo = (H + 2 * p - k) // s + 1, (w + 2 * p - k) // s + 1
    wl = workloads.custom(name, n, ci, co, H, w, k, s, p, g, ho, wo, S, seed=4300 + CASES.index(case))
    t = workloads.generate(wl)
    outs = _check(wl, t, range(S))
    L = wl.layers[0]
    # Shard(2) invariants: the shards' rows are the unsharded output and grad_input,
    # and their partials reduce to the full gradients
    assert_close(np.concatenate([host(r["y"]) for r in outs], axis=2),
                 oracle.conv_fwd(t.x, t.weights[0], t.biases[0], s, p, g), TOL_FWD, f"{name}: concatenated rows")
    assert_close(np.concatenate([host(r["dx"]) for r in outs], axis=2),
                 oracle.conv_bwd_input(t.g, t.weights[0], t.x.shape, s, p, g), TOL_DX, f"{name}: concatenated dx")
    red = torch.empty(outs[0]["gw"].numel() + co, device="cuda")
    sscnn.partial_reduce([torch.cat([r["gw"].flatten(), r["gb"]]) for r in outs], red)
    torch.cuda.synchronize()
    gw_full, gb_full = oracle.conv_bwd_weight(t.x, t.g, k, s, p, g)
    assert_close(host(red[:-co]).reshape(gw_full.shape), gw_full, TOL_GW, f"{name}: reduced grad_weight")
    assert_close(host(red[-co:]), gb_full, TOL_GW, f"{name}: reduced grad_bias")


def test_hshard_dw7_c256_full_shard():
    """The depthwise 7x7 C=256 map (7,256,128,256) split along H into four
    (7,256,32,256) slices: shard 1 in full against the oracle."""
    wl = workloads.WORKLOADS["dw7_c256_hshard"]
    t = workloads.generate(wl)
    _check(wl, t, [wl.shard])
