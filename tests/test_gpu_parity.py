"""GPU parity of every ABI call against the CPU oracle (needs an MI355X).

Each case runs shards of a layer through halo_gather -> conv_fwd ->
halo_gather(grad) -> conv_bwd_input -> conv_bwd_weight_partial (and the fused
conv_bwd) -> partial_reduce, then compares with the oracle computed on the
GLOBAL tensors:

* halos bit-exact against the neighbours' edge columns (zeros at the edges);
* forward / grad_input within 1e-5 and grad_weight / grad_bias within 1e-4,
  normwise (max abs error / max abs reference);
* the Shard(3) and _Partial invariants: concatenated shard outputs are the
  unsharded result, reduced partials are the full gradients.

Small cases span several kernel tiles with ragged tails; the workloads of
the pages' shapes run at full size, with the oracle either on the whole shard
(depthwise) or on sampled elements plus exact identities (dense 256->256).
"""
import numpy as np
import pytest
import torch

import oracle
from shard_harness import (TOL_DX, TOL_FWD, TOL_GW, assert_close, host, run_shard, slices,
                           to_dev)
from spatially_sharded_cnn_amd import sscnn, workloads

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


# (name, n, ci, co, h, W global, k, stride, pad, groups, S)
SMALL = [
    ("dw7_ragged", 2, 37, 37, 45, 4 * 50, 7, 1, 3, 37, 4),
    ("dw7_single_shard", 1, 16, 16, 20, 64, 7, 1, 3, 16, 1),
    ("dw3_two_shards", 2, 10, 10, 7, 2 * 9, 3, 1, 1, 10, 2),
    ("dw7_coltiles_raggedrows", 2, 19, 19, 45, 3 * 128, 7, 1, 3, 19, 3),
    ("dw7_h130", 1, 6, 6, 130, 2 * 64, 7, 1, 3, 6, 2),
    ("dw5_w32", 1, 8, 8, 70, 2 * 32, 5, 1, 2, 8, 2),
    ("dw3_w16", 2, 5, 5, 17, 4 * 16, 3, 1, 1, 5, 4),
    ("dw7_w48", 1, 7, 7, 33, 3 * 48, 7, 1, 3, 7, 3),
    ("dw7_w256", 1, 4, 4, 20, 2 * 256, 7, 1, 3, 4, 2),
    ("dw7_h16_w16", 2, 24, 24, 16, 4 * 16, 7, 1, 3, 24, 4),
    ("dw7_h16_w32", 2, 12, 12, 16, 3 * 32, 7, 1, 3, 12, 3),
    ("dw5_h20_w16", 1, 9, 9, 20, 2 * 16, 5, 1, 2, 9, 2),
    # 32-wide slices 16..63 rows high (two rows per thread in 32- and 16-row tiles), with a
    # last row tile moved up over its neighbour: rows 45 = 32 + 13, 20 = 16 + 4, 33 = 32 + 1
    ("dw7_w32_h45", 2, 11, 11, 45, 3 * 32, 7, 1, 3, 11, 3),
    ("dw5_w32_h20", 1, 9, 9, 20, 2 * 32, 5, 1, 2, 9, 2),
    ("dw3_w32_h33", 2, 6, 6, 33, 2 * 32, 3, 1, 1, 6, 2),
    # widths that are multiples of 64 (the register-window kernels): k = 3, a slice
    # of three 64-column blocks with a ragged strip group, a plane under one strip
    ("dw3_w64", 2, 6, 6, 23, 2 * 64, 3, 1, 1, 6, 2),
    ("dw5_w192_h70", 1, 5, 5, 70, 2 * 192, 5, 1, 2, 5, 2),
    ("dw7_h5_w64", 1, 3, 3, 5, 3 * 64, 7, 1, 3, 3, 3),
    # 1x1 convolutions (the ConvNeXt block's expansion and projection) on the matrix cores
    ("pw1x1_expand", 2, 32, 128, 12, 2 * 64, 1, 1, 0, 1, 2),
    ("pw1x1_project", 1, 128, 32, 9, 4 * 16, 1, 1, 0, 1, 4),
    ("dense5x5_ragged", 2, 40, 72, 13, 3 * 37, 5, 1, 2, 1, 3),
    ("mfma5x5_ragged_channels", 2, 44, 72, 13, 3 * 36, 5, 1, 2, 1, 3),
    ("mfma5x5_two_segments", 1, 16, 20, 6, 2 * 132, 5, 1, 2, 1, 2),
    ("mfma3x3_c96_c128", 1, 96, 128, 9, 2 * 64, 3, 1, 1, 1, 2),
    ("dense5x5_tiles", 1, 64, 64, 20, 2 * 96, 5, 1, 2, 1, 2),
    ("dense3x3", 2, 24, 40, 9, 2 * 30, 3, 1, 1, 1, 2),
    ("stem4x4s4", 2, 3, 64, 32, 4 * 64, 4, 4, 0, 1, 4),
    ("ds2x2s2", 2, 64, 96, 16, 4 * 32, 2, 2, 0, 1, 4),
    # patchify on the matrix cores: ragged row / column tiles, 80 pixels, k = 4 with a long reduction
    ("patch2_c80_p80", 3, 48, 80, 10, 2 * 32, 2, 2, 0, 1, 2),
    ("patch4_c48_k512", 2, 32, 48, 16, 4 * 64, 4, 4, 0, 1, 4),
    ("patch2_c256_tiles", 2, 256, 256, 32, 2 * 128, 2, 2, 0, 1, 2),
    ("patch2_wo8_direct", 1, 16, 32, 8, 2 * 16, 2, 2, 0, 1, 2),
    # ci * k * k <= 64: the 64-wide K tile of grad_input / grad_weight (K = 64 and 32; co not a multiple of 128)
    ("patch2_k64_narrow", 2, 16, 48, 32, 2 * 64, 2, 2, 0, 1, 2),
    ("patch2_k32_narrow", 1, 8, 160, 16, 2 * 32, 2, 2, 0, 1, 2),
    # enough 128 x 128 forward tiles (512) for the 128-row forward tile
    ("patch2_wide_fwd", 2, 16, 128, 256, 2 * 512, 2, 2, 0, 1, 2),
    ("grouped3x3", 1, 8, 12, 10, 3 * 12, 3, 1, 1, 4, 3),
    ("strided3x3p1", 1, 6, 10, 11, 2 * 16, 3, 2, 1, 1, 2),
]


def _custom(case, seed):
    name, n, ci, co, h, w, k, s, p, g, S = case
    ho, wo = (h + 2 * p - k) // s + 1, (w + 2 * p - k) // s + 1
    return workloads.custom(name, n, ci, co, h, w, k, s, p, g, ho, wo, S, seed=seed)


def _check_all_shards(wl, tensors, shards=None):
    """Run every shard, compare each with the oracle, then check the
    invariants.  Returns per-shard results (device tensors)."""
    L = wl.layers[0]
    S = wl.num_shards
    x, wt, b, g = tensors.x, tensors.weights[0], tensors.biases[0], tensors.g
    x_sl, g_sl = slices(x, S), slices(g, S)
    wt_d, b_d = to_dev(wt), to_dev(b)
    wl_in, wol = L.in_shape[3] // S, L.out_shape[3] // S
    outs = []
    shards = range(S) if shards is None else shards
    for s in shards:
        _say(f"  {wl.name}: shard {s}/{S} in={L.in_shape} k={L.k} s={L.stride} p={L.pad} g={L.groups}")
        r = run_shard(L, S, s, x_sl, g_sl, wt_d, b_d)
        torch.cuda.synchronize()
        c = r["conv"]
        # halos: a copy, so bit-exact
        np.testing.assert_array_equal(host(r["x_halo"]), oracle.halo_columns(x, S, s, c.halo_l, c.halo_r))
        np.testing.assert_array_equal(host(r["g_halo"]), oracle.halo_columns(g, S, s, c.ghalo_l, c.ghalo_r))
        cols_o, cols_i = (s * wol, (s + 1) * wol), (s * wl_in, (s + 1) * wl_in)
        assert_close(host(r["y"]), oracle.conv_fwd(x, wt, b, L.stride, L.pad, L.groups, cols=cols_o),
                     TOL_FWD, f"{wl.name} shard {s} forward")
        assert_close(host(r["dx"]), oracle.conv_bwd_input(g, wt, x.shape, L.stride, L.pad, L.groups,
                                                          cols=cols_i), TOL_DX, f"{wl.name} shard {s} grad_input")
        gw_ref, gb_ref = oracle.conv_bwd_weight(x, g, L.k, L.stride, L.pad, L.groups, cols=cols_o)
        assert_close(host(r["gw"]), gw_ref, TOL_GW, f"{wl.name} shard {s} grad_weight partial")
        assert_close(host(r["gb"]), gb_ref, TOL_GW, f"{wl.name} shard {s} grad_bias partial")
        # the fused backward: the same grad_input bit for bit, the partials to tolerance
        assert torch.equal(r["dx2"], r["dx"]), f"{wl.name} shard {s}: conv_bwd grad_input != conv_bwd_input"
        assert_close(host(r["gw2"]), gw_ref, TOL_GW, f"{wl.name} shard {s} conv_bwd grad_weight partial")
        assert_close(host(r["gb2"]), gb_ref, TOL_GW, f"{wl.name} shard {s} conv_bwd grad_bias partial")
        outs.append(r)
    return outs


def _check_invariants(wl, tensors, outs):
    L = wl.layers[0]
    x, wt, b, g = tensors.x, tensors.weights[0], tensors.biases[0], tensors.g
    y_cat = np.concatenate([host(r["y"]) for r in outs], axis=3)
    assert_close(y_cat, oracle.conv_fwd(x, wt, b, L.stride, L.pad, L.groups), TOL_FWD,
                 f"{wl.name}: concatenated shard outputs vs unsharded forward")
    dx_cat = np.concatenate([host(r["dx"]) for r in outs], axis=3)
    assert_close(dx_cat, oracle.conv_bwd_input(g, wt, x.shape, L.stride, L.pad, L.groups), TOL_DX,
                 f"{wl.name}: concatenated grad_input vs unsharded")
    gw_full, gb_full = oracle.conv_bwd_weight(x, g, L.k, L.stride, L.pad, L.groups)
    gw_red = torch.empty_like(outs[0]["gw"])
    gb_red = torch.empty_like(outs[0]["gb"])
    _say(f"  {wl.name}: partial_reduce over {len(outs)} shards")
    sscnn.partial_reduce([r["gw"] for r in outs], gw_red)
    sscnn.partial_reduce([r["gb"] for r in outs], gb_red)
    torch.cuda.synchronize()
    assert_close(host(gw_red), gw_full, TOL_GW, f"{wl.name}: reduced grad_weight vs full")
    assert_close(host(gb_red), gb_full, TOL_GW, f"{wl.name}: reduced grad_bias vs full")
    # the reduction is a left-to-right float32 sum: bit-exact against numpy doing the same
    acc = host(outs[0]["gw"]).copy()
    for r in outs[1:]:
        acc = acc + host(r["gw"])
    np.testing.assert_array_equal(host(gw_red), acc)


def test_dense5x5_tiny_all_shards():
    """The 3->8 5x5 case on (1,3,32,64), four 16-wide slices."""
    wl = workloads.WORKLOADS["dense5x5_tiny"]
    t = workloads.generate(wl)
    outs = _check_all_shards(wl, t)
    _check_invariants(wl, t, outs)


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_layer_all_shards(case):
    wl = _custom(case, seed=100 + SMALL.index(case))
    t = workloads.generate(wl)
    outs = _check_all_shards(wl, t)
    _check_invariants(wl, t, outs)


def test_dw7_c256_full_shard():
    """Depthwise 7x7 C=256: shard 1 of (7,256,128,256), whole shard vs oracle;
    the four partials reduce to the full grad_weight."""
    wl = workloads.WORKLOADS["dw7_c256"]
    t = workloads.generate(wl)
    outs = _check_all_shards(wl, t, shards=[wl.shard])
    r = outs[0]
    L = wl.layers[0]
    S = wl.num_shards
    x_sl, g_sl = slices(t.x, S), slices(t.g, S)
    wt_d, b_d = to_dev(t.weights[0]), to_dev(t.biases[0])
    parts = []
    for s in range(S):
        _say(f"  dw7_c256: partial of shard {s}")
        parts.append(run_shard(L, S, s, x_sl, g_sl, wt_d, b_d)["gw"])
    red = torch.empty_like(parts[0])
    sscnn.partial_reduce(parts, red)
    torch.cuda.synchronize()
    gw_full, _ = oracle.conv_bwd_weight(t.x, t.g, L.k, L.stride, L.pad, L.groups)
    assert_close(host(red), gw_full, TOL_GW, "dw7_c256 reduced grad_weight")
    # bitwise reproducible
    r2 = run_shard(L, S, wl.shard, x_sl, g_sl, wt_d, b_d)
    torch.cuda.synchronize()
    for key in ("y", "dx", "gw", "gb", "dx2", "gw2", "gb2"):
        assert torch.equal(r[key], r2[key]), f"{key} differs between two identical runs"


@pytest.mark.timeout(900)
def test_dense5x5_c256_full_shard():
    """Dense 5x5 256->256: shard 1 of (7,256,128,512), full size, in the launch
    configuration the benchmark uses.  The whole shard -- forward, grad_input,
    grad_weight and grad_bias partials, from the separate calls and from the
    fused conv_bwd the benchmark times -- is compared element by element with
    the oracle (about 1.1 TFLOP of double loops on the host).  The bilinear
    identity <Y - b, G>_shard = <W, gW_shard> is checked as well."""
    import time
    wl = workloads.WORKLOADS["dense5x5_c256"]
    t = workloads.generate(wl)
    L = wl.layers[0]
    S, s = wl.num_shards, wl.shard
    x_sl, g_sl = slices(t.x, S), slices(t.g, S)
    wt_d, b_d = to_dev(t.weights[0]), to_dev(t.biases[0])
    _say(f"  dense5x5_c256: shard {s}/{S}")
    r = run_shard(L, S, s, x_sl, g_sl, wt_d, b_d)
    torch.cuda.synchronize()
    c = r["conv"]
    np.testing.assert_array_equal(host(r["x_halo"]), oracle.halo_columns(t.x, S, s, c.halo_l, c.halo_r))
    np.testing.assert_array_equal(host(r["g_halo"]), oracle.halo_columns(t.g, S, s, c.ghalo_l, c.ghalo_r))
    got = {k: host(r[k]) for k in ("y", "dx", "gw", "gb", "dx2", "gw2", "gb2")}
    del r, x_sl, g_sl
    torch.cuda.empty_cache()
    wol, wli = c.w_out_local, c.w_local
    t0 = time.perf_counter()
    y_ref = oracle.conv_fwd(t.x, t.weights[0], t.biases[0], L.stride, L.pad, L.groups, cols=(s * wol, (s + 1) * wol))
    _say(f"  oracle forward {time.perf_counter() - t0:.1f} s")
    dx_ref = oracle.conv_bwd_input(t.g, t.weights[0], t.x.shape, L.stride, L.pad, L.groups,
                                   cols=(s * wli, (s + 1) * wli))
    _say(f"  oracle grad_input {time.perf_counter() - t0:.1f} s")
    gw_ref, gb_ref = oracle.conv_bwd_weight(t.x, t.g, L.k, L.stride, L.pad, L.groups, cols=(s * wol, (s + 1) * wol))
    _say(f"  oracle grad_weight {time.perf_counter() - t0:.1f} s")
    e = {}
    e["forward"] = assert_close(got["y"], y_ref, TOL_FWD, "dense5x5_c256 forward")
    e["grad_input"] = assert_close(got["dx"], dx_ref, TOL_DX, "dense5x5_c256 grad_input")
    e["grad_weight"] = assert_close(got["gw"], gw_ref, TOL_GW, "dense5x5_c256 grad_weight partial")
    e["grad_bias"] = assert_close(got["gb"], gb_ref, TOL_GW, "dense5x5_c256 grad_bias partial")
    e["fused grad_input"] = assert_close(got["dx2"], dx_ref, TOL_DX, "dense5x5_c256 fused conv_bwd grad_input")
    e["fused grad_weight"] = assert_close(got["gw2"], gw_ref, TOL_GW, "dense5x5_c256 fused conv_bwd grad_weight")
    e["fused grad_bias"] = assert_close(got["gb2"], gb_ref, TOL_GW, "dense5x5_c256 fused conv_bwd grad_bias")
    _say("  dense5x5_c256 normwise errors: " + ", ".join(f"{k} {v:.2e}" for k, v in e.items()))
    # <Y - b, G_s> over the shard equals <W, gW_s> (exact in exact arithmetic)
    gs = oracle.shard_columns(t.g, S, s).astype(np.float64)
    y, gw = got["y"], got["gw"]
    lhs = float(np.sum((y.astype(np.float64) - t.biases[0].astype(np.float64)[None, :, None, None]) * gs))
    rhs = float(np.sum(t.weights[0].astype(np.float64) * gw.astype(np.float64)))
    scale = float(np.sum(np.abs(t.weights[0].astype(np.float64) * gw)))
    assert abs(lhs - rhs) <= 1e-5 * scale, (lhs, rhs, scale)
