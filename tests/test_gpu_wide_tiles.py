"""GPU parity of the wide-tile forward and grad_input, and of the LDS-direct
grad_weight, of 2x2/2 layers (needs an MI355X).

The forward and the grad_input of a k = s = 2 layer can run as one product
over the pixels of all the images, in tiles of 128 rows (output channels,
or K = (ci, kh, kw)) x 224 pixels that may straddle two images.  The library
picks them when the tile count is a whole multiple of the CU count (the
ConvNeXt-style stack's downsamples), and 128-pixel forward tiles where the
224-pixel ones would be fewer than the CUs; SSCNN_PATCH_FWD=wide / =wide4 /
SSCNN_PATCH_BWI=wide force them wherever they apply and =tiled switch them
off, so these cases
run both forms on shapes chosen for their edges: channel counts that are not
a multiple of 128 rows, pixel counts that are not a multiple of 224, tiles
that straddle images, a single image, and the push form of the halo
exchange.  Every shard's result is compared with the oracle (1e-5
normwise), the two forms with each other, and the pushed halos bit for bit
with sscnn_halo_gather of the results.  The grad_weight kernel
(SSCNN_PATCH_BWW=dma with per-split slabs, =dma1 with one split written
straight to grad_weight) is compared the same way, partials within 1e-4 of
the oracle's sums over the shard's own output columns.  The 4x4/4 stem's
forward kernel (weights in registers, persistent over 64-pixel tiles;
SSCNN_PATCH_STEM=tiled switches it off) is checked the same way, and the
stem's backward against the oracle on the same shapes.
"""
import numpy as np
import pytest
import torch

import oracle
from shard_harness import TOL_DX, TOL_FWD, TOL_GW, assert_close, host, slices, to_dev
from spatially_sharded_cnn_amd import sscnn

pytestmark = pytest.mark.gpu

# (name, n, ci, co, h, w, shards)
CASES = [
    ("co80_ragged_pixels", 3, 8, 80, 20, 2 * 32, 2),          # 160 pixels per image and shard: tiles straddle images
    ("co144_one_image", 1, 16, 144, 24, 4 * 32, 4),            # two channel tiles, the second 16 rows
    ("co256_ci64", 2, 64, 256, 28, 2 * 64, 2),                 # 16 reduction stages, 448 pixels per image
    ("co512_ci256_many_tiles", 7, 256, 512, 16, 4 * 64, 4),    # the stack's shape class, 7 images
    ("ci40_co32_ragged_k", 2, 40, 32, 12, 2 * 32, 2),          # K = 160 rows: a 32-row second K tile
    ("ci12_odd_stages", 2, 12, 64, 16, 2 * 32, 2),             # 3 reduction stages: the halves take 2 and 1
    ("ci4_one_stage", 1, 4, 32, 8, 2 * 32, 2),                 # 1 stage: the second half adds zeros
]


def _say(*a):
    print(*a, flush=True)


def _fwd(monkeypatch, mode, conv, x, wd, bd, push=None):
    monkeypatch.setenv("SSCNN_PATCH_FWD", mode)
    y = torch.empty(conv.y_shape, device="cuda")
    if push is None:
        sscnn.conv_fwd(conv, x, None, wd, bd, y)
    else:
        sscnn.conv_fwd_push(conv, x, None, wd, bd, y, push)
    return y


@pytest.mark.parametrize("halves", ["1", "0"], ids=["two_halves", "one_half"])
@pytest.mark.parametrize("wmode", ["wide", "wide4"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_wide_forward_matches_oracle_and_tiled(case, wmode, halves, monkeypatch):
    """The wide forward against the oracle and the tiled kernel, in both of its forms: the
    reduction in one 256-thread half (every stage in order) and split between two halves of a
    512-thread workgroup (even / odd stages, added at the end), which launches with no more
    tiles than CUs take."""
    name, n, ci, co, h, w, S = case
    monkeypatch.setenv("SSCNN_WIDE_HALVES", halves)
    _say(f"  wide fwd {name} ({wmode}, halves={halves}): ({n},{ci},{h},{w}) -> {co} channels, {S} shards")
    rng = np.random.default_rng(4700 + CASES.index(case))
    x = rng.standard_normal((n, ci, h, w)).astype(np.float32)
    wt = (rng.standard_normal((co, ci, 2, 2)) * 0.05).astype(np.float32)
    b = (rng.standard_normal(co) * 0.1).astype(np.float32)
    xs = slices(x, S)
    wd, bd = to_dev(wt), to_dev(b)
    convs = [sscnn.conv_init(n, ci, co, h, w // S, 2, 2, 0, 1, s, S) for s in range(S)]
    # the consumer of the outputs: a depthwise 7x7 pad 3, whose input halo the push form fills
    cons = [sscnn.conv_init(n, co, co, h // 2, w // 2 // S, 7, 1, 3, co, s, S) for s in range(S)]
    y_full = oracle.conv_fwd(x, wt, b, 2, 0, 1)
    wol = w // 2 // S
    ys_wide, halos = [], [torch.full(c.halo_shape(sscnn.HALO_INPUT), float("nan"), device="cuda") for c in cons]
    nb = lambda lst, s: (lst[s - 1] if s > 0 else None, lst[s + 1] if s < S - 1 else None)
    for s in range(S):
        y_wide = _fwd(monkeypatch, wmode, convs[s], xs[s], wd, bd)
        y_tiled = _fwd(monkeypatch, "tiled", convs[s], xs[s], wd, bd)
        p = sscnn.make_push(cons[s], sscnn.HALO_INPUT, *nb(halos, s), halos[s])
        y_push = _fwd(monkeypatch, wmode, convs[s], xs[s], wd, bd, push=p)
        torch.cuda.synchronize()
        ref = y_full[:, :, :, s * wol:(s + 1) * wol]
        assert_close(host(y_wide), ref, TOL_FWD, f"{name} shard {s}: wide forward vs oracle")
        assert_close(host(y_tiled), ref, TOL_FWD, f"{name} shard {s}: tiled forward vs oracle")
        assert_close(host(y_wide), host(y_tiled), TOL_FWD, f"{name} shard {s}: wide vs tiled")
        assert torch.equal(y_push, y_wide), f"{name} shard {s}: pushing changed the wide forward's output"
        ys_wide.append(y_wide)
    for s in range(S):
        gathered = torch.empty(cons[s].halo_shape(sscnn.HALO_INPUT), device="cuda")
        sscnn.halo_gather(cons[s], sscnn.HALO_INPUT, *nb(ys_wide, s), gathered)
        torch.cuda.synchronize()
        assert torch.equal(halos[s], gathered), f"{name} shard {s}: pushed halo != gathered halo"


def test_wide_forward_is_reproducible(monkeypatch):
    """Two runs of the wide forward give the same bits (fixed reduction order, no atomics)."""
    rng = np.random.default_rng(4750)
    n, ci, co, h, w = 2, 32, 128, 16, 128
    x = to_dev(rng.standard_normal((n, ci, h, w)).astype(np.float32))
    wd = to_dev((rng.standard_normal((co, ci, 2, 2)) * 0.05).astype(np.float32))
    bd = to_dev((rng.standard_normal(co) * 0.1).astype(np.float32))
    c = sscnn.conv_init(n, ci, co, h, w, 2, 2, 0, 1, 0, 1)
    a = _fwd(monkeypatch, "wide", c, x, wd, bd)
    b2 = _fwd(monkeypatch, "wide", c, x, wd, bd)
    torch.cuda.synchronize()
    assert torch.equal(a, b2)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_wide_grad_input_matches_oracle_and_tiled(case, monkeypatch):
    name, n, ci, co, h, w, S = case
    _say(f"  wide grad_input {name}: ({n},{ci},{h},{w}) <- {co} channels, {S} shards")
    rng = np.random.default_rng(4800 + CASES.index(case))
    x_shape = (n, ci, h, w)
    g = rng.standard_normal((n, co, h // 2, w // 2)).astype(np.float32)
    wt = (rng.standard_normal((co, ci, 2, 2)) * 0.05).astype(np.float32)
    gs = slices(g, S)
    wd = to_dev(wt)
    convs = [sscnn.conv_init(n, ci, co, h, w // S, 2, 2, 0, 1, s, S) for s in range(S)]
    # the layer below: a depthwise 7x7 pad 3 on ci channels, whose grad_output halo the push form fills
    below = [sscnn.conv_init(n, ci, ci, h, w // S, 7, 1, 3, ci, s, S) for s in range(S)]
    dx_full = oracle.conv_bwd_input(g, wt, x_shape, 2, 0, 1)
    wl = w // S
    x_dummy = [torch.zeros(c.x_shape, device="cuda") for c in convs]
    halos = [torch.full(c.halo_shape(sscnn.HALO_GRAD_OUTPUT), float("nan"), device="cuda") for c in below]
    nb = lambda lst, s: (lst[s - 1] if s > 0 else None, lst[s + 1] if s < S - 1 else None)
    dxs = []
    for s in range(S):
        c = convs[s]
        out = {}
        for mode in ("wide", "tiled"):
            monkeypatch.setenv("SSCNN_PATCH_BWI", mode)
            out[mode] = torch.empty(c.x_shape, device="cuda")
            sscnn.conv_bwd_input(c, gs[s], None, wd, out[mode])
        monkeypatch.setenv("SSCNN_PATCH_BWI", "wide")
        dx_push = torch.empty(c.x_shape, device="cuda")
        gw, gb = torch.empty(c.w_shape, device="cuda"), torch.empty(co, device="cuda")
        p = sscnn.make_push(below[s], sscnn.HALO_GRAD_OUTPUT, *nb(halos, s), halos[s])
        sscnn.conv_bwd_push(c, x_dummy[s], None, gs[s], None, wd, dx_push, gw, gb, p, sscnn.new_workspace(c))
        torch.cuda.synchronize()
        ref = dx_full[:, :, :, s * wl:(s + 1) * wl]
        assert_close(host(out["wide"]), ref, TOL_DX, f"{name} shard {s}: wide grad_input vs oracle")
        assert_close(host(out["tiled"]), ref, TOL_DX, f"{name} shard {s}: tiled grad_input vs oracle")
        assert torch.equal(dx_push, out["wide"]), f"{name} shard {s}: conv_bwd_push grad_input != wide conv_bwd_input"
        dxs.append(out["wide"])
    for s in range(S):
        gathered = torch.empty(below[s].halo_shape(sscnn.HALO_GRAD_OUTPUT), device="cuda")
        sscnn.halo_gather(below[s], sscnn.HALO_GRAD_OUTPUT, *nb(dxs, s), gathered)
        torch.cuda.synchronize()
        assert torch.equal(halos[s], gathered), f"{name} shard {s}: pushed grad_output halo != gathered halo"


@pytest.mark.parametrize("mode", ["dma", "dma1"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_dma_grad_weight_matches_oracle_and_tiled(case, mode, monkeypatch):
    name, n, ci, co, h, w, S = case
    _say(f"  grad_weight {mode} {name}: ({n},{ci},{h},{w}) x {co} channels, {S} shards")
    rng = np.random.default_rng(4900 + CASES.index(case))
    x = rng.standard_normal((n, ci, h, w)).astype(np.float32)
    g = rng.standard_normal((n, co, h // 2, w // 2)).astype(np.float32)
    wt = (rng.standard_normal((co, ci, 2, 2)) * 0.05).astype(np.float32)
    xs, gs = slices(x, S), slices(g, S)
    wd = to_dev(wt)
    wol = w // 2 // S
    for s in range(S):
        c = sscnn.conv_init(n, ci, co, h, w // S, 2, 2, 0, 1, s, S)
        gw_ref, gb_ref = oracle.conv_bwd_weight(x, g, 2, 2, 0, 1, cols=(s * wol, (s + 1) * wol))
        res = {}
        for m in (mode, "tiled"):
            monkeypatch.setenv("SSCNN_PATCH_BWW", m)
            ws = sscnn.new_workspace(c)
            gw, gb = torch.empty(c.w_shape, device="cuda"), torch.empty(co, device="cuda")
            sscnn.conv_bwd_weight_partial(c, xs[s], None, gs[s], gw, gb, ws)
            dx2 = torch.empty(c.x_shape, device="cuda")
            gw2, gb2 = torch.empty_like(gw), torch.empty_like(gb)
            sscnn.conv_bwd(c, xs[s], None, gs[s], None, wd, dx2, gw2, gb2, ws)
            # without grad_bias
            gw3 = torch.empty_like(gw)
            sscnn.conv_bwd_weight_partial(c, xs[s], None, gs[s], gw3, None, ws)
            torch.cuda.synchronize()
            res[m] = (gw, gb, gw2, gb2, gw3)
        gw, gb, gw2, gb2, gw3 = res[mode]
        assert_close(host(gw), gw_ref, TOL_GW, f"{name} shard {s}: {mode} grad_weight partial vs oracle")
        assert_close(host(gb), gb_ref, TOL_GW, f"{name} shard {s}: {mode} grad_bias partial vs oracle")
        assert torch.equal(gw2, gw) and torch.equal(gb2, gb), f"{name} shard {s}: conv_bwd partials != conv_bwd_weight_partial"
        assert torch.equal(gw3, gw), f"{name} shard {s}: grad_weight without grad_bias differs"
        assert_close(host(gw), host(res["tiled"][0]), TOL_GW, f"{name} shard {s}: {mode} vs tiled grad_weight")


# (name, n, co, h, w, shards): the 4x4/4 stem on 3 input channels
STEM_CASES = [
    ("stem_co256", 2, 256, 32, 4 * 128, 4),
    ("stem_co48_ragged_tiles", 3, 48, 24, 2 * 64, 2),     # 96 pixels per image: 64-pixel tiles straddle images
    ("stem_co96_one_row", 1, 96, 4, 4 * 64, 4),           # one output row per image
    ("stem_co40_one_group", 2, 40, 16, 2 * 64, 2),        # wave 1 stores one group of 8 channels
    ("stem_co20_other_path", 2, 20, 16, 2 * 64, 2),       # not a multiple of 8: the general kernels
]


@pytest.mark.parametrize("case", STEM_CASES, ids=[c[0] for c in STEM_CASES])
def test_stem_forward_matches_oracle_and_tiled(case, monkeypatch):
    name, n, co, h, w, S = case
    _say(f"  stem fwd {name}: ({n},3,{h},{w}) -> {co} channels, {S} shards")
    rng = np.random.default_rng(5000 + STEM_CASES.index(case))
    x = rng.standard_normal((n, 3, h, w)).astype(np.float32)
    wt = (rng.standard_normal((co, 3, 4, 4)) * 0.1).astype(np.float32)
    b = (rng.standard_normal(co) * 0.1).astype(np.float32)
    xs = slices(x, S)
    wd, bd = to_dev(wt), to_dev(b)
    convs = [sscnn.conv_init(n, 3, co, h, w // S, 4, 4, 0, 1, s, S) for s in range(S)]
    cons = [sscnn.conv_init(n, co, co, h // 4, w // 4 // S, 7, 1, 3, co, s, S) for s in range(S)]
    y_full = oracle.conv_fwd(x, wt, b, 4, 0, 1)
    wol = w // 4 // S
    halos = [torch.full(c.halo_shape(sscnn.HALO_INPUT), float("nan"), device="cuda") for c in cons]
    nb = lambda lst, s: (lst[s - 1] if s > 0 else None, lst[s + 1] if s < S - 1 else None)
    ys = []
    for s in range(S):
        monkeypatch.setenv("SSCNN_PATCH_STEM", "tiled")
        y_tiled = torch.empty(convs[s].y_shape, device="cuda")
        sscnn.conv_fwd(convs[s], xs[s], None, wd, bd, y_tiled)
        monkeypatch.delenv("SSCNN_PATCH_STEM")
        y = torch.empty(convs[s].y_shape, device="cuda")
        sscnn.conv_fwd(convs[s], xs[s], None, wd, bd, y)
        y_push = torch.empty(convs[s].y_shape, device="cuda")
        p = sscnn.make_push(cons[s], sscnn.HALO_INPUT, *nb(halos, s), halos[s])
        sscnn.conv_fwd_push(convs[s], xs[s], None, wd, bd, y_push, p)
        torch.cuda.synchronize()
        ref = y_full[:, :, :, s * wol:(s + 1) * wol]
        assert_close(host(y), ref, TOL_FWD, f"{name} shard {s}: stem forward vs oracle")
        assert_close(host(y_tiled), ref, TOL_FWD, f"{name} shard {s}: tiled forward vs oracle")
        assert torch.equal(y_push, y), f"{name} shard {s}: pushing changed the stem forward's output"
        ys.append(y)
    for s in range(S):
        gathered = torch.empty(cons[s].halo_shape(sscnn.HALO_INPUT), device="cuda")
        sscnn.halo_gather(cons[s], sscnn.HALO_INPUT, *nb(ys, s), gathered)
        torch.cuda.synchronize()
        assert torch.equal(halos[s], gathered), f"{name} shard {s}: pushed halo != gathered halo"


@pytest.mark.parametrize("case", STEM_CASES, ids=[c[0] for c in STEM_CASES])
def test_stem_backward_matches_oracle(case):
    """The stem's backward (grad_input, grad_weight / grad_bias partials) on the same shapes:
    against the oracle, conv_bwd's grad_input bit for bit against conv_bwd_input's, and
    grad_weight computed with and without grad_bias equal."""
    name, n, co, h, w, S = case
    _say(f"  stem bwd {name}: ({n},3,{h},{w}) <- {co} channels, {S} shards")
    rng = np.random.default_rng(5100 + STEM_CASES.index(case))
    x = rng.standard_normal((n, 3, h, w)).astype(np.float32)
    g = rng.standard_normal((n, co, h // 4, w // 4)).astype(np.float32)
    wt = (rng.standard_normal((co, 3, 4, 4)) * 0.1).astype(np.float32)
    xs, gs = slices(x, S), slices(g, S)
    wd = to_dev(wt)
    dx_full = oracle.conv_bwd_input(g, wt, x.shape, 4, 0, 1)
    wl, wol = w // S, w // 4 // S
    for s in range(S):
        c = sscnn.conv_init(n, 3, co, h, wl, 4, 4, 0, 1, s, S)
        gw_ref, gb_ref = oracle.conv_bwd_weight(x, g, 4, 4, 0, 1, cols=(s * wol, (s + 1) * wol))
        ws = sscnn.new_workspace(c)
        dx = torch.empty(c.x_shape, device="cuda")
        gw, gb = torch.empty(c.w_shape, device="cuda"), torch.empty(co, device="cuda")
        sscnn.conv_bwd(c, xs[s], None, gs[s], None, wd, dx, gw, gb, ws)
        dx1 = torch.empty(c.x_shape, device="cuda")
        sscnn.conv_bwd_input(c, gs[s], None, wd, dx1)
        gw_nb = torch.empty_like(gw)
        sscnn.conv_bwd(c, xs[s], None, gs[s], None, wd, torch.empty_like(dx), gw_nb, None, ws)
        torch.cuda.synchronize()
        assert_close(host(dx), dx_full[:, :, :, s * wl:(s + 1) * wl], TOL_DX, f"{name} shard {s}: grad_input vs oracle")
        assert_close(host(gw), gw_ref, TOL_GW, f"{name} shard {s}: grad_weight partial vs oracle")
        assert_close(host(gb), gb_ref, TOL_GW, f"{name} shard {s}: grad_bias partial vs oracle")
        assert torch.equal(dx, dx1), f"{name} shard {s}: conv_bwd grad_input != conv_bwd_input"
        assert torch.equal(gw_nb, gw), f"{name} shard {s}: grad_weight without grad_bias differs"
