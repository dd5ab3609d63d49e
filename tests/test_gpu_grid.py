"""GPU parity of 2-D H x W sharding (needs an MI355X).

Every block of a num_h x num_w grid runs the two exchange phases (rows from
the blocks above and below, then columns over the extended rows from the
blocks beside it and their row halos, so the corners come from the diagonal
blocks), then the forward, grad_input and grad_weight partial, against the
oracle on the global tensors, for depthwise, patchify and dense 3x3 / 5x5
layers (the dense ones on the matrix cores, whose tiles read the row halo
and the column halo over the extended rows directly):
* both halos bit-exact against the zero-padded neighbourhood of the block;
* forward and grad_input within 1e-5 of the unsharded layer's block,
  grad_weight / grad_bias partials within 1e-4 of the sums over the block's
  own outputs, and the reduced partials within 1e-4 of the full gradients.
"""
import numpy as np
import pytest
import torch

import oracle
from shard_harness import TOL_DX, TOL_FWD, TOL_GW, assert_close, host, to_dev
from spatially_sharded_cnn_amd import sscnn

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


# (name, n, c_in, c_out, H, W, k, stride, pad, groups, num_h, num_w)
CASES = [
    ("dw7_2x2", 2, 8, 8, 2 * 16, 2 * 32, 7, 1, 3, 8, 2, 2),
    ("dw3_3x3", 1, 6, 6, 3 * 16, 3 * 16, 3, 1, 1, 6, 3, 3),
    ("dw5_2x3_tall", 1, 4, 4, 2 * 40, 3 * 64, 5, 1, 2, 4, 2, 3),
    ("dw7_2x2_64rows", 1, 4, 4, 2 * 64, 2 * 64, 7, 1, 3, 4, 2, 2),     # 64-row blocks: 4 rows per thread
    ("dw7_2x2_w32_h45", 1, 4, 4, 2 * 45, 2 * 32, 7, 1, 3, 4, 2, 2),    # 32-wide blocks, 32-row tiles, ragged rows
    ("patch2_2x2_no_halo", 1, 16, 32, 2 * 8, 2 * 32, 2, 2, 0, 1, 2, 2),
    ("pw1x1_2x2_no_halo", 2, 16, 48, 2 * 8, 2 * 32, 1, 1, 0, 1, 2, 2),
    # dense layers on the matrix cores, reading both halos (the 5x5 pad-2 example of the pages)
    ("mfma5x5_2x2", 1, 24, 32, 2 * 12, 2 * 64, 5, 1, 2, 1, 2, 2),
    ("mfma3x3_3x2_ragged", 2, 20, 36, 3 * 10, 2 * 36, 3, 1, 1, 1, 3, 2),      # ragged row, column, channel tiles
    ("mfma5x5_2x3_tiles", 1, 64, 72, 2 * 20, 3 * 132, 5, 1, 2, 1, 2, 3),      # several tiles per block
    ("mfma5x5_2x2_c128", 2, 128, 128, 2 * 32, 2 * 128, 5, 1, 2, 1, 2, 2),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_grid_shards_match_oracle(case):
    name, n, ci, co, H, W, k, s, p, g, NH, NW = case
    _say(f"  grid {name}: ({n},{ci},{H},{W}) k={k} s={s} p={p} g={g} on {NH}x{NW}")
    rng = np.random.default_rng(4400 + CASES.index(case))
    x = rng.standard_normal((n, ci, H, W)).astype(np.float32)
    wt = (rng.standard_normal((co, ci // g, k, k)) * 0.1).astype(np.float32)
    b = (rng.standard_normal(co) * 0.1).astype(np.float32)
    Ho, Wo = (H + 2 * p - k) // s + 1, (W + 2 * p - k) // s + 1
    gy = rng.standard_normal((n, co, Ho, Wo)).astype(np.float32)
    bh, bw, oh, ow = H // NH, W // NW, Ho // NH, Wo // NW
    convs = {(i, j): sscnn.gconv_init(n, ci, co, bh, bw, k, s, p, g, i, NH, j, NW) for i in range(NH) for j in range(NW)}
    X = {ij: to_dev(oracle.shard_block(x, NH, NW, *ij)) for ij in convs}
    G = {ij: to_dev(oracle.shard_block(gy, NH, NW, *ij)) for ij in convs}
    hh = convs[(0, 0)].halo
    nb = lambda d, i, j: d.get((i, j))
    # phase 1 for every block, then phase 2 (which reads the neighbours' phase-1 results)
    RX, RG, CX, CG = {}, {}, {}, {}
    for (i, j), c in convs.items():
        RX[i, j] = torch.empty(c.row_halo_shape(sscnn.HALO_INPUT), device="cuda") if hh else None
        RG[i, j] = torch.empty(c.row_halo_shape(sscnn.HALO_GRAD_OUTPUT), device="cuda") if hh else None
        sscnn.grid_row_halo_gather(c, sscnn.HALO_INPUT, nb(X, i - 1, j), nb(X, i + 1, j), RX[i, j])
        sscnn.grid_row_halo_gather(c, sscnn.HALO_GRAD_OUTPUT, nb(G, i - 1, j), nb(G, i + 1, j), RG[i, j])
    for (i, j), c in convs.items():
        CX[i, j] = torch.empty(c.col_halo_shape(sscnn.HALO_INPUT), device="cuda") if hh else None
        CG[i, j] = torch.empty(c.col_halo_shape(sscnn.HALO_GRAD_OUTPUT), device="cuda") if hh else None
        sscnn.grid_col_halo_gather(c, sscnn.HALO_INPUT, nb(X, i, j - 1), nb(RX, i, j - 1), nb(X, i, j + 1),
                                   nb(RX, i, j + 1), CX[i, j])
        sscnn.grid_col_halo_gather(c, sscnn.HALO_GRAD_OUTPUT, nb(G, i, j - 1), nb(RG, i, j - 1), nb(G, i, j + 1),
                                   nb(RG, i, j + 1), CG[i, j])
    torch.cuda.synchronize()
    wt_d, b_d = to_dev(wt), to_dev(b)
    y_full = oracle.conv_fwd(x, wt, b, s, p, g)
    dx_full = oracle.conv_bwd_input(gy, wt, x.shape, s, p, g)
    gw_full, gb_full = oracle.conv_bwd_weight(x, gy, k, s, p, g)
    parts = []
    for (i, j), c in convs.items():
        if hh:
            rx, cx = oracle.block_halos(x, NH, NW, i, j, hh, hh, hh, hh)
            rg, cg = oracle.block_halos(gy, NH, NW, i, j, hh, hh, hh, hh)
            np.testing.assert_array_equal(host(RX[i, j]), rx)
            np.testing.assert_array_equal(host(CX[i, j]), cx)
            np.testing.assert_array_equal(host(RG[i, j]), rg)
            np.testing.assert_array_equal(host(CG[i, j]), cg)
        y = torch.empty(c.y_shape, device="cuda")
        dx, dx2 = torch.empty(c.x_shape, device="cuda"), torch.empty(c.x_shape, device="cuda")
        pw, pb = torch.empty(c.w_shape, device="cuda"), torch.empty(co, device="cuda")
        gw2, gb2 = torch.empty(c.w_shape, device="cuda"), torch.empty(co, device="cuda")
        ws = sscnn.new_gworkspace(c)
        sscnn.gconv_fwd(c, X[i, j], RX[i, j], CX[i, j], wt_d, b_d, y)
        sscnn.gconv_bwd_input(c, G[i, j], RG[i, j], CG[i, j], wt_d, dx)
        sscnn.gconv_bwd_weight_partial(c, X[i, j], RX[i, j], CX[i, j], G[i, j], pw, pb, ws)
        sscnn.gconv_bwd(c, X[i, j], RX[i, j], CX[i, j], G[i, j], RG[i, j], CG[i, j], wt_d, dx2, gw2, gb2, ws)
        torch.cuda.synchronize()
        rows, cols = (i * oh, (i + 1) * oh), (j * ow, (j + 1) * ow)
        assert_close(host(y), y_full[:, :, rows[0]:rows[1], cols[0]:cols[1]], TOL_FWD, f"{name} ({i},{j}) forward")
        assert_close(host(dx), dx_full[:, :, i * bh:(i + 1) * bh, j * bw:(j + 1) * bw], TOL_DX,
                     f"{name} ({i},{j}) grad_input")
        gw_ref, gb_ref = oracle.conv_bwd_weight_block(x, gy, k, s, p, g, rows, cols)
        assert_close(host(pw), gw_ref, TOL_GW, f"{name} ({i},{j}) grad_weight partial")
        assert_close(host(pb), gb_ref, TOL_GW, f"{name} ({i},{j}) grad_bias partial")
        assert torch.equal(dx2, dx)
        assert_close(host(gw2), gw_ref, TOL_GW, f"{name} ({i},{j}) gconv_bwd grad_weight")
        parts.append(torch.cat([pw.flatten(), pb]))
    red = torch.empty_like(parts[0])
    sscnn.partial_reduce(parts, red)
    torch.cuda.synchronize()
    assert_close(host(red[:-co]).reshape(gw_full.shape), gw_full, TOL_GW, f"{name} reduced grad_weight")
    assert_close(host(red[-co:]), gb_full, TOL_GW, f"{name} reduced grad_bias")
