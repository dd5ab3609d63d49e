"""Host-side tests of the C ABI (no GPU needed, no kernel is launched).

* the library loads and exports every function include/sscnn.h declares;
* sscnn_conv_init derives the halo widths the pages give (5x5 / pad 2 /
  stride 1 -> 2 columns each side: NVIDIA blog "Perception Model Training for
  Autonomous Vehicles with Tensor Parallelism", Figure 1 text) and, for every
  other layer kind, the widths a brute-force enumeration of the taps gives;
* every call validates its arguments before launching and reports errors.
"""
import ctypes
import json
import pathlib
import re

import pytest

from spatially_sharded_cnn_amd import sscnn

ROOT = pathlib.Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "sscnn.h"
GOLDEN = ROOT / "tests" / "golden" / "page_facts.json"


def _declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sscnn_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = sscnn.lib()
    declared = _declared_functions()
    assert len(declared) >= 10
    for name in declared:
        assert hasattr(L, name), f"{name} declared in sscnn.h but not exported"
    assert set(declared) == set(sscnn.EXPORTED)


def test_abi_version_matches_header():
    m = re.search(r"#define SSCNN_ABI_VERSION (\d+)", HEADER.read_text())
    assert sscnn.abi_version() == int(m.group(1))


def test_status_codes_match_header():
    text = HEADER.read_text()
    for name, val in [("SSCNN_OK", 0), ("SSCNN_EINVAL", -1), ("SSCNN_EUNSUPPORTED", -2),
                      ("SSCNN_EWORKSPACE", -3), ("SSCNN_EHIP", -4)]:
        assert re.search(rf"#define {name} \(?{val}\)?", text), name
    assert sscnn.status_string(0) == "ok"
    assert "invalid" in sscnn.status_string(-1)


def _brute_force_halos(k, s, p, wl, num_shards=3, shard=1):
    """Columns outside the shard that its outputs read (forward), and
    grad_output columns outside its output range that its grad_input reads."""
    w = wl * num_shards
    wo = (w + 2 * p - k) // s + 1
    wol = wo // num_shards
    lo_in, hi_in = shard * wl, (shard + 1) * wl
    reads = set()
    for j in range(shard * wol, (shard + 1) * wol):
        for kw in range(k):
            reads.add(j * s + kw - p)
    hl = max([lo_in - q for q in reads if q < lo_in] + [0])
    hr = max([q - hi_in + 1 for q in reads if q >= hi_in] + [0])
    greads = set()
    for x in range(lo_in, hi_in):
        for kw in range(k):
            u = x + p - kw
            if u % s == 0:
                greads.add(u // s)
    lo_o, hi_o = shard * wol, (shard + 1) * wol
    ghl = max([lo_o - j for j in greads if j < lo_o] + [0])
    ghr = max([j - hi_o + 1 for j in greads if j >= hi_o] + [0])
    return hl, hr, ghl, ghr


@pytest.mark.parametrize("k,s,p", [(5, 1, 2), (7, 1, 3), (3, 1, 1), (1, 1, 0), (4, 4, 0),
                                   (2, 2, 0), (3, 2, 1), (5, 2, 2), (6, 2, 2)])
def test_conv_init_halo_widths_match_brute_force(k, s, p):
    wl = 8 * s
    c = sscnn.conv_init(2, 4, 6, 10, wl, k, s, p, 1, 1, 3)
    assert (c.halo_l, c.halo_r, c.ghalo_l, c.ghalo_r) == _brute_force_halos(k, s, p, wl)
    assert c.w_out_local == wl // s
    assert c.h_out == (10 + 2 * p - k) // s + 1


def test_conv_init_matches_page_example():
    facts = json.loads(GOLDEN.read_text())
    for ex in facts["halo_examples"]:
        c = sscnn.conv_init(1, 3, 8, 32, 16, ex["kernel"], ex["stride"], ex["pad"], 1, 1, 4)
        n = ex["halo_columns_each_side"]
        assert (c.halo_l, c.halo_r) == (n, n)
        assert (c.ghalo_l, c.ghalo_r) == (n, n)


@pytest.mark.parametrize("args,status", [
    ((1, 3, 8, 8, 16, 5, 1, 5, 1, 0, 2), sscnn.EINVAL),        # pad >= k
    ((1, 3, 8, 8, 16, 5, 1, 2, 2, 0, 2), sscnn.EINVAL),        # groups does not divide c_in
    ((1, 4, 8, 8, 16, 5, 1, 2, 1, 2, 2), sscnn.EINVAL),        # shard out of range
    ((0, 4, 8, 8, 16, 5, 1, 2, 1, 0, 2), sscnn.EINVAL),        # empty batch
    ((1, 4, 8, 2, 16, 7, 1, 1, 1, 0, 2), sscnn.EINVAL),        # image smaller than kernel
    ((1, 4, 8, 8, 15, 2, 2, 0, 1, 0, 2), sscnn.EUNSUPPORTED),  # w_local % stride
    ((1, 4, 8, 8, 2, 7, 1, 3, 1, 0, 2), sscnn.EUNSUPPORTED),   # halo wider than a slice
    ((1, 4, 8, 8, 16, 3, 2, 0, 1, 0, 2), sscnn.EUNSUPPORTED),  # output columns do not split evenly
    ((1, 4, 8, 8, 16, 5, 1, 0, 1, 0, 2), sscnn.EUNSUPPORTED),  # 'valid' conv shrinks W
])
def test_conv_init_rejects(args, status):
    with pytest.raises(sscnn.SscnnError) as ei:
        sscnn.conv_init(*args)
    assert ei.value.status == status
    assert sscnn.last_error()


# Raw calls with fake, never-dereferenced device addresses: every case below
# fails validation before anything is launched.
FAKE = 0x10000


def _conv(shard=1, num_shards=4):
    return sscnn.conv_init(1, 3, 8, 32, 16, 5, 1, 2, 1, shard, num_shards)


def test_calls_reject_null_and_misaligned_pointers():
    L = sscnn.lib()
    c = _conv()
    r = ctypes.byref(c)
    assert L.sscnn_conv_fwd(r, None, FAKE, FAKE, None, FAKE, None) == sscnn.EINVAL
    assert L.sscnn_conv_fwd(r, FAKE, None, FAKE, None, FAKE, None) == sscnn.EINVAL  # halo needed
    assert L.sscnn_conv_fwd(r, FAKE + 4, FAKE, FAKE, None, FAKE, None) == sscnn.EINVAL
    assert "aligned" in sscnn.last_error()
    assert L.sscnn_conv_fwd(None, FAKE, FAKE, FAKE, None, FAKE, None) == sscnn.EINVAL
    assert L.sscnn_conv_bwd_input(r, FAKE, None, FAKE, FAKE, None) == sscnn.EINVAL
    assert L.sscnn_conv_bwd_input(r, FAKE, FAKE, None, FAKE, None) == sscnn.EINVAL
    assert L.sscnn_conv_bwd_weight_partial(r, FAKE, FAKE, FAKE, None, None, None, 0, None) == sscnn.EINVAL
    assert L.sscnn_conv_bwd_weight_partial(r, FAKE, FAKE, FAKE, FAKE, FAKE + 8, None, 0, None) == sscnn.EINVAL


def test_fused_backward_validation():
    L = sscnn.lib()
    c = _conv()
    r = ctypes.byref(c)
    F = FAKE
    ok = (F, F + 4096, F + 8192, F + 12288, F + 16384, F + 20480, F + 24576, F + 28672)
    # every required pointer, one at a time
    for i in range(7):
        args = list(ok[:7])
        args[i] = None
        assert L.sscnn_conv_bwd(r, *args, None, None, 0, None) == sscnn.EINVAL, i
    assert L.sscnn_conv_bwd(r, F + 4, *ok[1:7], None, None, 0, None) == sscnn.EINVAL   # misaligned x
    # grad_x aliasing an input
    assert L.sscnn_conv_bwd(r, *ok[:5], ok[2], ok[6], None, None, 0, None) == sscnn.EINVAL
    assert "alias" in sscnn.last_error()
    # a depthwise layer needs its workspace
    d = sscnn.conv_init(1, 16, 16, 64, 16, 7, 1, 3, 16, 1, 4)
    need = L.sscnn_conv_bwd_weight_workspace_bytes(ctypes.byref(d))
    assert need > 0
    assert L.sscnn_conv_bwd(ctypes.byref(d), *ok[:7], None, None, 0, None) == sscnn.EWORKSPACE
    assert L.sscnn_conv_bwd(ctypes.byref(d), *ok[:7], None, F + 32768, need - 4, None) == sscnn.EWORKSPACE


def test_halo_gather_neighbour_rules():
    L = sscnn.lib()
    first, mid, last = _conv(0), _conv(1), _conv(3)
    # shard 0 has no left neighbour, the last shard no right one
    assert L.sscnn_halo_gather(ctypes.byref(first), 0, FAKE, FAKE, FAKE, None) == sscnn.EINVAL
    assert L.sscnn_halo_gather(ctypes.byref(mid), 0, None, FAKE, FAKE, None) == sscnn.EINVAL
    assert L.sscnn_halo_gather(ctypes.byref(mid), 0, FAKE, None, FAKE, None) == sscnn.EINVAL
    assert L.sscnn_halo_gather(ctypes.byref(last), 0, FAKE, FAKE, FAKE, None) == sscnn.EINVAL
    assert L.sscnn_halo_gather(ctypes.byref(mid), 7, FAKE, FAKE, FAKE, None) == sscnn.EINVAL
    assert L.sscnn_halo_gather(ctypes.byref(mid), 0, FAKE, FAKE, None, None) == sscnn.EINVAL


def test_patchify_layer_needs_no_halo_and_launches_nothing_for_it():
    L = sscnn.lib()
    c = sscnn.conv_init(1, 3, 16, 16, 16, 4, 4, 0, 1, 1, 4)
    assert (c.halo_l, c.halo_r, c.ghalo_l, c.ghalo_r) == (0, 0, 0, 0)
    # zero-width halo: returns OK without launching (halo may be NULL)
    assert L.sscnn_halo_gather(ctypes.byref(c), 0, FAKE, FAKE, None, None) == sscnn.OK


def test_edited_descriptor_is_rejected():
    L = sscnn.lib()
    c = _conv()
    c.halo_l = 3   # derived field no longer matches the layer
    assert L.sscnn_conv_fwd(ctypes.byref(c), FAKE, FAKE, FAKE, None, FAKE, None) == sscnn.EINVAL
    assert "sscnn_conv_init" in sscnn.last_error()
    assert L.sscnn_conv_bwd_weight_workspace_bytes(ctypes.byref(c)) == 0


def test_partial_reduce_validation():
    L = sscnn.lib()
    vp = ctypes.c_void_p
    ptrs = (vp * 2)(FAKE, FAKE + 4096)
    assert L.sscnn_partial_reduce(None, 2, 16, FAKE + 8192, None) == sscnn.EINVAL
    assert L.sscnn_partial_reduce(ptrs, 0, 16, FAKE + 8192, None) == sscnn.EINVAL
    assert L.sscnn_partial_reduce(ptrs, 65, 16, FAKE + 8192, None) == sscnn.EINVAL
    assert L.sscnn_partial_reduce(ptrs, 2, -1, FAKE + 8192, None) == sscnn.EINVAL
    assert L.sscnn_partial_reduce(ptrs, 2, 16, None, None) == sscnn.EINVAL
    assert L.sscnn_partial_reduce(ptrs, 2, 16, FAKE, None) == sscnn.EINVAL   # aliasing
    nulls = (vp * 2)(FAKE, None)
    assert L.sscnn_partial_reduce(nulls, 2, 16, FAKE + 8192, None) == sscnn.EINVAL


def test_binding_rejects_host_tensors():
    import torch
    c = _conv()
    x = torch.zeros(c.x_shape)
    with pytest.raises(ValueError):
        sscnn.conv_fwd(c, x, None, None, None, None)


def test_autograd_shard_round_trip_and_host_tensors_rejected():
    """The autograd layer marshals only: shard / unshard are exact, and host
    tensors are refused before anything is launched."""
    import torch
    from spatially_sharded_cnn_amd import autograd as sa
    x = torch.arange(2 * 3 * 4 * 12, dtype=torch.float32).reshape(2, 3, 4, 12)
    xs = sa.shard(x, 4)
    assert [tuple(t.shape) for t in xs] == [(2, 3, 4, 3)] * 4 and all(t.is_contiguous() for t in xs)
    assert torch.equal(sa.unshard(xs), x)
    with pytest.raises(ValueError):
        sa.shard(x, 5)
    layer = sa.ShardedConv2d(3, 6, 3, padding=1, device="cpu")
    assert layer.weight.shape == (6, 3, 3, 3) and layer.bias.shape == (6,)
    with pytest.raises(ValueError):
        layer(xs)
    rows = sa.shard(x, 2, dim=2)
    assert [tuple(t.shape) for t in rows] == [(2, 3, 2, 12)] * 2 and all(t.is_contiguous() for t in rows)
    assert torch.equal(sa.unshard(rows, dim=2), x)
    with pytest.raises(ValueError):
        sa.shard(x, 3, dim=2)
    with pytest.raises(ValueError):
        sa.ShardedConv2d(3, 6, 3, padding=1, device="cpu", dim=1)
    hlayer = sa.ShardedConv2d(3, 6, 3, padding=1, device="cpu", dim=2)
    with pytest.raises(ValueError):
        hlayer(rows)


def test_split_calls_validate_before_launching():
    """The interior / edge halves of a split convolution check their own
    arguments; an edge call of a layer without halo columns returns OK with
    nothing to launch."""
    L = sscnn.lib()
    c = _conv()
    r = ctypes.byref(c)
    F = FAKE
    # interior calls need no halo, but every other operand
    assert L.sscnn_conv_fwd_interior(r, None, F, None, F + 4096, None) == sscnn.EINVAL
    assert L.sscnn_conv_fwd_interior(r, F, None, None, F + 4096, None) == sscnn.EINVAL
    assert L.sscnn_conv_fwd_interior(r, F, F, F + 4, F + 4096, None) == sscnn.EINVAL       # misaligned bias
    assert L.sscnn_conv_bwd_input_interior(r, F, F, None, None) == sscnn.EINVAL
    assert L.sscnn_conv_bwd_weight_partial_interior(r, F, F, None, None, None, 0, None) == sscnn.EINVAL
    assert L.sscnn_conv_bwd_interior(r, F, F, F, F, F + 4096, None, None, 0, None) == sscnn.EINVAL  # grad_x is x
    assert "alias" in sscnn.last_error()
    assert L.sscnn_conv_bwd_interior(r, F, F + 4096, F + 8192, F + 12288, None, None, None, 0, None) == sscnn.EINVAL
    # edge calls need the halo and refuse outputs that alias it
    assert L.sscnn_conv_fwd_edge(r, None, F, F + 4096, None) == sscnn.EINVAL
    assert L.sscnn_conv_fwd_edge(r, F, F + 4096, F, None) == sscnn.EINVAL
    assert L.sscnn_conv_bwd_input_edge(r, None, F, F + 4096, None) == sscnn.EINVAL
    assert L.sscnn_conv_bwd_input_edge(r, F, F + 4096, None, None) == sscnn.EINVAL
    assert L.sscnn_conv_bwd_weight_edge(r, None, F, F + 4096, None) == sscnn.EINVAL
    assert L.sscnn_conv_bwd_weight_edge(r, F, F + 4096, F, None) == sscnn.EINVAL
    # a depthwise layer's interior grad_weight still needs its workspace
    d = sscnn.conv_init(1, 16, 16, 64, 16, 7, 1, 3, 16, 1, 4)
    assert L.sscnn_conv_bwd_weight_partial_interior(ctypes.byref(d), F, F + 4096, F + 8192, None, None, 0,
                                                    None) == sscnn.EWORKSPACE
    assert L.sscnn_conv_bwd_interior(ctypes.byref(d), F, F + 4096, F + 8192, F + 12288, F + 16384, None,
                                     None, 0, None) == sscnn.EWORKSPACE
    # patchify: no halo columns, so the edge calls have nothing to add
    p = sscnn.conv_init(1, 3, 16, 16, 16, 4, 4, 0, 1, 1, 4)
    rp = ctypes.byref(p)
    assert L.sscnn_conv_fwd_edge(rp, None, None, None, None) == sscnn.OK
    assert L.sscnn_conv_bwd_input_edge(rp, None, None, None, None) == sscnn.OK
    assert L.sscnn_conv_bwd_weight_edge(rp, None, None, None, None) == sscnn.OK


@pytest.mark.parametrize("k,s,p", [(5, 1, 2), (7, 1, 3), (3, 1, 1), (1, 1, 0), (4, 4, 0),
                                   (2, 2, 0), (3, 2, 1), (5, 2, 2), (6, 2, 2)])
def test_hconv_init_row_halos_match_brute_force(k, s, p):
    """Height sharding: the row halos are the column halos' rule along H (the
    same brute-force enumeration of the taps, with rows for columns)."""
    hl = 8 * s
    c = sscnn.hconv_init(2, 4, 6, hl, 12 * s, k, s, p, 1, 1, 3)
    assert (c.halo_u, c.halo_d, c.ghalo_u, c.ghalo_d) == _brute_force_halos(k, s, p, hl)
    assert c.h_out_local == hl // s and c.w_out == 12


@pytest.mark.parametrize("args,status", [
    ((1, 3, 8, 16, 8, 5, 1, 5, 1, 0, 2), sscnn.EINVAL),        # pad >= k
    ((1, 3, 8, 16, 8, 5, 1, 2, 2, 0, 2), sscnn.EINVAL),        # groups does not divide c_in
    ((1, 4, 8, 16, 8, 5, 1, 2, 1, 2, 2), sscnn.EINVAL),        # shard out of range
    ((1, 4, 8, 16, 2, 7, 1, 1, 1, 0, 2), sscnn.EINVAL),        # image narrower than the kernel
    ((1, 4, 8, 15, 8, 2, 2, 0, 1, 0, 2), sscnn.EUNSUPPORTED),  # h_local % stride
    ((1, 4, 8, 2, 8, 7, 1, 3, 1, 0, 2), sscnn.EUNSUPPORTED),   # row halo taller than a slice
    ((1, 4, 8, 16, 8, 5, 1, 0, 1, 0, 2), sscnn.EUNSUPPORTED),  # 'valid' conv shrinks H
])
def test_hconv_init_rejects(args, status):
    with pytest.raises(sscnn.SscnnError) as ei:
        sscnn.hconv_init(*args)
    assert ei.value.status == status


def test_hconv_calls_validate_before_launching():
    L = sscnn.lib()
    F = FAKE
    first, mid, last = (sscnn.hconv_init(1, 3, 8, 16, 32, 5, 1, 2, 1, s, 4) for s in (0, 1, 3))
    r = ctypes.byref(mid)
    # neighbour rules of the row exchange
    assert L.sscnn_row_halo_gather(ctypes.byref(first), 0, F, F, F, None) == sscnn.EINVAL
    assert L.sscnn_row_halo_gather(r, 0, None, F, F, None) == sscnn.EINVAL
    assert L.sscnn_row_halo_gather(r, 0, F, None, F, None) == sscnn.EINVAL
    assert L.sscnn_row_halo_gather(ctypes.byref(last), 0, F, F, F, None) == sscnn.EINVAL
    assert L.sscnn_row_halo_gather(r, 5, F, F, F, None) == sscnn.EINVAL
    assert L.sscnn_row_halo_gather(r, 0, F, F, None, None) == sscnn.EINVAL
    # every required operand
    assert L.sscnn_hconv_fwd(r, None, F, F, None, F, None) == sscnn.EINVAL
    assert L.sscnn_hconv_fwd(r, F, None, F, None, F, None) == sscnn.EINVAL     # row halo needed
    assert L.sscnn_hconv_fwd(r, F + 4, F, F, None, F, None) == sscnn.EINVAL
    assert L.sscnn_hconv_bwd_input(r, F, None, F, F, None) == sscnn.EINVAL
    assert L.sscnn_hconv_bwd_weight_partial(r, F, F, F, None, None, None, 0, None) == sscnn.EINVAL
    assert L.sscnn_hconv_bwd(r, F, F, F, F, F, F, F + 4096, None, None, 0, None) == sscnn.EINVAL   # grad_x is x
    # an edited descriptor
    mid.halo_u = 1
    assert L.sscnn_hconv_fwd(r, F, F, F, None, F, None) == sscnn.EINVAL
    assert "sscnn_hconv_init" in sscnn.last_error()
    # patchify: no row halo, nothing to launch for the exchange
    p = sscnn.hconv_init(1, 3, 16, 16, 16, 4, 4, 0, 1, 1, 4)
    assert (p.halo_u, p.halo_d, p.ghalo_u, p.ghalo_d) == (0, 0, 0, 0)
    assert L.sscnn_row_halo_gather(ctypes.byref(p), 0, F, F, None, None) == sscnn.OK


def test_block_op_calls_validate_before_launching():
    """The ConvNeXt block's other steps check shapes, pointers and aliasing on
    the host and launch nothing when they fail; empty work returns OK."""
    L = sscnn.lib()
    F, G = FAKE, FAKE + 4096
    eps = ctypes.c_float(1e-6)
    # LayerNorm: dims, eps, required pointers, misalignment, aliasing of the saved statistics
    assert L.sscnn_layernorm_fwd(0, 4, 2, 2, eps, F, F, F, F, F + 64, F + 128, None) == sscnn.EINVAL
    assert L.sscnn_layernorm_fwd(1, 4, 2, 2, ctypes.c_float(0.0), F, F, F, G, F + 64, F + 128, None) == sscnn.EINVAL
    assert L.sscnn_layernorm_fwd(1, 4, 2, 2, eps, None, F, F, G, F + 64, F + 128, None) == sscnn.EINVAL
    assert L.sscnn_layernorm_fwd(1, 4, 2, 2, eps, F + 4, F, F, G, F + 64, F + 128, None) == sscnn.EINVAL
    assert L.sscnn_layernorm_fwd(1, 4, 2, 2, eps, F, F, F, G, F + 64, F + 64, None) == sscnn.EINVAL
    assert L.sscnn_layernorm_bwd(1, 4, 2, 2, F, G, F, F, F, F, None, None, None) == sscnn.EINVAL   # dx is x
    assert L.sscnn_layernorm_bwd(1, 4, 2, 2, F, G, F, F, F, None, F + 64, F + 64, None) == sscnn.EINVAL
    # GELU: negative count; zero count is a no-op even with no pointers
    assert L.sscnn_gelu_fwd(-1, F, F, None) == sscnn.EINVAL
    assert L.sscnn_gelu_fwd(0, None, None, None) == sscnn.OK
    assert L.sscnn_gelu_bwd(16, F, None, F, None) == sscnn.EINVAL
    # DropPath factors: keep_prob in (0, inf), n >= 0
    assert L.sscnn_droppath_scales(1, 0, 4, 0.0, F, None) == sscnn.EINVAL
    assert L.sscnn_droppath_scales(1, 0, 4, float("nan"), F, None) == sscnn.EINVAL
    assert L.sscnn_droppath_scales(1, 0, -1, 0.5, F, None) == sscnn.EINVAL
    assert L.sscnn_droppath_scales(1, 0, 0, 0.5, None, None) == sscnn.OK
    assert L.sscnn_droppath_scales(1, 0, 4, 0.5, None, None) == sscnn.EINVAL
    # layer scale + residual: h*w a multiple of 4, required pointers, dh aliasing what dgamma reads
    assert L.sscnn_layer_scale_residual_fwd(1, 4, 3, 3, F, F, F, None, G, None) == sscnn.EINVAL
    assert L.sscnn_layer_scale_residual_fwd(1, 4, 2, 2, F, None, F, None, G, None) == sscnn.EINVAL
    assert L.sscnn_layer_scale_residual_bwd(1, 4, 2, 2, F, G, F, None, G, F + 64, None) == sscnn.EINVAL
    assert "aliases" in sscnn.last_error()


def test_pointwise_gelu_calls_validate_before_launching():
    """The fused 1x1 + GELU calls take only pointwise layers on the matrix-core
    path and need every pointer; they refuse the rest on the host."""
    L = sscnn.lib()
    F, G = FAKE, FAKE + (1 << 20)
    pw = sscnn.conv_init(1, 16, 32, 4, 16, 1, 1, 0, 1, 0, 1)
    by = ctypes.byref
    for bad in (sscnn.conv_init(1, 16, 32, 8, 16, 3, 1, 1, 1, 0, 1),    # 3x3
                sscnn.conv_init(1, 16, 32, 8, 16, 2, 2, 0, 1, 0, 1),    # 2x2 patchify
                sscnn.conv_init(1, 12, 32, 4, 16, 1, 1, 0, 1, 0, 1),    # c_in not a multiple of 16
                sscnn.conv_init(1, 16, 32, 4, 8, 1, 1, 0, 1, 0, 1)):    # slice width not a multiple of 16
        assert L.sscnn_pointwise_gelu_fwd(by(bad), F, F, None, G, G + 4096, None) == sscnn.EUNSUPPORTED
        assert L.sscnn_pointwise_bwd_input_gelu(by(bad), F, F, F, G, None) == sscnn.EUNSUPPORTED
    assert L.sscnn_pointwise_gelu_fwd(by(pw), F, F, None, G, None, None) == sscnn.EINVAL       # no y_act
    assert L.sscnn_pointwise_gelu_fwd(by(pw), None, F, None, G, G + 4096, None) == sscnn.EINVAL
    assert L.sscnn_pointwise_bwd_input_gelu(by(pw), F, F, None, G, None) == sscnn.EINVAL      # no pre
    assert L.sscnn_pointwise_bwd_input_gelu(by(pw), F, F, F + 4, G, None) == sscnn.EINVAL     # misaligned
    assert L.sscnn_pointwise_gelu_fwd(by(pw), F, F, None, G, G, None) == sscnn.EINVAL         # y_act is y
    assert L.sscnn_pointwise_bwd_input_gelu(by(pw), F, F, G, G, None) == sscnn.EINVAL         # grad_x is pre
    assert "aliases" in sscnn.last_error()


def test_block_op_bindings_refuse_host_tensors():
    import torch
    x = torch.zeros(1, 4, 2, 2)
    with pytest.raises(ValueError):
        sscnn.layernorm_fwd(x, torch.ones(4), torch.zeros(4), x.clone(), torch.zeros(1, 2, 2), torch.zeros(1, 2, 2))
    with pytest.raises(ValueError):
        sscnn.gelu_fwd(x, x.clone())


def test_gconv_init_and_gathers_validate():
    """2-D shards: the supported layer kinds, the grid bounds and the
    neighbour rules of the two exchange phases, checked before any launch."""
    L = sscnn.lib()
    F = FAKE
    c = sscnn.gconv_init(2, 8, 8, 16, 32, 7, 1, 3, 8, 1, 3, 0, 2)        # depthwise 7x7, middle row, left column
    assert (c.halo, c.h_out_local, c.w_out_local) == (3, 16, 32)
    p = sscnn.gconv_init(1, 16, 32, 8, 16, 2, 2, 0, 1, 0, 2, 1, 2)       # 2x2/2 downsample: no halo
    d = sscnn.gconv_init(1, 16, 24, 12, 20, 5, 1, 2, 1, 1, 2, 1, 2)      # dense 5x5 pad 2: the pages' example
    assert (d.halo, d.h_out_local, d.w_out_local) == (2, 12, 20)
    assert (p.halo, p.h_out_local, p.w_out_local) == (0, 4, 8)
    with pytest.raises(sscnn.SscnnError) as e:
        sscnn.gconv_init(1, 8, 8, 16, 32, 3, 1, 1, 1, 0, 2, 0, 2)        # dense 3x3 with 8 channels (< 16)
    assert e.value.status == sscnn.EUNSUPPORTED
    with pytest.raises(sscnn.SscnnError) as e:
        sscnn.gconv_init(1, 8, 8, 16, 24, 7, 1, 3, 8, 0, 2, 0, 2)        # depthwise block width 24
    assert e.value.status == sscnn.EUNSUPPORTED
    with pytest.raises(sscnn.SscnnError) as e:
        sscnn.gconv_init(1, 8, 8, 16, 32, 7, 1, 3, 8, 2, 2, 0, 2)        # shard_h outside the grid
    assert e.value.status == sscnn.EINVAL
    r = ctypes.byref(c)
    # phase 1: middle row needs both up and down
    assert L.sscnn_grid_row_halo_gather(r, 0, None, F, F, None) == sscnn.EINVAL
    assert L.sscnn_grid_row_halo_gather(r, 0, F, None, F, None) == sscnn.EINVAL
    # phase 2: left column has no left neighbour; a right neighbour needs its row halo
    assert L.sscnn_grid_col_halo_gather(r, 0, F, F, F, F, F, None) == sscnn.EINVAL
    assert L.sscnn_grid_col_halo_gather(r, 0, None, None, F, None, F, None) == sscnn.EINVAL
    assert L.sscnn_grid_col_halo_gather(r, 2, None, None, F, F, F, None) == sscnn.EINVAL
    # the convolution calls need both halos when the layer has one
    assert L.sscnn_gconv_fwd(r, F, None, F, F, None, F, None) == sscnn.EINVAL
    assert L.sscnn_gconv_fwd(r, F, F, None, F, None, F, None) == sscnn.EINVAL
    c.halo = 1
    assert L.sscnn_gconv_fwd(r, F, F, F, F, None, F, None) == sscnn.EINVAL      # edited descriptor
    # no halo: the gathers have nothing to do
    assert L.sscnn_grid_row_halo_gather(ctypes.byref(p), 0, F, None, None, None) == sscnn.OK


def test_stream_copy_validation():
    L = sscnn.lib()
    assert L.sscnn_stream_copy(FAKE, FAKE + 4096, 0, None) == sscnn.OK          # nothing to do
    assert L.sscnn_stream_copy(FAKE, FAKE + 4096, -1, None) == sscnn.EINVAL
    assert L.sscnn_stream_copy(None, FAKE + 4096, 16, None) == sscnn.EINVAL
    assert L.sscnn_stream_copy(FAKE, None, 16, None) == sscnn.EINVAL
    assert L.sscnn_stream_copy(FAKE + 4, FAKE + 4096, 16, None) == sscnn.EINVAL   # misaligned
    assert L.sscnn_stream_copy(FAKE, FAKE + 32, 16, None) == sscnn.EINVAL         # overlapping
    assert "overlap" in sscnn.last_error()


def test_push_validation():
    L = sscnn.lib()
    F = FAKE
    first, mid, last = (sscnn.conv_init(1, 16, 32, 16, 32, 2, 2, 0, 1, s, 4) for s in (0, 1, 3))
    args = (F, None, F + 4096, F + 8192, F + 12288)            # x, x_halo, weight, bias, y
    P = sscnn.Push
    # the neighbour pointers must match the shard's position
    assert L.sscnn_conv_fwd_push(ctypes.byref(mid), *args, ctypes.byref(P(3, 3, None, F + 16384, None)), None) \
        == sscnn.EINVAL
    assert L.sscnn_conv_fwd_push(ctypes.byref(first), *args, ctypes.byref(P(3, 3, F + 16384, F + 20480, F)), None) \
        == sscnn.EINVAL
    # an edge shard needs its own halo for the open side
    assert L.sscnn_conv_fwd_push(ctypes.byref(last), *args, ctypes.byref(P(3, 3, F + 16384, None, None)), None) \
        == sscnn.EINVAL
    # widths beyond the pushed slice (16 output columns)
    assert L.sscnn_conv_fwd_push(ctypes.byref(mid), *args, ctypes.byref(P(17, 3, F + 16384, F + 20480, None)),
                                 None) == sscnn.EINVAL
    # a halo buffer aliasing the output
    assert L.sscnn_conv_fwd_push(ctypes.byref(mid), *args, ctypes.byref(P(3, 3, F + 12288, F + 20480, None)),
                                 None) == sscnn.EINVAL
    assert "alias" in sscnn.last_error()
    # negative widths
    assert L.sscnn_conv_fwd_push(ctypes.byref(mid), *args, ctypes.byref(P(-1, 3, F + 16384, F + 20480, None)),
                                 None) == sscnn.EINVAL
