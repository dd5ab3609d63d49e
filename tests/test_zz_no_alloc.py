"""sscnn_conv_bwd_noalloc: the backward entry point that allocates nothing.

Its split-reduction scratch is the library's own device array instead of a
caller workspace.  The GPU tests call it through the C ABI twice in a row --
a depthwise 7x7 C=256 shard of (7,256,128,256), then a smaller depthwise
5x5 layer -- and compare every output with sscnn_conv_bwd on the same inputs
(which the parity tests compare with the oracle): the same kernels run, so
the results must be bitwise equal.  The host tests check that layers needing
more than the scratch, and bad pointers, are rejected before anything is
launched.
"""
import ctypes

import numpy as np
import pytest
import torch

from spatially_sharded_cnn_amd import sscnn, workloads

FAKE = 0x10000


def _ok_ptrs():
    return tuple(FAKE + 4096 * i for i in range(8))   # x .. grad_b_part


def test_noalloc_rejects_layers_beyond_its_scratch():
    """The dense 5x5 256->256 shard needs ~210 MB of split-K scratch: rejected
    with SSCNN_EWORKSPACE on the host, before any device call."""
    L = sscnn.lib()
    wl = workloads.WORKLOADS["dense5x5_c256"]
    Lr = wl.layers[0]
    n, ci, h, w = Lr.in_shape
    c = sscnn.conv_init(n, ci, Lr.co, h, w // 4, Lr.k, Lr.stride, Lr.pad, Lr.groups, 1, 4)
    assert L.sscnn_conv_bwd_weight_workspace_bytes(ctypes.byref(c)) > sscnn.NOALLOC_SCRATCH_BYTES
    p = _ok_ptrs()
    assert L.sscnn_conv_bwd_noalloc(ctypes.byref(c), *p, None) == sscnn.EWORKSPACE
    assert "scratch" in sscnn.last_error()


def test_noalloc_validates_pointers_first():
    L = sscnn.lib()
    c = sscnn.conv_init(1, 16, 16, 64, 16, 7, 1, 3, 16, 1, 4)
    r = ctypes.byref(c)
    p = list(_ok_ptrs())
    for i in range(7):                     # every required pointer
        q = list(p)
        q[i] = None
        assert L.sscnn_conv_bwd_noalloc(r, *q, None) == sscnn.EINVAL, i
    q = list(p)
    q[5] = q[2]                            # grad_x aliasing grad_y
    assert L.sscnn_conv_bwd_noalloc(r, *q, None) == sscnn.EINVAL
    assert "alias" in sscnn.last_error()
    q = list(p)
    q[0] += 4                              # misaligned x
    assert L.sscnn_conv_bwd_noalloc(r, *q, None) == sscnn.EINVAL
    assert L.sscnn_conv_bwd_noalloc(None, *p, None) == sscnn.EINVAL


def _layer_tensors(n, c, h, w_local, k, shard, num_shards, seed):
    """A depthwise layer's shard: input, halos from real neighbours, grad_output."""
    conv = sscnn.conv_init(n, c, c, h, w_local, k, 1, k // 2, c, shard, num_shards)
    rng = np.random.default_rng(seed)
    w = w_local * num_shards
    x = rng.standard_normal((n, c, h, w), dtype=np.float32)
    g = rng.standard_normal((n, c, h, w), dtype=np.float32)
    wt = (rng.standard_normal((c, 1, k, k), dtype=np.float32) * np.float32(0.02))

    def sl(a, i):
        return torch.from_numpy(np.ascontiguousarray(a[:, :, :, i * w_local:(i + 1) * w_local])).cuda()

    left = shard - 1 if shard > 0 else None
    right = shard + 1 if shard < num_shards - 1 else None
    xs, gs = sl(x, shard), sl(g, shard)
    xh = torch.empty(conv.halo_shape(sscnn.HALO_INPUT), device="cuda")
    gh = torch.empty(conv.halo_shape(sscnn.HALO_GRAD_OUTPUT), device="cuda")
    sscnn.halo_gather(conv, sscnn.HALO_INPUT, sl(x, left) if left is not None else None,
                      sl(x, right) if right is not None else None, xh)
    sscnn.halo_gather(conv, sscnn.HALO_GRAD_OUTPUT, sl(g, left) if left is not None else None,
                      sl(g, right) if right is not None else None, gh)
    return conv, xs, xh, gs, gh, torch.from_numpy(wt).cuda()


def _both(conv, xs, xh, gs, gh, wt):
    """(conv_bwd with a workspace, conv_bwd_noalloc) outputs; the noalloc
    outputs start as NaN so that an unwritten element shows."""
    ref = dict(dx=torch.empty(conv.x_shape, device="cuda"), gw=torch.empty(conv.w_shape, device="cuda"),
               gb=torch.empty((conv.c_out,), device="cuda"))
    got = {k: torch.full_like(v, float("nan")) for k, v in ref.items()}
    sscnn.conv_bwd(conv, xs, xh, gs, gh, wt, ref["dx"], ref["gw"], ref["gb"], sscnn.new_workspace(conv))
    sscnn.conv_bwd_noalloc(conv, xs, xh, gs, gh, wt, got["dx"], got["gw"], got["gb"])
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.gpu
def test_noalloc_equals_conv_bwd_two_calls_second_smaller():
    print("  noalloc: call 1, depthwise 7x7 C=256 shard (7,256,128,64) of 4", flush=True)
    big = _layer_tensors(7, 256, 128, 64, 7, 1, 4, seed=11)
    need = sscnn.conv_bwd_weight_workspace_bytes(big[0])
    assert 0 < need <= sscnn.NOALLOC_SCRATCH_BYTES
    ref, got = _both(*big)
    for k in ref:
        assert torch.equal(got[k], ref[k]), f"call 1: {k} differs from conv_bwd"
    del big, ref, got
    print("  noalloc: call 2, depthwise 5x5 C=64 shard (2,64,32,32) of 3, edge shard", flush=True)
    small = _layer_tensors(2, 64, 32, 32, 5, 2, 3, seed=12)
    assert sscnn.conv_bwd_weight_workspace_bytes(small[0]) < need
    ref, got = _both(*small)
    for k in ref:
        assert torch.equal(got[k], ref[k]), f"call 2: {k} differs from conv_bwd"


@pytest.mark.gpu
def test_noalloc_rejection_leaves_outputs_untouched():
    wl = workloads.WORKLOADS["dense5x5_tiny"]
    Lr = wl.layers[0]
    # a layer whose scratch need is zero runs (small dense layer, direct kernels)
    n, ci, h, w = Lr.in_shape
    c = sscnn.conv_init(n, ci, Lr.co, h, w // 4, Lr.k, Lr.stride, Lr.pad, Lr.groups, 1, 4)
    rng = np.random.default_rng(3)
    t = lambda shape: torch.from_numpy(rng.uniform(-1, 1, size=shape).astype(np.float32)).cuda()
    xs, gs = t(c.x_shape), t(c.y_shape)
    xh, gh = t(c.halo_shape(sscnn.HALO_INPUT)), t(c.halo_shape(sscnn.HALO_GRAD_OUTPUT))
    wt = t(c.w_shape)
    ref, got = _both(c, xs, xh, gs, gh, wt)
    for k in ref:
        assert torch.equal(got[k], ref[k]), k
    # the dense 256->256 shard is refused and nothing is written
    Ld = workloads.WORKLOADS["dense5x5_c256"].layers[0]
    n, ci, h, w = Ld.in_shape
    d = sscnn.conv_init(1, ci, Ld.co, 8, w // 4, Ld.k, Ld.stride, Ld.pad, Ld.groups, 1, 4)
    if sscnn.conv_bwd_weight_workspace_bytes(d) <= sscnn.NOALLOC_SCRATCH_BYTES:
        d = sscnn.conv_init(n, ci, Ld.co, h, w // 4, Ld.k, Ld.stride, Ld.pad, Ld.groups, 1, 4)
    z = lambda shape: torch.zeros(shape, device="cuda")
    dx, gw, gb = (torch.full(s, 7.0, device="cuda") for s in (d.x_shape, d.w_shape, (d.c_out,)))
    with pytest.raises(sscnn.SscnnError) as ei:
        sscnn.conv_bwd_noalloc(d, z(d.x_shape), z(d.halo_shape(sscnn.HALO_INPUT)), z(d.y_shape),
                               z(d.halo_shape(sscnn.HALO_GRAD_OUTPUT)), z(d.w_shape), dx, gw, gb)
    assert ei.value.status == sscnn.EWORKSPACE
    torch.cuda.synchronize()
    assert bool((dx == 7).all()) and bool((gw == 7).all()) and bool((gb == 7).all())
