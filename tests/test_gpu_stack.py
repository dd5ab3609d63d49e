"""GPU parity of the sharded ConvNeXt-style convolution stack (needs an MI355X).

* A stack with the layer structure of the ConvNeXt-XL stack (stem 4x4/4,
  depthwise 7x7, 2x2/2 downsamples) at the pages' map sizes but fewer
  channels runs through the oracle's unsharded chain: every layer's forward
  output, grad_input and grad_weight / grad_bias partials of every shard are
  compared element by element, and the reduced gradients with the full ones.
* The full-size stacks on (7,3,512,2048) and (7,3,512,4096) inputs are run on
  all four shards, in the launch configuration the benchmark times.  For the
  measured shard (1 of 4) every layer's forward output, grad_input, and
  grad_weight / grad_bias partials are compared element by element with the
  oracle's share of the unsharded chain (``oracle.stack_shard``, computed from
  the seeded global tensors only).  As extra checks, every layer of every
  shard satisfies identities that hold exactly in exact arithmetic:
  <Y_s - b, G_s> = <W, gW_s> per shard (the grad_weight partial is the
  adjoint of the forward over the shard's own columns),
  sum_s <X_s, dX_s> = sum_s <Y_s - b, G_s> (grad_input is the adjoint of the
  whole sharded forward), and the reduced gradients equal the shard sum.
"""
import time

import numpy as np
import pytest
import torch

import oracle
from shard_harness import TOL_DX, TOL_FWD, TOL_GW, assert_close, host, slices
from spatially_sharded_cnn_amd import stack as sstack
from spatially_sharded_cnn_amd import workloads

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _oracle_layers(wl, T):
    return [dict(wt=T.weights[l], b=T.biases[l], k=L.k, stride=L.stride, pad=L.pad, groups=L.groups)
            for l, L in enumerate(wl.layers)]


@pytest.mark.parametrize("push", [True, False], ids=["push_halos", "gather_halos"])
def test_reduced_convnext_stack_all_layers_vs_oracle(push):
    """Stem -> dw -> ds -> dw -> ds -> dw -> ds -> dw on a (1,3,256,1024) input
    split four ways, channels 32/64/128/256; the depthwise layers' halos
    pushed by the layers before them, or gathered by the layers themselves."""
    layers = workloads.convnext_stack(1, 1024, h=256, dims=(32, 64, 128, 256))
    wl = workloads.stack("convnext_reduced", layers, num_shards=4, seed=2001)
    T = workloads.generate(wl)
    S = wl.num_shards
    _say(f"  reduced stack: input {wl.x_shape}, S={S}, push={push}")
    st = sstack.ShardedStack(wl.layers, S, T.weights, T.biases, push=push)
    st.forward(slices(T.x, S))
    st.backward(slices(T.g, S))
    torch.cuda.synchronize()

    OL = _oracle_layers(wl, T)
    acts = oracle.stack_forward(T.x, OL)
    grads = oracle.stack_backward(acts, OL, T.g)
    for l, L in enumerate(wl.layers):
        ls = st.state[l]
        wol, wli = L.out_shape[3] // S, L.in_shape[3] // S
        g_out, dx_full, gw_full, gb_full = grads[l]
        for s in range(S):
            co, ci = (s * wol, (s + 1) * wol), (s * wli, (s + 1) * wli)
            assert_close(host(ls.y[s]), acts[l + 1][..., co[0]:co[1]], TOL_FWD, f"{L.name} shard {s} forward")
            assert_close(host(ls.dx[s]), dx_full[..., ci[0]:ci[1]], TOL_DX, f"{L.name} shard {s} grad_input")
            gw_s, gb_s = oracle.conv_bwd_weight(acts[l], g_out, L.k, L.stride, L.pad, L.groups, cols=co)
            assert_close(host(ls.gw_parts[s]), gw_s, TOL_GW, f"{L.name} shard {s} grad_weight partial")
            assert_close(host(ls.gb_parts[s]), gb_s, TOL_GW, f"{L.name} shard {s} grad_bias partial")
        assert_close(host(ls.gw), gw_full, TOL_GW, f"{L.name} reduced grad_weight")
        assert_close(host(ls.gb), gb_full, TOL_GW, f"{L.name} reduced grad_bias")


def test_stack_on_a_side_stream_equals_default_stream():
    """The same small stack run on a stream of its own (kernels and every
    temporary on that stream) gives bitwise the results of the default stream."""
    layers = workloads.convnext_stack(1, 512, h=128, dims=(16, 32, 64, 128))
    wl = workloads.stack("convnext_small", layers, num_shards=4, seed=2002)
    T = workloads.generate(wl)
    S = wl.num_shards
    runs = []
    for stream in (None, torch.cuda.Stream()):
        st = sstack.ShardedStack(wl.layers, S, T.weights, T.biases, stream=stream)
        xs, gs = slices(T.x, S), slices(T.g, S)
        torch.cuda.synchronize()
        st.forward(xs)
        st.backward(gs)
        torch.cuda.synchronize()
        runs.append([(torch.cat(ls.y, 3), torch.cat(ls.dx, 3), ls.gw.clone(), ls.gb.clone()) for ls in st.state])
    for l, (a, b) in enumerate(zip(*runs)):
        for t0, t1 in zip(a, b):
            assert torch.equal(t0, t1), f"layer {l} differs between the default and a side stream"


def _dot(a, b):
    return float(torch.sum(a.double() * b.double()))


def _absdot(a, b):
    return float(torch.sum((a.double() * b.double()).abs()))


@pytest.mark.parametrize("name", ["convnext_xl_w2048", "convnext_xl_w4096"])
def test_full_size_convnext_stack_identities(name):
    wl = workloads.WORKLOADS[name]
    T = workloads.generate(wl)
    S = wl.num_shards
    _say(f"  {name}: input {wl.x_shape}, S={S}")
    st = sstack.ShardedStack(wl.layers, S, T.weights, T.biases)
    st.forward(slices(T.x, S))
    st.backward(slices(T.g, S))
    torch.cuda.synchronize()

    # stem forward at sampled outputs of the measured shard against the oracle
    L0 = wl.layers[0]
    s = wl.shard
    y0 = host(st.state[0].y[s])
    rng = np.random.default_rng(5)
    m = 3000
    idx = np.stack([rng.integers(0, d, m) for d in y0.shape], axis=1)
    gidx = idx.copy()
    gidx[:, 3] += s * (L0.out_shape[3] // S)
    ref = oracle.conv_fwd_at(T.x, T.weights[0], T.biases[0], L0.stride, L0.pad, L0.groups, gidx)
    assert_close(y0[tuple(idx.T)], ref, TOL_FWD, f"{name} stem forward (sampled)")

    for l, L in enumerate(wl.layers):
        ls = st.state[l]
        b = st.b[l].double().view(1, -1, 1, 1)
        w = st.w[l]
        total_yg = total_xdx = scale_all = 0.0
        for sh in range(S):
            ym = ls.y[sh].double() - b
            lhs = _dot(ym, ls.g[sh])
            gw_s = ls.gw_parts[sh]
            rhs = _dot(w, gw_s)
            scale = _absdot(w, gw_s) + 1e-30
            assert abs(lhs - rhs) <= 1e-5 * scale, f"{name} {L.name} shard {sh}: <Y-b,G>={lhs} <W,gW>={rhs}"
            total_yg += lhs
            total_xdx += _dot(ls.x[sh], ls.dx[sh])
            scale_all += _absdot(ls.x[sh], ls.dx[sh])
            assert torch.isfinite(ls.dx[sh]).all() and torch.isfinite(ls.y[sh]).all()
        assert abs(total_yg - total_xdx) <= 1e-5 * (scale_all + 1e-30), \
            f"{name} {L.name}: sum <Y-b,G> = {total_yg}, sum <X,dX> = {total_xdx}"
        acc_w, acc_b = ls.gw_parts[0].clone(), ls.gb_parts[0].clone()
        for sh in range(1, S):
            acc_w, acc_b = acc_w + ls.gw_parts[sh], acc_b + ls.gb_parts[sh]
        assert torch.equal(ls.gw, acc_w) and torch.equal(ls.gb, acc_b), f"{name} {L.name}: bucketed reduction"
        _say(f"  {name} {L.name}: identities hold")


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", ["convnext_xl_w2048", "convnext_xl_w4096"])
def test_full_size_convnext_stack_measured_shard_vs_oracle(name):
    wl = workloads.WORKLOADS[name]
    T = workloads.generate(wl)
    S, s = wl.num_shards, wl.shard
    _say(f"  {name}: input {wl.x_shape}, S={S}, measured shard {s}")
    st = sstack.ShardedStack(wl.layers, S, T.weights, T.biases)
    st.forward(slices(T.x, S))
    st.backward(slices(T.g, S))
    torch.cuda.synchronize()
    got = [dict(y=host(ls.y[s]), dx=host(ls.dx[s]), gw=host(ls.gw_parts[s]), gb=host(ls.gb_parts[s]))
           for ls in st.state]
    del st
    torch.cuda.empty_cache()
    t0 = time.perf_counter()
    ref = oracle.stack_shard(T.x, _oracle_layers(wl, T), T.g, S, s)
    _say(f"  {name}: oracle share of the chain in {time.perf_counter() - t0:.1f} s")
    for l, L in enumerate(wl.layers):
        r, gl = ref[l], got[l]
        e_y = assert_close(gl["y"], r["y"], TOL_FWD, f"{name} {L.name} forward")
        e_dx = assert_close(gl["dx"], r["dx"], TOL_DX, f"{name} {L.name} grad_input")
        e_gw = assert_close(gl["gw"], r["gw"], TOL_GW, f"{name} {L.name} grad_weight partial")
        e_gb = assert_close(gl["gb"], r["gb"], TOL_GW, f"{name} {L.name} grad_bias partial")
        _say(f"  {name} {L.name}: normwise errors forward {e_y:.2e} grad_input {e_dx:.2e} "
             f"grad_weight {e_gw:.2e} grad_bias {e_gb:.2e}")
