#!/usr/bin/env python3
"""Benchmark of the width-sharded convolution hot path on one MI355X.

One step is one pass of the whole path for the measured shard (shard 1 of 4)
of a layer: halo_gather(X) -> conv_fwd -> halo_gather(G) -> conv_bwd_input ->
conv_bwd_weight_partial -> partial_reduce (grad_weight and grad_bias of the
four shards).  Inputs are seeded synthetic tensors already resident in HBM;
each step uses the next of several independent buffer sets so that the
256 MB last-level cache cannot serve one step's data to the next.

Prints ONE JSON line.  `value` is the algorithmic GB/s of a step:
  forward  X_ext + W + b + Y
  backward G_ext + X_ext + W + dX + gW + gB
  reduce   (S + 1) * (|gW| + |gB|)
(halo copies are inside the timed step but not counted as useful bytes).
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

METRIC = "W-shard conv fwd+bwd GB/s & TFLOP/s FP32; % of HBM/MFMA roofline, 1 GPU"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
MFMA_F32_PEAK_TFLOPS = 157.3     # MI355X dense FP32 matrix
# FP32 vector FMA without packed math: 256 CUs x 4 SIMDs x 16 lanes x 2 FLOP x 2.4 GHz.
VALU_F32_PEAK_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12


def _parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dw7_c256",
                    help="dw7_c256 (default), dense5x5_c256 or dense5x5_tiny")
    ap.add_argument("--sets", type=int, default=3, help="independent buffer sets rotated per step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def main():
    args = _parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU's share of the sharded path; --gpus {args.gpus} "
              f"(WORLD_SIZE={world}) is not supported: the halo exchange and the partial "
              "reduction run on one device here.", file=sys.stderr)
        return 2

    import torch
    from spatially_sharded_cnn_amd import sscnn, workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = "cuda"
    wl = workloads.WORKLOADS[args.workload]
    assert len(wl.layers) == 1, "bench.py times single-layer workloads"
    L = wl.layers[0]
    S, s = wl.num_shards, wl.shard
    T = workloads.generate(wl)

    def shard_of(a, i):
        w = a.shape[3] // S
        return np.ascontiguousarray(a[:, :, :, i * w:(i + 1) * w])

    c = sscnn.conv_init(L.in_shape[0], L.ci, L.co, L.in_shape[2], L.in_shape[3] // S, L.k, L.stride,
                        L.pad, L.groups, s, S)
    left, right = s - 1 if s > 0 else None, s + 1 if s < S - 1 else None
    wt = torch.from_numpy(T.weights[0]).to(dev)
    b = torch.from_numpy(T.biases[0]).to(dev)

    def dev_of(a):
        return torch.from_numpy(a).to(dev)

    xs_h = {i: shard_of(T.x, i) for i in range(S)}
    gs_h = {i: shard_of(T.g, i) for i in range(S)}
    sets = []
    for k in range(args.sets):
        st = dict(
            x=dev_of(xs_h[s]), g=dev_of(gs_h[s]),
            xl=dev_of(xs_h[left]) if left is not None else None,
            xr=dev_of(xs_h[right]) if right is not None else None,
            gl=dev_of(gs_h[left]) if left is not None else None,
            gr=dev_of(gs_h[right]) if right is not None else None,
            xh=torch.empty(c.halo_shape(sscnn.HALO_INPUT), device=dev),
            gh=torch.empty(c.halo_shape(sscnn.HALO_GRAD_OUTPUT), device=dev),
            y=torch.empty(c.y_shape, device=dev), dx=torch.empty(c.x_shape, device=dev),
            gw=torch.empty(c.w_shape, device=dev), gb=torch.empty((c.c_out,), device=dev),
            gw_red=torch.empty(c.w_shape, device=dev), gb_red=torch.empty((c.c_out,), device=dev),
        )
        sets.append(st)
    ws = sscnn.new_workspace(c)
    del xs_h, gs_h

    # The other shards' partial gradients (computed once, untimed): partial_reduce
    # sums all four in shard order, this shard's fresh partial in its slot.
    other_gw, other_gb = {}, {}
    for i in range(S):
        if i == s:
            continue
        ci_ = sscnn.conv_init(L.in_shape[0], L.ci, L.co, L.in_shape[2], L.in_shape[3] // S, L.k,
                              L.stride, L.pad, L.groups, i, S)
        xi, gi = dev_of(shard_of(T.x, i)), dev_of(shard_of(T.g, i))
        li = dev_of(shard_of(T.x, i - 1)) if i > 0 else None
        ri = dev_of(shard_of(T.x, i + 1)) if i < S - 1 else None
        xhi = torch.empty(ci_.halo_shape(sscnn.HALO_INPUT), device=dev)
        sscnn.halo_gather(ci_, sscnn.HALO_INPUT, li, ri, xhi)
        gwi, gbi = torch.empty(c.w_shape, device=dev), torch.empty((c.c_out,), device=dev)
        sscnn.conv_bwd_weight_partial(ci_, xi, xhi, gi, gwi, gbi, sscnn.new_workspace(ci_))
        other_gw[i], other_gb[i] = gwi, gbi
        del xi, gi, li, ri, xhi
    torch.cuda.synchronize()

    names = ["halo_gather_x", "conv_fwd", "halo_gather_g", "conv_bwd_input",
             "conv_bwd_weight_partial", "partial_reduce"]

    def step(st, ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        sscnn.halo_gather(c, sscnn.HALO_INPUT, st["xl"], st["xr"], st["xh"])
        mark(1)
        sscnn.conv_fwd(c, st["x"], st["xh"], wt, b, st["y"])
        mark(2)
        sscnn.halo_gather(c, sscnn.HALO_GRAD_OUTPUT, st["gl"], st["gr"], st["gh"])
        mark(3)
        sscnn.conv_bwd_input(c, st["g"], st["gh"], wt, st["dx"])
        mark(4)
        sscnn.conv_bwd_weight_partial(c, st["x"], st["xh"], st["g"], st["gw"], st["gb"], ws)
        mark(5)
        parts_w = [st["gw"] if i == s else other_gw[i] for i in range(S)]
        parts_b = [st["gb"] if i == s else other_gb[i] for i in range(S)]
        sscnn.partial_reduce(parts_w, st["gw_red"])
        sscnn.partial_reduce(parts_b, st["gb_red"])
        mark(6)

    for i in range(args.warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()

    # Timed region: K steps, events only at the ends.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        step(sets[i % len(sets)])
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_per_step = e0.elapsed_time(e1) / args.steps

    # Per-call durations: the same K steps again with an event pair around
    # every call, on the stream the kernels run on (torch's current stream).
    per = {n: [] for n in names}
    for i in range(args.steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(7)]
        step(sets[i % len(sets)], ev)
        torch.cuda.synchronize()
        for j, n in enumerate(names):
            per[n].append(ev[j].elapsed_time(ev[j + 1]))
    per_us = {n: 1e3 * float(np.mean(v)) for n, v in per.items()}

    # Algorithmic work.
    f4 = 4
    n, ci, h, wl_ = c.n, c.c_in, c.h, c.w_local
    co, ho, wol = c.c_out, c.h_out, c.w_out_local
    x_ext = n * ci * h * (wl_ + c.halo_l + c.halo_r) * f4
    g_ext = n * co * ho * (wol + c.ghalo_l + c.ghalo_r) * f4
    x_b, y_b, g_b = n * ci * h * wl_ * f4, n * co * ho * wol * f4, n * co * ho * wol * f4
    w_b = co * (ci // c.groups) * c.k * c.k * f4
    b_b = co * f4
    red_b = (S + 1) * (w_b + b_b)
    bytes_fwd = x_ext + w_b + b_b + y_b
    bytes_bwd = g_ext + x_ext + w_b + x_b + w_b + b_b
    step_bytes = bytes_fwd + bytes_bwd + red_b
    flops_pass = 2 * (ci // c.groups) * c.k * c.k * n * co * ho * wol
    step_flops = 3 * flops_pass
    kern_bytes = {
        "halo_gather_x": 2 * n * ci * h * (c.halo_l + c.halo_r) * f4,
        "conv_fwd": x_ext + w_b + b_b + y_b,
        "halo_gather_g": 2 * n * co * ho * (c.ghalo_l + c.ghalo_r) * f4,
        "conv_bwd_input": g_ext + w_b + x_b,
        "conv_bwd_weight_partial": x_ext + g_b + w_b + b_b,
        "partial_reduce": red_b,
    }
    kern_flops = {"conv_fwd": flops_pass, "conv_bwd_input": flops_pass, "conv_bwd_weight_partial": flops_pass}
    dense = c.groups == 1 and min(c.c_in, c.c_out) >= 16
    compute_peak = MFMA_F32_PEAK_TFLOPS if dense else VALU_F32_PEAK_TFLOPS
    dom = max(per_us, key=per_us.get)
    t_hbm = kern_bytes[dom] / (HBM_PEAK_GBS * 1e9)
    t_cmp = kern_flops.get(dom, 0) / (compute_peak * 1e12)
    if t_cmp > t_hbm:
        achieved = kern_flops[dom] / (per_us[dom] * 1e-6) / 1e12
        roof = {"bound": "mfma" if dense else "alu", "achieved": round(achieved, 3),
                "peak": round(compute_peak, 1), "unit": "TFLOP/s"}
    else:
        achieved = kern_bytes[dom] / (per_us[dom] * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = None
    roof["kernel"] = dom
    roof["avg_us"] = round(per_us[dom], 2)

    step_s = ms_per_step * 1e-3
    value = step_bytes / step_s / 1e9
    step_roof_s = sum(max(kern_bytes[k] / (HBM_PEAK_GBS * 1e9),
                          kern_flops.get(k, 0) / (compute_peak * 1e12)) for k in kern_bytes)
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description, "shard": f"{s} of {S}",
                   "shard_input": list(c.x_shape), "weight": list(c.w_shape),
                   "buffer_sets": args.sets},
        "tflops": round(step_flops / step_s / 1e12, 3),
        "step_bytes": step_bytes, "step_flops": step_flops,
        "hbm_roofline_frac": round(step_bytes / (HBM_PEAK_GBS * 1e9) / step_s, 4),
        "roofline_frac_step": round(step_roof_s / step_s, 4),
        "roofline": roof,
        "kernels_us": {k: round(v, 2) for k, v in per_us.items()},
        "wall_s_timed": round(wall, 4),
    }

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, T, L, S, s)

    print(json.dumps(out), flush=True)
    return 0


def cpu_baseline(wl, T, L, S, s):
    """The oracle (plain C, double, OpenMP) on the same unit as a step: this
    shard's forward, grad_input and grad_weight/grad_bias partial.  The sample
    is bounded to roughly 10-30 s of host work: the whole shard for the small
    and depthwise layers, the first image's first 16 rows for the dense
    256->256 layer (a smaller image of the same layer)."""
    import oracle
    n, _, h_full, _ = T.x.shape
    imgs, rows = n, h_full
    if L.ci // L.groups * L.k * L.k >= 1024:
        imgs, rows = 1, 16
    x = T.x[:imgs, :, :rows]
    g = T.g[:imgs, :, :rows // L.stride]
    wt, b = T.weights[0], T.biases[0]
    wl_, wol = L.in_shape[3] // S, L.out_shape[3] // S
    t0 = time.perf_counter()
    oracle.conv_fwd(x, wt, b, L.stride, L.pad, L.groups, cols=(s * wol, (s + 1) * wol))
    oracle.conv_bwd_input(g, wt, x.shape, L.stride, L.pad, L.groups, cols=(s * wl_, (s + 1) * wl_))
    oracle.conv_bwd_weight(x, g, L.k, L.stride, L.pad, L.groups, cols=(s * wol, (s + 1) * wol))
    dt = time.perf_counter() - t0
    f4 = 4
    ci, co, ho = L.ci, L.co, g.shape[2]
    x_ext = imgs * ci * rows * (wl_ + 2 * L.pad) * f4
    y_b = imgs * co * ho * wol * f4
    w_b = co * (ci // L.groups) * L.k * L.k * f4
    # same accounting as the GPU step (forward + backward, no reduction)
    sample_bytes = (x_ext + w_b + co * f4 + y_b) + (y_b + x_ext + w_b + imgs * ci * rows * wl_ * f4
                                                      + w_b + co * f4)
    return {"value": round(sample_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"images 0..{imgs - 1} of {n}, rows 0..{rows - 1} of {h_full}, shard {s} of {S}: "
                      "forward + grad_input + grad_weight/grad_bias partial (C, double, OpenMP)",
            "cpu": platform.processor() or platform.machine()}


if __name__ == "__main__":
    sys.exit(main())
