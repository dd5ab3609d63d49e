#!/usr/bin/env python3
"""Benchmark of the width-sharded convolution hot path on one MI355X.

The default workload is the largest configuration, the ConvNeXt-XL
convolution stack on shard 1 of 4 of a (7,3,512,4096) input (the shard of the
pages' 4-GPU run).  One step is the shard's forward chain -- per layer
halo_gather(X) where the layer has a halo, then conv_fwd -- and its backward
chain in reverse -- per layer halo_gather(G), conv_bwd (grad_input and the
grad_weight / grad_bias partials in one call) and partial_reduce of the four
shards' [gW | gB].  `value` is the step's algorithmic GB/s; `roofline` is for
its dominant operation; `layers` gives every layer's operations and roofline
fraction.  The same JSON line carries `sub_records` for the other full-size
configurations, each timed on its own with its own roofline: dense5x5_c256
(one 5x5 256->256 layer), dw7_c256 (one depthwise 7x7 C=256 layer) and
convnext_xl_w2048 (the stack on a (7,3,512,2048) input).

For one layer, one step is halo_gather(X) -> conv_fwd -> halo_gather(G) ->
conv_bwd -> partial_reduce.  The separate conv_bwd_input and
conv_bwd_weight_partial calls are timed on their own as well ("ops_us"), and so
is the layer as an interior/edge split ("split": each interior and edge call,
the split step on one stream, and with the halo gathers on a second stream
beside the interior calls; not part of `value`).  Inputs are seeded
synthetic tensors already resident in HBM; each step uses the next of several
independent buffer sets so that the 256 MB last-level cache cannot hand one
step's data to the next.

Algorithmic bytes:
  forward   X_ext + W + b + Y
  backward  G_ext + X_ext + W + dX + gW + gB
  reduce    (S + 1) * (|gW| + |gB|)
(halo copies are inside the timed step but not counted as useful bytes).

`roofline` is for the dominant operation of the step, timed on its own over
back-to-back calls with events on the stream the kernels run on (after
OP_WARM_CALLS untimed calls of it); its bound is
whichever of HBM bytes / 8 TB/s and FLOPs / compute peak is larger, with the
compute peak of the unit it runs on: the FP32 matrix cores (157.3 TFLOP/s)
for the dense layers, the FP32 vector FMA (157.3 TFLOP/s published; plain
v_fmac_f32 with vector-register operands reaches it without packed math)
for the depthwise ones.

    python bench.py [--steps K] [--warmup W] [--no-sub]    # convnext_xl_w4096 + sub-records
    python bench.py --workload dw7_c256|dense5x5_c256|dense5x5_tiny|convnext_xl_w2048
    python bench.py --workload dw7_c256_hshard   # the depthwise step on a split along H (row halos)
    python bench.py --workload convnext_block_c256   # a whole ConvNeXt block on the C=256 shard, per op
    python bench.py --workload dw7_c256_grid   # the depthwise step on a 2 x 2 grid of blocks (2-D shards)
    python bench.py --workload dense5x5_c256_hshard|dense5x5_c256_grid   # the dense 5x5 step split along H / 2-D
    python bench.py --workload convnext_xl_w4096 --profile-op ds3.conv_bwd   # one operation, for counters
    python bench.py --summarize DIR [DIR ...] [--traffic-op OP --traffic-kernels "K1;K2" [--after-calibration]]
                                      # text summary of rocprofv3 output directories
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import pathlib
import platform
import sys
import time

import numpy as np

ROOT = pathlib.Path(__file__).resolve().parent
METRIC = "W-shard conv fwd+bwd GB/s & TFLOP/s FP32; % of HBM/MFMA roofline, 1 GPU"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
MFMA_F32_PEAK_TFLOPS = 157.3     # MI355X dense FP32 matrix
VALU_F32_PEAK_TFLOPS = 157.3     # MI355X FP32 vector FMA
COPY_CAL_BYTES = 256 << 20       # plain device copy used to calibrate FETCH_SIZE / WRITE_SIZE


STEPS_DEFAULT, WARMUP_DEFAULT = 50, 5
# Untimed calls of an operation before it is timed on its own: the matrix-core
# kernels start ~15% slower right after memory-bound work while the shader
# clock comes back up (the chained step's `value` keeps that cost).
OP_WARM_CALLS = 3
STACK_STEPS, STACK_WARMUP = 5, 2   # stack steps run for milliseconds each
DEFAULT_WORKLOAD = "convnext_xl_w4096"
# timed beside the default workload, each as its own record in the same line
SUB_WORKLOADS = ("dense5x5_c256", "dw7_c256", "convnext_xl_w2048")


def _parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help=f"timed steps (default {STEPS_DEFAULT} for one layer, {STACK_STEPS} for a stack)")
    ap.add_argument("--warmup", type=int, default=None,
                    help=f"untimed steps first (default {WARMUP_DEFAULT} for one layer, {STACK_WARMUP} for a stack)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help=f"{DEFAULT_WORKLOAD} (default; the largest configuration), convnext_xl_w2048, "
                         "dense5x5_c256, dw7_c256, dense5x5_tiny, dw7_c256_hshard (the depthwise map split "
                         "along H), convnext_block_c256 (a ConvNeXt block), dw7_c256_grid (2-D shards)")
    ap.add_argument("--no-sub", action="store_true",
                    help="with the default workload: skip the sub-records of " + ", ".join(SUB_WORKLOADS))
    ap.add_argument("--profile-op", metavar="OP",
                    help="stack workloads: after the set-up, run only operation OP (e.g. ds3.conv_bwd) "
                         "--profile-reps times and exit (for counter runs of one operation)")
    ap.add_argument("--profile-reps", type=int, default=10)
    ap.add_argument("--no-push", action="store_true",
                    help="stack workloads: every layer gathers its halos (no push form from the layer before)")
    ap.add_argument("--sets", type=int, default=3, help="independent buffer sets rotated per step")
    ap.add_argument("--op-reps", type=int, default=20, help="back-to-back calls per operation timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-split", action="store_true", help="skip the interior/edge split timings")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the HBM ceiling measurement (for counter runs: its 1 GiB copy would otherwise be "
                         "taken for the 256 MiB calibration copy)")
    ap.add_argument("--summarize", metavar="DIR", nargs="+",
                    help="summarize rocprofv3 output directories and exit")
    ap.add_argument("--traffic-op", help="with --summarize over FETCH_SIZE / WRITE_SIZE runs: the operation "
                    "whose kernels' calibrated HBM bytes per launch are recorded")
    ap.add_argument("--traffic-kernels", help="semicolon-separated substrings naming that operation's kernels")
    ap.add_argument("--after-calibration", action="store_true",
                    help="with --summarize: the operation's figures from the dispatches after the last device "
                         "copy only (in a --profile-op run: the operation's repetitions)")
    return ap.parse_args()


def kernel_source_hash() -> str:
    """Hash of the library sources: a recorded traffic figure is valid only for it."""
    h = hashlib.sha256()
    for p in sorted((ROOT / "spatially_sharded_cnn_amd" / "csrc").glob("*")):
        if p.suffix in (".hip", ".cpp", ".h"):
            h.update(p.name.encode())
            h.update(p.read_bytes())
    h.update((ROOT / "include" / "sscnn.h").read_bytes())
    return h.hexdigest()[:16]


def step_spread(step, n):
    """Median and minimum of n single steps, each between its own pair of
    events (a pass after the timed region; the reported value comes from the
    timed region)."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i, (a, b) in enumerate(ev):
        a.record()
        step(i)
        b.record()
    torch.cuda.synchronize()
    us = sorted(1e3 * a.elapsed_time(b) for a, b in ev)
    return {"step_us_median": round(us[len(us) // 2], 2), "step_us_min": round(us[0], 2), "samples": n}


def gpu_clocks():
    """The current shader and memory clock levels of the GPUs the driver
    lists, read from sysfs (the level marked '*' in pp_dpm_sclk / pp_dpm_mclk),
    or None where those files are not readable."""
    out = {}
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        rec = {}
        for clk in ("sclk", "mclk"):
            try:
                cur = [ln for ln in pathlib.Path(dev, f"pp_dpm_{clk}").read_text().splitlines() if "*" in ln]
            except OSError:
                continue
            if cur:
                rec[clk] = cur[0].split(":", 1)[-1].replace("*", "").strip()
        if rec:
            out[pathlib.Path(dev).parent.name] = rec
    return out or None


def hbm_ceiling(nbytes=1 << 30, reps=10):
    """The copy rate of this device: the library's plain streaming kernel
    (sscnn_stream_copy) and torch's copy_, each over nbytes one way (a read
    and a write of every byte, so 2 * nbytes of HBM traffic per copy), far
    larger than the 256 MB last-level cache; GB/s from events around reps
    back-to-back copies."""
    import torch
    from spatially_sharded_cnn_amd import sscnn
    src = torch.empty(nbytes // 4, device="cuda").normal_()
    dst = torch.empty_like(src)
    res = {}
    for name, f in (("stream_copy_gbs", lambda: sscnn.stream_copy(src, dst)),
                    ("torch_copy_gbs", lambda: dst.copy_(src))):
        f()
        torch.cuda.synchronize()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        for _ in range(reps):
            f()
        a1.record()
        torch.cuda.synchronize()
        res[name] = round(2 * nbytes * reps / (a0.elapsed_time(a1) * 1e-3) / 1e9, 1)
    ok = bool(torch.equal(src, dst))
    del src, dst
    torch.cuda.empty_cache()
    res.update(bytes_each_way=nbytes, copy_correct=ok, peak_gbs=HBM_PEAK_GBS,
               stream_copy_frac_of_peak=round(res["stream_copy_gbs"] / HBM_PEAK_GBS, 4))
    return res


def recorded_traffic(workload: str):
    """Counter-measured HBM bytes per launch of the dominant operation, from
    profiles/traffic_<workload>.md, if recorded for the current sources."""
    p = ROOT / "profiles" / f"traffic_{workload}.md"
    if not p.exists():
        return None
    for line in p.read_text().splitlines():
        if line.startswith("traffic_json:"):
            rec = json.loads(line.split(":", 1)[1])
            if rec.get("source_hash") == kernel_source_hash():
                return rec
    return None


def main():
    args = _parse()
    if args.summarize:
        return summarize(args.summarize, args.traffic_op, args.traffic_kernels, args.after_calibration)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU's share of the sharded path; --gpus {args.gpus} "
              f"(WORLD_SIZE={world}) is not supported: the halo exchange and the partial "
              "reduction run on one device here.", file=sys.stderr)
        return 2

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    out = run_workload(args, args.workload)
    if out is None:                 # --profile-op: the run printed its own line
        return 0
    if not args.no_ceiling:
        out["hbm_ceiling"] = hbm_ceiling()
    if args.workload == DEFAULT_WORKLOAD and not args.no_sub and not args.profile_op:
        # The other full-size configurations, each timed on its own with its own
        # defaults for steps and warmup, and with its own roofline.
        out["sub_records"] = {}
        for name in SUB_WORKLOADS:
            sub = argparse.Namespace(**vars(args))
            sub.steps = sub.warmup = None
            sub.no_cpu_baseline = args.no_cpu_baseline or name == "convnext_xl_w2048"
            rec = run_workload(sub, name)
            for k in ("metric", "n_gpus", "higher_is_better", "scaling", "vs_baseline", "data", "source_hash",
                      "gpu_clocks"):
                rec.pop(k, None)
            out["sub_records"][name] = rec
    print(json.dumps(out), flush=True)
    return 0


def run_workload(args, name):
    """Benchmark one workload; returns its record (None in --profile-op mode)."""
    from spatially_sharded_cnn_amd import workloads
    wl = workloads.WORKLOADS[name]
    a = argparse.Namespace(**vars(args))
    a.workload = name
    stack = wl.kind == "conv" and len(wl.layers) > 1
    if a.steps is None:
        a.steps = STACK_STEPS if stack else (20 if wl.kind == "block" else STEPS_DEFAULT)
    if a.warmup is None:
        a.warmup = STACK_WARMUP if stack else WARMUP_DEFAULT
    if wl.kind == "block":
        return block_bench(a, wl)
    if wl.kind == "grid":
        return grid_bench(a, wl)
    if stack:
        return stack_bench(a, wl)
    return layer_bench(a, wl)


def layer_bench(args, wl):
    """One layer's step on the measured shard (see the module docstring)."""
    import torch
    from spatially_sharded_cnn_amd import sscnn, workloads

    dev = "cuda"
    L = wl.layers[0]
    S, s = wl.num_shards, wl.shard
    T = workloads.generate(wl)
    hsplit = wl.axis == 2           # Shard(2): the same step on a split along H (row halos)
    A = _HOps(sscnn) if hsplit else _WOps(sscnn)

    def shard_of(a, i):
        if hsplit:
            h = a.shape[2] // S
            return np.ascontiguousarray(a[:, :, i * h:(i + 1) * h, :])
        w = a.shape[3] // S
        return np.ascontiguousarray(a[:, :, :, i * w:(i + 1) * w])

    def conv_of(i):
        if hsplit:
            return sscnn.hconv_init(L.in_shape[0], L.ci, L.co, L.in_shape[2] // S, L.in_shape[3], L.k,
                                    L.stride, L.pad, L.groups, i, S)
        return sscnn.conv_init(L.in_shape[0], L.ci, L.co, L.in_shape[2], L.in_shape[3] // S, L.k,
                               L.stride, L.pad, L.groups, i, S)

    c = conv_of(s)
    left, right = s - 1 if s > 0 else None, s + 1 if s < S - 1 else None
    wt = torch.from_numpy(T.weights[0]).to(dev)
    b = torch.from_numpy(T.biases[0]).to(dev)
    nw, nb = int(np.prod(c.w_shape)), c.c_out

    def dev_of(a):
        return torch.from_numpy(a).to(dev)

    def grads():
        buf = torch.empty(nw + nb, device=dev)      # [gW | gB], reduced with one call
        return buf, buf[:nw].view(c.w_shape), buf[nw:]

    xs_h = {i: shard_of(T.x, i) for i in range(S)}
    gs_h = {i: shard_of(T.g, i) for i in range(S)}
    sets = []
    for _ in range(args.sets):
        gbuf, gw, gb = grads()
        st = dict(
            x=dev_of(xs_h[s]), g=dev_of(gs_h[s]),
            xl=dev_of(xs_h[left]) if left is not None else None,
            xr=dev_of(xs_h[right]) if right is not None else None,
            gl=dev_of(gs_h[left]) if left is not None else None,
            gr=dev_of(gs_h[right]) if right is not None else None,
            xh=torch.empty(c.halo_shape(sscnn.HALO_INPUT), device=dev),
            gh=torch.empty(c.halo_shape(sscnn.HALO_GRAD_OUTPUT), device=dev),
            y=torch.empty(c.y_shape, device=dev), dx=torch.empty(c.x_shape, device=dev),
            gbuf=gbuf, gw=gw, gb=gb, red=torch.empty(nw + nb, device=dev),
        )
        sets.append(st)
    ws = A.new_workspace(c)
    del xs_h, gs_h

    # The other shards' partial gradients (computed once, untimed): the step's
    # partial_reduce sums all four in shard order, this shard's fresh partial in its slot.
    others = {}
    for i in range(S):
        if i == s:
            continue
        ci_ = conv_of(i)
        xi, gi = dev_of(shard_of(T.x, i)), dev_of(shard_of(T.g, i))
        li = dev_of(shard_of(T.x, i - 1)) if i > 0 else None
        ri = dev_of(shard_of(T.x, i + 1)) if i < S - 1 else None
        xhi = torch.empty(ci_.halo_shape(sscnn.HALO_INPUT), device=dev)
        A.halo_gather(ci_, sscnn.HALO_INPUT, li, ri, xhi)
        gbuf, gw, gb = grads()
        A.conv_bwd_weight_partial(ci_, xi, xhi, gi, gw, gb, A.new_workspace(ci_))
        others[i] = gbuf
        del xi, gi, li, ri, xhi
    torch.cuda.synchronize()

    ops = {
        "halo_gather_x": lambda st: A.halo_gather(c, sscnn.HALO_INPUT, st["xl"], st["xr"], st["xh"]),
        "conv_fwd": lambda st: A.conv_fwd(c, st["x"], st["xh"], wt, b, st["y"]),
        "halo_gather_g": lambda st: A.halo_gather(c, sscnn.HALO_GRAD_OUTPUT, st["gl"], st["gr"], st["gh"]),
        "conv_bwd": lambda st: A.conv_bwd(c, st["x"], st["xh"], st["g"], st["gh"], wt, st["dx"],
                                          st["gw"], st["gb"], ws),
        "partial_reduce": lambda st: sscnn.partial_reduce(
            [st["gbuf"] if i == s else others[i] for i in range(S)], st["red"]),
    }
    # the same backward as two calls (timed on their own, not part of the step)
    extra_ops = {
        "conv_bwd_input": lambda st: A.conv_bwd_input(c, st["g"], st["gh"], wt, st["dx"]),
        "conv_bwd_weight_partial": lambda st: A.conv_bwd_weight_partial(
            c, st["x"], st["xh"], st["g"], st["gw"], st["gb"], ws),
    }

    def step(st):
        for f in ops.values():
            f(st)

    # A plain device copy of known size (untimed): the reference that calibrates
    # the FETCH_SIZE / WRITE_SIZE counters in a counter run of this command.
    cal_src = torch.empty(COPY_CAL_BYTES // 4, device=dev)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    torch.cuda.synchronize()
    del cal_src, cal_dst

    for i in range(args.warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()

    # Timed region: K steps, events at the ends only.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        step(sets[i % len(sets)])
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_per_step = e0.elapsed_time(e1) / args.steps

    spread = step_spread(lambda i: step(sets[i % len(sets)]), args.steps)

    # Each operation on its own: back-to-back calls between two events.
    op_us = {}
    for name, f in list(ops.items()) + list(extra_ops.items()):
        for i in range(OP_WARM_CALLS):
            f(sets[i % len(sets)])
        torch.cuda.synchronize()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        for i in range(args.op_reps):
            f(sets[i % len(sets)])
        a1.record()
        torch.cuda.synchronize()
        op_us[name] = 1e3 * a0.elapsed_time(a1) / args.op_reps

    split = None if (args.no_split or hsplit) else split_bench(args, c, sets, ops, wt, b, ws, op_us)

    # Algorithmic work.
    f4 = 4
    if hsplit:
        n, ci, h, wl_ = c.n, c.c_in, c.h_local, c.w
        co, ho, wol = c.c_out, c.h_out_local, c.w_out
        x_ext = n * ci * (h + c.halo_u + c.halo_d) * wl_ * f4
        g_ext = n * co * (ho + c.ghalo_u + c.ghalo_d) * wol * f4
        halo_x_b = 2 * n * ci * (c.halo_u + c.halo_d) * wl_ * f4
        halo_g_b = 2 * n * co * (c.ghalo_u + c.ghalo_d) * wol * f4
    else:
        n, ci, h, wl_ = c.n, c.c_in, c.h, c.w_local
        co, ho, wol = c.c_out, c.h_out, c.w_out_local
        x_ext = n * ci * h * (wl_ + c.halo_l + c.halo_r) * f4
        g_ext = n * co * ho * (wol + c.ghalo_l + c.ghalo_r) * f4
        halo_x_b = 2 * n * ci * h * (c.halo_l + c.halo_r) * f4
        halo_g_b = 2 * n * co * ho * (c.ghalo_l + c.ghalo_r) * f4
    x_b, y_b = n * ci * h * wl_ * f4, n * co * ho * wol * f4
    w_b, b_b = nw * f4, nb * f4
    red_b = (S + 1) * (w_b + b_b)
    bytes_fwd = x_ext + w_b + b_b + y_b
    bytes_bwd = g_ext + x_ext + w_b + x_b + w_b + b_b
    step_bytes = bytes_fwd + bytes_bwd + red_b
    flops_pass = 2 * (ci // c.groups) * c.k * c.k * n * co * ho * wol
    step_flops = 3 * flops_pass
    op_bytes = {
        "halo_gather_x": halo_x_b,
        "conv_fwd": x_ext + w_b + b_b + y_b,
        "halo_gather_g": halo_g_b,
        "conv_bwd": bytes_bwd,
        "partial_reduce": red_b,
        "conv_bwd_input": g_ext + w_b + x_b,
        "conv_bwd_weight_partial": x_ext + y_b + w_b + b_b,
    }
    op_flops = {"conv_fwd": flops_pass, "conv_bwd": 2 * flops_pass, "conv_bwd_input": flops_pass,
                "conv_bwd_weight_partial": flops_pass}
    step_ops = list(ops)
    dense = c.groups == 1 and min(c.c_in, c.c_out) >= 16
    compute_peak = MFMA_F32_PEAK_TFLOPS if dense else VALU_F32_PEAK_TFLOPS

    def roof_time(k):
        return max(op_bytes[k] / (HBM_PEAK_GBS * 1e9), op_flops.get(k, 0) / (compute_peak * 1e12))

    dom = max(step_ops, key=op_us.get)
    t_hbm = op_bytes[dom] / (HBM_PEAK_GBS * 1e9)
    t_cmp = op_flops.get(dom, 0) / (compute_peak * 1e12)
    if t_cmp > t_hbm:
        achieved = op_flops[dom] / (op_us[dom] * 1e-6) / 1e12
        roof = {"bound": "mfma" if dense else "alu", "achieved": round(achieved, 2),
                "peak": round(compute_peak, 1), "unit": "TFLOP/s"}
    else:
        achieved = op_bytes[dom] / (op_us[dom] * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    tr = recorded_traffic(wl.name)
    roof["traffic"] = (tr["fetch_bytes"] + tr["write_bytes"]) if tr and tr.get("op") == dom else None
    roof["op"] = dom
    roof["avg_us"] = round(op_us[dom], 2)
    roof["algorithmic_bytes"] = op_bytes[dom]
    roof["algorithmic_flops"] = op_flops.get(dom, 0)

    step_s = ms_per_step * 1e-3
    out = {
        "metric": METRIC, "value": round(step_bytes / step_s / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description, "shard": f"{s} of {S}",
                   "split_axis": "H" if hsplit else "W",
                   "shard_input": list(c.x_shape), "weight": list(c.w_shape),
                   "buffer_sets": args.sets},
        "tflops": round(step_flops / step_s / 1e12, 2),
        "step_bytes": step_bytes, "step_flops": step_flops,
        "hbm_roofline_frac": round(step_bytes / (HBM_PEAK_GBS * 1e9) / step_s, 4),
        "compute_roofline_frac": round(step_flops / (compute_peak * 1e12) / step_s, 4),
        "roofline_frac_step": round(sum(roof_time(k) for k in step_ops) / step_s, 4),
        "roofline": roof,
        "ops_us": {k: round(v, 2) for k, v in op_us.items()},
        "step_spread": spread,
        "split": split,
        "wall_s_timed": round(wall, 4),
        "gpu_clocks": gpu_clocks(),
        "source_hash": kernel_source_hash(),
    }
    if not args.no_cpu_baseline and not hsplit:
        out["cpu_baseline"] = cpu_baseline(wl, T, L, S, s)
    return out


class _WOps:
    """The step's calls for a split along W (Shard(3))."""
    def __init__(self, sscnn):
        self.halo_gather = sscnn.halo_gather
        self.conv_fwd = sscnn.conv_fwd
        self.conv_bwd = sscnn.conv_bwd
        self.conv_bwd_input = sscnn.conv_bwd_input
        self.conv_bwd_weight_partial = sscnn.conv_bwd_weight_partial
        self.new_workspace = sscnn.new_workspace


class _HOps:
    """The same calls for a split along H (Shard(2)): row halos."""
    def __init__(self, sscnn):
        self.halo_gather = sscnn.row_halo_gather
        self.conv_fwd = sscnn.hconv_fwd
        self.conv_bwd = sscnn.hconv_bwd
        self.conv_bwd_input = sscnn.hconv_bwd_input
        self.conv_bwd_weight_partial = sscnn.hconv_bwd_weight_partial
        self.new_workspace = sscnn.new_hworkspace


def split_bench(args, c, sets, ops, wt, b, ws, op_us):
    """The layer as an interior/edge split (kwkr.cn retelling, section 5.2):
    each split call timed on its own; the split step with every call on one
    stream; and the split step with the two halo gathers on a second stream,
    running beside the interior calls, which is what a multi-GPU run does
    with its halo exchange.  compute_cost is (interior + edge calls) over the
    monolithic conv_fwd + conv_bwd, minus one."""
    import torch
    from spatially_sharded_cnn_amd import sscnn

    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    sops = {
        "conv_fwd_interior": lambda st: sscnn.conv_fwd_interior(c, st["x"], wt, b, st["y"]),
        "conv_fwd_edge": lambda st: sscnn.conv_fwd_edge(c, st["xh"], wt, st["y"]),
        "conv_bwd_interior": lambda st: sscnn.conv_bwd_interior(c, st["x"], st["g"], wt, st["dx"], st["gw"],
                                                                st["gb"], ws),
        "conv_bwd_input_edge": lambda st: sscnn.conv_bwd_input_edge(c, st["gh"], wt, st["dx"]),
        "conv_bwd_weight_edge": lambda st: sscnn.conv_bwd_weight_edge(c, st["xh"], st["g"], st["gw"]),
    }

    def serial(st):
        ops["halo_gather_x"](st)
        sops["conv_fwd_interior"](st)
        sops["conv_fwd_edge"](st)
        ops["halo_gather_g"](st)
        sops["conv_bwd_interior"](st)
        sops["conv_bwd_input_edge"](st)
        sops["conv_bwd_weight_edge"](st)
        ops["partial_reduce"](st)

    def overlapped(st):
        start = torch.cuda.Event()
        start.record(main)
        side.wait_event(start)
        with torch.cuda.stream(side):
            ops["halo_gather_x"](st)
            x_ready = torch.cuda.Event()
            x_ready.record(side)
            ops["halo_gather_g"](st)
            g_ready = torch.cuda.Event()
            g_ready.record(side)
        sops["conv_fwd_interior"](st)
        main.wait_event(x_ready)
        sops["conv_fwd_edge"](st)
        sops["conv_bwd_interior"](st)
        main.wait_event(g_ready)
        sops["conv_bwd_input_edge"](st)
        sops["conv_bwd_weight_edge"](st)
        ops["partial_reduce"](st)

    def timed(step, reps):
        for i in range(args.warmup):
            step(sets[i % len(sets)])
        torch.cuda.synchronize()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        for i in range(reps):
            step(sets[i % len(sets)])
        a1.record()
        torch.cuda.synchronize()
        return 1e3 * a0.elapsed_time(a1) / reps

    sus = {name: round(timed(f, args.op_reps), 2) for name, f in sops.items()}
    split_us = sum(sus.values())
    mono_us = op_us["conv_fwd"] + op_us["conv_bwd"]
    return {"ops_us": sus,
            "step_us_serial": round(timed(serial, args.steps), 2),
            "step_us_overlapped": round(timed(overlapped, args.steps), 2),
            "compute_cost": round(split_us / mono_us - 1.0, 4)}


def _layer_work(c, L):
    """Algorithmic bytes and FLOPs of one layer's forward, backward (grad_input +
    grad_weight/grad_bias partial) and partial reduction, for one shard."""
    f4 = 4
    n, ci, h, wl_ = c.n, c.c_in, c.h, c.w_local
    co, ho, wol = c.c_out, c.h_out, c.w_out_local
    x_ext = n * ci * h * (wl_ + c.halo_l + c.halo_r) * f4
    g_ext = n * co * ho * (wol + c.ghalo_l + c.ghalo_r) * f4
    x_b, y_b = n * ci * h * wl_ * f4, n * co * ho * wol * f4
    w_b, b_b = co * (ci // c.groups) * c.k * c.k * f4, co * f4
    flops = 2 * (ci // c.groups) * c.k * c.k * n * co * ho * wol
    return {"fwd": (x_ext + w_b + b_b + y_b, flops),
            "bwd": (g_ext + x_ext + w_b + x_b + w_b + b_b, 2 * flops),
            "reduce": ((c.num_shards + 1) * (w_b + b_b), 0),
            "halo_x": (2 * n * ci * h * (c.halo_l + c.halo_r) * f4, 0),
            "halo_g": (2 * n * co * ho * (c.ghalo_l + c.ghalo_r) * f4, 0)}


def grid_bench(args, wl):
    """2-D H x W shards on a 2 x 2 grid: one step is the measured block's
    row-then-column halo exchange of its input, its forward, the same exchange
    of its grad_output, its backward and the reduction of the four blocks'
    partials.  The neighbours' blocks and their phase-1 row halos (which carry
    the corners) are prepared untimed; so are the other blocks' partials."""
    import torch
    from spatially_sharded_cnn_amd import sscnn, workloads

    dev = "cuda"
    L = wl.layers[0]
    NH = NW = 2
    bi, bj = divmod(wl.shard, NW)
    T = workloads.generate(wl)
    n, C, H, W = L.in_shape
    bh, bw = H // NH, W // NW
    blocks = [(i, j) for i in range(NH) for j in range(NW)]
    cv = {ij: sscnn.gconv_init(n, L.ci, L.co, bh, bw, L.k, L.stride, L.pad, L.groups, ij[0], NH, ij[1], NW)
          for ij in blocks}
    blk = lambda a, i, j: torch.from_numpy(np.ascontiguousarray(a[:, :, i * bh:(i + 1) * bh, j * bw:(j + 1) * bw])).to(dev)
    X = {ij: blk(T.x, *ij) for ij in blocks}
    G = {ij: blk(T.g, *ij) for ij in blocks}
    wt, b = torch.from_numpy(T.weights[0]).to(dev), torch.from_numpy(T.biases[0]).to(dev)
    c = cv[bi, bj]
    e = lambda shape: torch.empty(shape, device=dev)
    RX = {ij: e(cv[ij].row_halo_shape(sscnn.HALO_INPUT)) for ij in blocks}
    RG = {ij: e(cv[ij].row_halo_shape(sscnn.HALO_GRAD_OUTPUT)) for ij in blocks}
    nb = lambda d, i, j: d.get((i, j))
    for (i, j) in blocks:       # phase 1 everywhere (the neighbours' row halos are phase 2's input)
        sscnn.grid_row_halo_gather(cv[i, j], sscnn.HALO_INPUT, nb(X, i - 1, j), nb(X, i + 1, j), RX[i, j])
        sscnn.grid_row_halo_gather(cv[i, j], sscnn.HALO_GRAD_OUTPUT, nb(G, i - 1, j), nb(G, i + 1, j), RG[i, j])
    cx, cg = e(c.col_halo_shape(sscnn.HALO_INPUT)), e(c.col_halo_shape(sscnn.HALO_GRAD_OUTPUT))
    y, dx = e(c.y_shape), e(c.x_shape)
    nw_ = int(np.prod(c.w_shape))
    parts = [e((nw_ + c.c_out,)).normal_() for _ in blocks]
    me = blocks.index((bi, bj))
    gw, gb = parts[me][:nw_].view(c.w_shape), parts[me][nw_:]
    red = e((nw_ + c.c_out,))
    ws = sscnn.new_gworkspace(c)
    i, j = bi, bj
    ops = [
        ("row_halo_x", lambda: sscnn.grid_row_halo_gather(c, sscnn.HALO_INPUT, nb(X, i - 1, j), nb(X, i + 1, j),
                                                          RX[i, j])),
        ("col_halo_x", lambda: sscnn.grid_col_halo_gather(c, sscnn.HALO_INPUT, nb(X, i, j - 1), nb(RX, i, j - 1),
                                                          nb(X, i, j + 1), nb(RX, i, j + 1), cx)),
        ("conv_fwd", lambda: sscnn.gconv_fwd(c, X[i, j], RX[i, j], cx, wt, b, y)),
        ("row_halo_g", lambda: sscnn.grid_row_halo_gather(c, sscnn.HALO_GRAD_OUTPUT, nb(G, i - 1, j),
                                                          nb(G, i + 1, j), RG[i, j])),
        ("col_halo_g", lambda: sscnn.grid_col_halo_gather(c, sscnn.HALO_GRAD_OUTPUT, nb(G, i, j - 1),
                                                          nb(RG, i, j - 1), nb(G, i, j + 1), nb(RG, i, j + 1), cg)),
        ("conv_bwd", lambda: sscnn.gconv_bwd(c, X[i, j], RX[i, j], cx, G[i, j], RG[i, j], cg, wt, dx, gw, gb, ws)),
        ("partial_reduce", lambda: sscnn.partial_reduce(parts, red)),
    ]

    def step():
        for _, f in ops:
            f()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_per_step = e0.elapsed_time(e1) / args.steps
    spread = step_spread(lambda k: step(), args.steps)
    op_us = {}
    for name, f in ops:
        for _ in range(OP_WARM_CALLS):
            f()
        torch.cuda.synchronize()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        for _ in range(args.op_reps):
            f()
        a1.record()
        torch.cuda.synchronize()
        op_us[name] = round(1e3 * a0.elapsed_time(a1) / args.op_reps, 2)

    f4, hh = 4, c.halo
    x_ext = n * C * (bh + 2 * hh) * (bw + 2 * hh) * f4
    x_b = n * C * bh * bw * f4
    w_b, b_b = int(np.prod(c.w_shape)) * f4, c.c_out * f4
    flops = 2 * (L.ci // L.groups) * L.k * L.k * n * L.co * bh * bw
    work = {"conv_fwd": (x_ext + w_b + b_b + x_b, flops),
            "conv_bwd": (2 * x_ext + w_b + x_b + w_b + b_b, 2 * flops),
            "partial_reduce": ((len(blocks) + 1) * (w_b + b_b), 0)}
    step_bytes = sum(v[0] for v in work.values())
    step_flops = sum(v[1] for v in work.values())
    t = op_us["conv_bwd"]
    bb, ff = work["conv_bwd"]
    dense = L.groups == 1 and min(L.ci, L.co) >= 16
    peak = MFMA_F32_PEAK_TFLOPS if dense else VALU_F32_PEAK_TFLOPS
    if ff / (peak * 1e12) > bb / (HBM_PEAK_GBS * 1e9):
        roof = {"bound": "mfma" if dense else "alu", "achieved": round(ff / (t * 1e-6) / 1e12, 2), "peak": peak,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(bb / (t * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof.update(frac=round(roof["achieved"] / roof["peak"], 4), traffic=None, op="conv_bwd", avg_us=t,
                algorithmic_bytes=bb, algorithmic_flops=ff)
    step_s = ms_per_step * 1e-3
    out = {
        "metric": METRIC, "value": round(step_bytes / step_s / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description, "block": [bi, bj], "grid": [NH, NW],
                   "shard_input": list(c.x_shape)},
        "tflops": round(step_flops / step_s / 1e12, 2), "step_bytes": step_bytes, "step_flops": step_flops,
        "hbm_roofline_frac": round(step_bytes / step_s / 1e9 / HBM_PEAK_GBS, 4),
        "compute_roofline_frac": round(step_flops / (peak * 1e12) / step_s, 4), "roofline": roof,
        "ops_us": op_us, "step_spread": spread, "wall_s_timed": round(wall, 4), "gpu_clocks": gpu_clocks(),
        "source_hash": kernel_source_hash(),
    }
    return out


def block_bench(args, wl):
    """A ConvNeXt block on the measured shard (the depthwise, LayerNorm, 1x1,
    GELU, 1x1, layer scale + DropPath + residual steps): one step is its
    forward and its backward, each weight gradient reduced over the shards
    like the convolutions'.  The neighbours' slices come from the global input
    (and, for the grad_output halo of the depthwise layer, from a synthetic
    gradient of the same shape); the other shards' partials are synthetic."""
    import torch
    from spatially_sharded_cnn_amd import sscnn, workloads

    dev = "cuda"
    S, s = wl.num_shards, wl.shard
    steps = args.steps
    warmup = args.warmup
    T = workloads.generate(wl)
    dw, pw1, pw2 = wl.layers
    n, C, H, Wg = dw.in_shape
    wl_ = Wg // S
    P = H * wl_
    keep = 0.9
    rng = np.random.default_rng(wl.seed + 1)

    def dev_t(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    def slices(a):
        return [dev_t(a[..., i * wl_:(i + 1) * wl_]) for i in range(S)]

    xs = slices(T.x)
    g_dw_nbrs = slices(rng.standard_normal(T.x.shape).astype(np.float32))   # grad at the dw output, neighbours
    gout = slices(T.g)[s]
    convs = [sscnn.conv_init(n, L.ci, L.co, H, wl_, L.k, L.stride, L.pad, L.groups, s, S) for L in wl.layers]
    cdw, c1, c2 = convs
    wts = [dev_t(w) for w in T.weights]
    bss = [dev_t(b) for b in T.biases]
    ln_w, ln_b = dev_t(1 + 0.02 * rng.standard_normal(C)), dev_t(0.02 * rng.standard_normal(C))
    gamma = dev_t(np.full(C, 1e-6))
    nbr = lambda lst: (lst[s - 1] if s > 0 else None, lst[s + 1] if s < S - 1 else None)
    e = lambda shape: torch.empty(shape, device=dev)
    x = xs[s]
    xh, y_dw, y_ln = e(cdw.halo_shape(sscnn.HALO_INPUT)), e(cdw.y_shape), e(cdw.y_shape)
    mean, rstd = e((n, H, wl_)), e((n, H, wl_))
    y1, a1, y2, scales, out = e(c1.y_shape), e(c1.y_shape), e(c2.y_shape), e((n,)), e(c2.y_shape)
    dh2, da1, dy1 = e(c2.y_shape), e(c1.y_shape), e(c1.y_shape)
    dln, ddw, dx = e(cdw.y_shape), e(cdw.y_shape), e(cdw.x_shape)
    gh = e(cdw.halo_shape(sscnn.HALO_GRAD_OUTPUT))
    parts = {name: [e((cnt,)) for _ in range(S)] for name, cnt in
             (("gamma", C), ("pw2", int(np.prod(c2.w_shape)) + c2.c_out), ("pw1", int(np.prod(c1.w_shape)) + c1.c_out),
              ("ln", 2 * C), ("dw", int(np.prod(cdw.w_shape)) + cdw.c_out))}
    for lst in parts.values():
        for t in lst:
            t.normal_()
    reds = {k: e(v[0].shape) for k, v in parts.items()}
    ws = {k: sscnn.new_workspace(c) for k, c in (("dw", cdw), ("pw1", c1), ("pw2", c2))}

    def wparts(name, c):
        t = parts[name][s]
        nw = int(np.prod(c.w_shape))
        return t[:nw].view(c.w_shape), t[nw:]

    f4 = 4
    act, act4 = n * C * P * f4, n * 4 * C * P * f4
    wk = {k: _layer_work(c, L) for k, c, L in (("dw", cdw, dw), ("pw1", c1, pw1), ("pw2", c2, pw2))}
    red_b = lambda name: ((S + 1) * parts[name][0].numel() * f4, 0)
    # (name, call, algorithmic bytes, flops, dense)
    ops = [
        ("dw.halo_x", lambda: sscnn.halo_gather(cdw, sscnn.HALO_INPUT, *nbr(xs), xh), *wk["dw"]["halo_x"], False),
        ("dw.fwd", lambda: sscnn.conv_fwd(cdw, x, xh, wts[0], bss[0], y_dw), *wk["dw"]["fwd"], False),
        ("ln.fwd", lambda: sscnn.layernorm_fwd(y_dw, ln_w, ln_b, y_ln, mean, rstd), 2 * act + 2 * n * P * f4, 0,
         False),
        # pw1 with GELU in its epilogue: y1 (pre-activation, kept for the backward) and a1 = GELU(y1)
        ("pw1.fwd_gelu", lambda: sscnn.pointwise_gelu_fwd(c1, y_ln, wts[1], bss[1], y1, a1),
         wk["pw1"]["fwd"][0] + act4, wk["pw1"]["fwd"][1], True),
        ("pw2.fwd", lambda: sscnn.conv_fwd(c2, a1, None, wts[2], bss[2], y2), *wk["pw2"]["fwd"], True),
        ("droppath", lambda: sscnn.droppath_scales(wl.seed, 0, keep, scales), n * f4, 0, False),
        ("scale.fwd", lambda: sscnn.layer_scale_residual_fwd(x, y2, gamma, scales, out), 3 * act, 0, False),
        ("scale.bwd", lambda: sscnn.layer_scale_residual_bwd(y2, gout, gamma, scales, dh2, parts["gamma"][s]),
         3 * act, 0, False),
        ("scale.reduce", lambda: sscnn.partial_reduce(parts["gamma"], reds["gamma"]), *red_b("gamma"), False),
        # (the fused sscnn_pointwise_bwd_input_gelu measured slower than these two passes)
        ("pw2.bwd", lambda: sscnn.conv_bwd(c2, a1, None, dh2, None, wts[2], da1, *wparts("pw2", c2), ws["pw2"]),
         *wk["pw2"]["bwd"], True),
        ("pw2.reduce", lambda: sscnn.partial_reduce(parts["pw2"], reds["pw2"]), *red_b("pw2"), False),
        ("gelu.bwd", lambda: sscnn.gelu_bwd(y1, da1, dy1), 3 * act4, 0, False),
        ("pw1.bwd", lambda: sscnn.conv_bwd(c1, y_ln, None, dy1, None, wts[1], dln, *wparts("pw1", c1), ws["pw1"]),
         *wk["pw1"]["bwd"], True),
        ("pw1.reduce", lambda: sscnn.partial_reduce(parts["pw1"], reds["pw1"]), *red_b("pw1"), False),
        ("ln.bwd", lambda: sscnn.layernorm_bwd(y_dw, dln, ln_w, mean, rstd, ddw, parts["ln"][s][:C],
                                               parts["ln"][s][C:]), 3 * act + 2 * n * P * f4, 0, False),
        ("ln.reduce", lambda: sscnn.partial_reduce(parts["ln"], reds["ln"]), *red_b("ln"), False),
        ("dw.halo_g", lambda: sscnn.halo_gather(cdw, sscnn.HALO_GRAD_OUTPUT, *nbr(g_dw_nbrs), gh),
         *wk["dw"]["halo_g"], False),
        ("dw.bwd", lambda: sscnn.conv_bwd(cdw, x, xh, ddw, gh, wts[0], dx, *wparts("dw", cdw), ws["dw"]),
         *wk["dw"]["bwd"], False),
        ("dw.reduce", lambda: sscnn.partial_reduce(parts["dw"], reds["dw"]), *red_b("dw"), False),
    ]

    def step():
        for op in ops:
            op[1]()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_per_step = e0.elapsed_time(e1) / steps
    spread = step_spread(lambda i: step(), steps)

    rows, step_bytes, step_flops, dom = [], 0, 0, None
    for name, f, b_, f_, dense in ops:
        for _ in range(OP_WARM_CALLS):
            f()
        torch.cuda.synchronize()
        reps = max(2, min(args.op_reps, 20))
        a0, a1_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        for _ in range(reps):
            f()
        a1_.record()
        torch.cuda.synchronize()
        t = 1e3 * a0.elapsed_time(a1_) / reps
        peak = MFMA_F32_PEAK_TFLOPS if dense else VALU_F32_PEAK_TFLOPS
        t_mem, t_fl = b_ / (HBM_PEAK_GBS * 1e9), f_ / (peak * 1e12)
        bound = ("mfma" if dense else "alu") if t_fl > t_mem else "hbm"
        row = {"op": name, "us": round(t, 2), "bound": bound,
               "gbs": round(b_ / (t * 1e-6) / 1e9, 1), "tflops": round(f_ / (t * 1e-6) / 1e12, 2),
               "roofline_frac": round(max(t_mem, t_fl) / (t * 1e-6), 4)}
        rows.append(row)
        if not name.endswith(("halo_x", "halo_g")):
            step_bytes += b_
            step_flops += f_
        if dom is None or t > dom[1]:
            dom = (name, t, b_, f_, dense, bound)
    name, t, b_, f_, dense, bound = dom
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(b_ / (t * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        peak = MFMA_F32_PEAK_TFLOPS if dense else VALU_F32_PEAK_TFLOPS
        roof = {"bound": bound, "achieved": round(f_ / (t * 1e-6) / 1e12, 2), "peak": peak, "unit": "TFLOP/s"}
    roof.update(frac=round(roof["achieved"] / roof["peak"], 4), traffic=None, op=name, avg_us=round(t, 2),
                algorithmic_bytes=b_, algorithmic_flops=f_)
    step_s = ms_per_step * 1e-3
    out_d = {
        "metric": METRIC, "value": round(step_bytes / step_s / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description, "shard": f"{s} of {S}",
                   "shard_input": list(cdw.x_shape), "drop_path": round(1 - keep, 3)},
        "tflops": round(step_flops / step_s / 1e12, 2), "step_bytes": step_bytes, "step_flops": step_flops,
        "roofline": roof, "ops": rows, "step_spread": spread, "wall_s_timed": round(wall, 4),
        "gpu_clocks": gpu_clocks(), "source_hash": kernel_source_hash(),
    }
    return out_d


def stack_bench(args, wl):
    """A ConvNeXt-style stack (on (7,3,512,2048) or (7,3,512,4096) inputs): one step is the
    measured shard's forward chain (halo_gather + conv_fwd per layer, each
    layer's output feeding the next), its backward chain in reverse
    (halo_gather(G) + conv_bwd per layer, each grad_input feeding the layer
    below, each layer's grad_weight / grad_bias partials written into the
    shard's gradient bucket), and one partial_reduce of the four shards'
    buckets.  A stem or downsample followed by a layer with a halo pushes that
    halo from its epilogue (conv_fwd_push / conv_bwd_push) instead of the
    consumer gathering it.  The neighbours' activations and gradients and the other shards'
    buckets come from an untimed run of all shards."""
    import torch
    from spatially_sharded_cnn_amd import sscnn, workloads
    from spatially_sharded_cnn_amd.stack import ShardedStack

    dev = "cuda"
    S, s = wl.num_shards, wl.shard
    steps, warmup = args.steps, args.warmup
    T = workloads.generate(wl)

    def slices(a):
        w = a.shape[3] // S
        return [torch.from_numpy(np.ascontiguousarray(a[:, :, :, i * w:(i + 1) * w])).to(dev) for i in range(S)]

    xs, gs = slices(T.x), slices(T.g)
    st = ShardedStack(wl.layers, S, T.weights, T.biases, push=not args.no_push)
    st.forward(xs)
    st.backward(gs)
    torch.cuda.synchronize()
    nl = len(wl.layers)
    convs = [st.state[l].convs[s] for l in range(nl)]
    nbr = lambda lst: (lst[s - 1] if s > 0 else None, lst[s + 1] if s < S - 1 else None)
    ys = [torch.empty(c.y_shape, device=dev) for c in convs]
    dxs = [torch.empty(c.x_shape, device=dev) for c in convs]
    xhs = [torch.empty(c.halo_shape(sscnn.HALO_INPUT), device=dev) if c.halo_l + c.halo_r else None for c in convs]
    ghs = [torch.empty(c.halo_shape(sscnn.HALO_GRAD_OUTPUT), device=dev) if c.ghalo_l + c.ghalo_r else None
           for c in convs]
    offs, total = st.offsets
    bucket = torch.zeros(total, device=dev)       # this shard's partials of every layer
    reduced = torch.zeros(total, device=dev)
    gws = [bucket[offs[l][0]:offs[l][0] + offs[l][2]].view(c.w_shape) for l, c in enumerate(convs)]
    gbs = [bucket[offs[l][1]:offs[l][1] + offs[l][3]] for l in range(nl)]
    wss = [sscnn.new_workspace(c) for c in convs]
    ins = [xs[s]] + ys[:-1]                       # each layer's input: the previous layer's output
    gouts = dxs[1:] + [gs[s]]                     # each layer's grad_output: the next layer's grad_input
    # Push-form halos (a stem / downsample writing the next layer's halos from its epilogue): this
    # shard's step pushes into its neighbours' halo buffers (those of the untimed all-shard run); its
    # own halos, which its neighbours push, are copied from that run once, before timing.
    fpush = [st.pushes_forward(l) for l in range(nl)]
    bpush = [st.pushes_backward(l) for l in range(nl)]
    for l in range(nl):
        if fpush[l]:
            xhs[l + 1].copy_(st.state[l + 1].x_halo[s])
        if bpush[l]:
            ghs[l - 1].copy_(st.state[l - 1].g_halo[s])
    torch.cuda.synchronize()

    def fwd_push(l):
        lft, rgt = nbr(st.state[l + 1].x_halo)
        return sscnn.make_push(convs[l + 1], sscnn.HALO_INPUT, lft, rgt, xhs[l + 1])

    def bwd_push(l):
        lft, rgt = nbr(st.state[l - 1].g_halo)
        return sscnn.make_push(convs[l - 1], sscnn.HALO_GRAD_OUTPUT, lft, rgt, ghs[l - 1])

    def op_list():
        ops = []
        for l, c in enumerate(convs):
            if xhs[l] is not None and not (l > 0 and fpush[l - 1]):
                ops.append((l, "halo_x", lambda l=l, c=c: sscnn.halo_gather(
                    c, sscnn.HALO_INPUT, *nbr(st.state[l].x), xhs[l])))
            if fpush[l]:
                p = fwd_push(l)
                ops.append((l, "fwd", lambda l=l, c=c, p=p: sscnn.conv_fwd_push(
                    c, ins[l], xhs[l], st.w[l], st.b[l], ys[l], p)))
            else:
                ops.append((l, "fwd", lambda l=l, c=c: sscnn.conv_fwd(c, ins[l], xhs[l], st.w[l], st.b[l],
                                                                      ys[l])))
        for l in range(nl - 1, -1, -1):
            c = convs[l]
            if ghs[l] is not None and not (l + 1 < nl and bpush[l + 1]):
                ops.append((l, "halo_g", lambda l=l, c=c: sscnn.halo_gather(
                    c, sscnn.HALO_GRAD_OUTPUT, *nbr(st.state[l].g), ghs[l])))
            if bpush[l]:
                p = bwd_push(l)
                ops.append((l, "bwd", lambda l=l, c=c, p=p: sscnn.conv_bwd_push(
                    c, ins[l], xhs[l], gouts[l], ghs[l], st.w[l], dxs[l], gws[l], gbs[l], p, wss[l])))
            else:
                ops.append((l, "bwd", lambda l=l, c=c: sscnn.conv_bwd(
                    c, ins[l], xhs[l], gouts[l], ghs[l], st.w[l], dxs[l], gws[l], gbs[l], wss[l])))
        ops.append((-1, "reduce", lambda: sscnn.partial_reduce(
            [bucket if i == s else st.buckets[i] for i in range(S)], reduced)))
        return ops

    ops = op_list()

    def step():
        for _, _, f in ops:
            f()

    # A plain device copy of known size (untimed): the reference that calibrates
    # the FETCH_SIZE / WRITE_SIZE counters in a counter run of this command.
    cal_src = torch.empty(COPY_CAL_BYTES // 4, device=dev)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    torch.cuda.synchronize()
    del cal_src, cal_dst

    if args.profile_op:
        # Counter runs of one operation: its launches are the dispatches after
        # the calibration copy just made (bench.py --summarize --after-calibration).
        sel = [(l, name, f) for l, name, f in ops if (l >= 0 and (f"{wl.layers[l].name}.conv_{name}" == args.profile_op
               or f"{wl.layers[l].name}.{name}" == args.profile_op)) or (l < 0 and name == args.profile_op)]
        if not sel:
            raise SystemExit(f"--profile-op {args.profile_op}: no such operation (layer.conv_fwd, "
                             "layer.conv_bwd, layer.halo_x, layer.halo_g, reduce)")
        f = sel[0][2]
        for _ in range(args.profile_reps):
            f()
        torch.cuda.synchronize()
        print(json.dumps({"profile_op": args.profile_op, "reps": args.profile_reps, "workload": wl.name}),
              flush=True)
        return None

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_per_step = e0.elapsed_time(e1) / steps

    spread = step_spread(lambda i: step(), steps)

    # each operation on its own, back to back
    op_us = {}
    for l, name, f in ops:
        for _ in range(OP_WARM_CALLS):
            f()
        torch.cuda.synchronize()
        reps = max(2, min(args.op_reps, 20))
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        for _ in range(reps):
            f()
        a1.record()
        torch.cuda.synchronize()
        op_us[(l, name)] = 1e3 * a0.elapsed_time(a1) / reps

    layers = []
    step_bytes = step_flops = 0
    dom, dom_t = None, -1.0
    for l, (L, c) in enumerate(zip(wl.layers, convs)):
        work = _layer_work(c, L)
        dense = c.groups == 1
        peak = MFMA_F32_PEAK_TFLOPS if dense else VALU_F32_PEAK_TFLOPS
        row = {"layer": L.name, "shard_input": list(c.x_shape), "k": c.k, "stride": c.stride,
               "groups": c.groups, "bound_unit": "mfma" if dense else "alu"}
        lay_t = lay_roof = 0.0
        for name in ("halo_x", "fwd", "halo_g", "bwd"):
            if (l, name) not in op_us:
                continue
            b_, f_ = work[name]
            t = op_us[(l, name)]
            row[name + "_us"] = round(t, 2)
            lay_t += t
            if name in ("fwd", "bwd"):
                step_bytes += b_
                step_flops += f_
            lay_roof += max(b_ / (HBM_PEAK_GBS * 1e9), f_ / (peak * 1e12)) * 1e6
            if name in ("fwd", "bwd") and t > dom_t:
                dom, dom_t = (l, name, b_, f_, dense, peak), t
        row["us"] = round(lay_t, 2)
        row["roofline_us"] = round(lay_roof, 2)
        row["roofline_frac"] = round(lay_roof / lay_t, 4) if lay_t else None
        row["gbs"] = round((work["fwd"][0] + work["bwd"][0]) / (lay_t * 1e-6) / 1e9, 1)
        row["tflops"] = round((work["fwd"][1] + work["bwd"][1]) / (lay_t * 1e-6) / 1e12, 2)
        layers.append(row)

    # the bucketed reduction of every layer's partials, once per step
    red_bytes = (S + 1) * total * 4
    red_t = op_us[(-1, "reduce")]
    red_roof_us = red_bytes / (HBM_PEAK_GBS * 1e9) * 1e6
    step_bytes += red_bytes
    bucket_reduce = {"us": round(red_t, 2), "bucket_floats": total, "algorithmic_bytes": red_bytes,
                     "gbs": round(red_bytes / (red_t * 1e-6) / 1e9, 1), "roofline_us": round(red_roof_us, 2),
                     "roofline_frac": round(red_roof_us / red_t, 4)}

    l, name, b_, f_, dense, peak = dom
    t = op_us[(l, name)]
    if f_ / (peak * 1e12) > b_ / (HBM_PEAK_GBS * 1e9):
        roof = {"bound": "mfma" if dense else "alu", "achieved": round(f_ / (t * 1e-6) / 1e12, 2),
                "peak": peak, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(b_ / (t * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["op"] = f"{wl.layers[l].name}.conv_{name}"
    tr = recorded_traffic(wl.name)
    roof["traffic"] = (tr["fetch_bytes"] + tr["write_bytes"]) if tr and tr.get("op") == roof["op"] else None
    roof["avg_us"] = round(t, 2)
    roof["algorithmic_bytes"] = b_
    roof["algorithmic_flops"] = f_

    step_s = ms_per_step * 1e-3
    out = {
        "metric": METRIC, "value": round(step_bytes / step_s / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description, "shard": f"{s} of {S}",
                   "shard_input": list(convs[0].x_shape), "layers": len(convs),
                   "halos": "gathered" if args.no_push else "pushed where the layer before is a stem or downsample"},
        "tflops": round(step_flops / step_s / 1e12, 2),
        "step_bytes": step_bytes, "step_flops": step_flops,
        "roofline_frac_step": round((sum(r["roofline_us"] for r in layers) + red_roof_us) * 1e-6 / step_s, 4),
        "roofline": roof,
        "layers": layers,
        "bucket_reduce": bucket_reduce,
        "step_spread": spread,
        "wall_s_timed": round(wall, 4),
        "gpu_clocks": gpu_clocks(),
        "source_hash": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_stack(wl, convs, step_flops)
    return out


def cpu_baseline_stack(wl, convs, step_flops):
    """The oracle on the stack's layers for the measured shard, each layer on
    seeded tensors of its own shapes (the cost does not depend on values),
    over the first `imgs` images: forward + grad_input + grad_weight/grad_bias
    partial per layer.  imgs is chosen for roughly 10-20 s of host work."""
    import oracle
    S, s = wl.num_shards, wl.shard
    n = wl.layers[0].in_shape[0]
    imgs = max(1, min(n, int(round(n * 12.0 / max(step_flops / 30e9, 1e-9)))))
    rng = np.random.default_rng(7)
    total_t = total_b = 0.0
    for L, c in zip(wl.layers, convs):
        _, ci, h, w = L.in_shape
        _, co, ho, wo = L.out_shape
        x = rng.standard_normal((imgs, ci, h, w), dtype=np.float32)
        g = rng.standard_normal((imgs, co, ho, wo), dtype=np.float32)
        wt = rng.standard_normal((co, ci // L.groups, L.k, L.k), dtype=np.float32)
        b = rng.standard_normal((co,), dtype=np.float32)
        wl_, wol = w // S, wo // S
        t0 = time.perf_counter()
        oracle.conv_fwd(x, wt, b, L.stride, L.pad, L.groups, cols=(s * wol, (s + 1) * wol))
        oracle.conv_bwd_input(g, wt, x.shape, L.stride, L.pad, L.groups, cols=(s * wl_, (s + 1) * wl_))
        oracle.conv_bwd_weight(x, g, L.k, L.stride, L.pad, L.groups, cols=(s * wol, (s + 1) * wol))
        total_t += time.perf_counter() - t0
        work = _layer_work(c, L)
        total_b += (work["fwd"][0] + work["bwd"][0]) * imgs / n
    return {"value": round(total_b / total_t / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": round(total_t, 3),
            "sample": f"images 0..{imgs - 1} of {n}, every layer of the stack, shard {s} of {S}: forward + "
                      "grad_input + grad_weight/grad_bias partial per layer (C, double, OpenMP)",
            "cpu": platform.processor() or platform.machine()}


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


def summarize(dirs, traffic_op=None, traffic_kernels=None, after_cal=False):
    """Text summary of rocprofv3 output directories (kernel stats, kernel
    traces and/or counter collection CSVs), for the files committed under
    profiles/.

    Kernel traces are also grouped by kernel and grid size, which tells apart
    the launches of one kernel template for layers of different shapes.

    With traffic_op / traffic_kernels (semicolon-separated substrings of the
    operation's kernel names): the operation's per-launch figures.  With
    after_cal they come only from the dispatches after the last device copy
    -- in a `bench.py --profile-op OP` run, the calibration copy made just
    before the operation's repetitions.  From a kernel trace: the operation's kernels, grids and mean
    durations.  From FETCH_SIZE / WRITE_SIZE counter runs: the HBM traffic per
    launch -- each counter's KB per dispatch, scaled by what the same counter
    reads for the plain device copy of COPY_CAL_BYTES each way that the
    command runs (`__amd_rocclr_copyBuffer`), summed over the operation's
    kernels -- as a `traffic_json:` line that bench.py reads back while the
    sources match."""
    stats, cc, kt = [], [], []
    for d in dirs:
        d = pathlib.Path(d)
        stats += sorted(glob.glob(str(d / "**" / "*kernel_stats.csv"), recursive=True))
        cc += sorted(glob.glob(str(d / "**" / "*counter_collection.csv"), recursive=True))
        kt += sorted(glob.glob(str(d / "**" / "*kernel_trace.csv"), recursive=True))
    subs = [t for t in (traffic_kernels or "").split(";") if t]

    def picks(name):
        return any(t in name for t in subs)

    def after_marker(rows):
        """Rows (sorted by dispatch) after the last device copy, if after_cal."""
        if not after_cal:
            return rows
        marks = [i for i, r in enumerate(rows) if "copyBuffer" in r["Kernel_Name"]]
        return rows[marks[-1] + 1:] if marks else rows

    for f in stats:
        print(f"## kernel statistics ({pathlib.Path(f).name})\n")
        print("| kernel | calls | average us | min us | max us | share |")
        print("|---|---:|---:|---:|---:|---:|")
        for r in csv.DictReader(open(f)):
            print(f"| `{r['Name'][:110]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                  f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
        print()
    for f in kt:
        rows = list(csv.DictReader(open(f)))
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        groups = {}
        for r in rows:
            grid = tuple(int(r[f"Grid_Size_{a}"]) for a in "XYZ")
            wg = tuple(int(r[f"Workgroup_Size_{a}"]) for a in "XYZ")
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            groups.setdefault((r["Kernel_Name"], grid, wg), []).append(dur)
        print(f"## kernel trace by kernel and launch shape ({pathlib.Path(f).name})\n")
        print("| kernel | workgroups | threads | calls | average us | min us | max us |")
        print("|---|---:|---:|---:|---:|---:|---:|")
        for (kname, grid, wg), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
            nwg = (grid[0] // max(1, wg[0])) * (grid[1] // max(1, wg[1])) * (grid[2] // max(1, wg[2]))
            print(f"| `{kname[:100]}` | {nwg} | {wg[0] * wg[1] * wg[2]} | {len(v)} | {sum(v) / len(v):.2f} | "
                  f"{min(v):.2f} | {max(v):.2f} |")
        print()
        if traffic_op and subs:
            byk = {}
            for r in after_marker(rows):
                if picks(r["Kernel_Name"]):
                    byk.setdefault(r["Kernel_Name"], []).append(r)
            print(f"Operation `{traffic_op}`" + (", dispatches after the calibration copy" if after_cal else "")
                  + ":\n")
            print("| kernel | workgroups | dispatches | average us |")
            print("|---|---:|---:|---:|")
            tot = 0.0
            for kname, rs in sorted(byk.items()):
                durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rs]
                nwg = sorted({(int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))) *
                              int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]) for r in rs})
                avg = sum(durs) / len(durs)
                tot += avg
                print(f"| `{kname[:100]}` | {'/'.join(map(str, nwg))} | {len(durs)} | {avg:.2f} |")
            print(f"\nSum of the kernels' mean durations: {tot:.2f} us per launch of `{traffic_op}`.\n")
            print("op_trace_json: " + json.dumps({"op": traffic_op, "us_per_launch": round(tot, 2),
                                                 "source_hash": kernel_source_hash()}))
            print()
    if not cc:
        return 0
    agg, op_agg = {}, {}
    for f in cc:
        rows = list(csv.DictReader(open(f)))
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        for r in rows:
            k = (r["Kernel_Name"], r["Counter_Name"])
            agg.setdefault(k, []).append(float(r["Counter_Value"]))
        for r in after_marker(rows):
            k = (r["Kernel_Name"], r["Counter_Name"])
            op_agg.setdefault(k, []).append(float(r["Counter_Value"]))
    print("## counters (mean per dispatch)\n")
    print("| kernel | counter | mean | dispatches |")
    print("|---|---|---:|---:|")
    for (kname, cname), v in sorted(agg.items()):
        print(f"| `{kname[:110]}` | {cname} | {sum(v) / len(v):.1f} | {len(v)} |")
    print()
    if not (traffic_op and subs):
        return 0
    cal = COPY_CAL_BYTES / 1024
    copy = [k for (k, c) in agg if "copyBuffer" in k]
    if not copy:
        print("no calibration copy kernel found")
        return 1
    # the calibration copy is the largest copy dispatch (smaller device copies run the same kernel)
    big = {c: max(agg[(copy[0], c)]) for c in ("FETCH_SIZE", "WRITE_SIZE") if (copy[0], c) in agg}
    fs = cal / big["FETCH_SIZE"] if "FETCH_SIZE" in big else None
    wsc = cal / big["WRITE_SIZE"] if "WRITE_SIZE" in big else None
    names = sorted({k for (k, c) in op_agg if picks(k)})

    def per_launch(k, c):
        v = op_agg.get((k, c), [])
        return sum(v) / len(v) if v else 0.0

    fetch = sum(per_launch(k, "FETCH_SIZE") for k in names) * 1024 * (fs or 0)
    write = sum(per_launch(k, "WRITE_SIZE") for k in names) * 1024 * (wsc or 0)
    print(f"Calibration: the {COPY_CAL_BYTES >> 20} MiB device copy reads FETCH_SIZE "
          f"{big.get('FETCH_SIZE', float('nan')):.1f} KB and WRITE_SIZE "
          f"{big.get('WRITE_SIZE', float('nan')):.1f} KB, so counter KB are scaled by "
          f"{fs or float('nan'):.4f} (reads) and {wsc or float('nan'):.4f} (writes).\n")
    print(f"Operation `{traffic_op}` = " + " + ".join(f"`{k[:80]}`" for k in names) +
          (" (dispatches after the calibration copy)" if after_cal else "") +
          f": {fetch / 1e6:.1f} MB read + {write / 1e6:.1f} MB written per launch.\n")
    rec = {"op": traffic_op, "kernels": [k[:120] for k in names], "fetch_bytes": round(fetch),
           "write_bytes": round(write), "fetch_scale": round(fs or 0, 4), "write_scale": round(wsc or 0, 4),
           "after_calibration": bool(after_cal), "source_hash": kernel_source_hash()}
    print("traffic_json: " + json.dumps(rec))
    return 0


if __name__ == "__main__":
    sys.exit(main())
