"""Seeded synthetic workloads for the width-sharded convolution.

This module is shared by the product's tests and benchmark and by the oracle
side of those tests.  It holds NO convolution arithmetic: tensor shapes are
written out (the stack's maps are the input's divided by the 4x4/4 stem and
halved by each 2x2/2 downsample), and the only computation here is drawing
seeded random numbers.

Values: numpy ``default_rng(seed)`` (PCG64), float32.  Draw order within a
workload: input X (global), then per layer (weight, bias) in chain order, then
grad_output G (global).  Distributions: U[-1, 1] for the tiny dense case;
otherwise activations and grad_output N(0, 1) and every weight and bias
N(0, 0.02) (standard normal float32 draws scaled by float32 0.02).

The shapes follow the pages: a (7, 3, 512, 2048) input split four ways on W
into (7, 3, 512, 512) slices, the 5x5 / pad 2 / stride 1 halo example, and the
(7, 3, 512, 4096) input of the 4-GPU run (NVIDIA blog "Perception Model
Training for Autonomous Vehicles with Tensor Parallelism", DTensor section and
results section).  The pages train on camera images that are not available;
seeded tensors of the same shapes stand in, since the cost of the path depends
only on shapes.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class Layer:
    """One convolution: square kernel k, stride, pad, groups, channels in/out,
    and the global input / output shapes it maps between."""
    name: str
    ci: int
    co: int
    k: int
    stride: int
    pad: int
    groups: int
    in_shape: Tuple[int, int, int, int]    # global (N, Ci, H, W)
    out_shape: Tuple[int, int, int, int]   # global (N, Co, Ho, Wo)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    layers: Tuple[Layer, ...]
    num_shards: int
    shard: int           # the shard whose share is measured
    seed: int
    dist: str            # "uniform" or "normal"
    description: str
    axis: int = 3        # the sharded dimension: 3 = W (Shard(3)), 2 = H (Shard(2))
    kind: str = "conv"   # "conv" (one layer or a stack of convolutions) or "block" (a ConvNeXt block)

    @property
    def x_shape(self):
        return self.layers[0].in_shape

    @property
    def g_shape(self):
        return self.layers[-1].out_shape


def _layer(name, ci, co, k, stride, pad, groups, in_shape, out_shape):
    return Layer(name, ci, co, k, stride, pad, groups, tuple(in_shape), tuple(out_shape))


def convnext_stack(n, w, h=512, dims=(256, 512, 1024, 2048), name_prefix=""):
    """Layers of a ConvNeXt-style convolution stack on a global (n, 3, h, w)
    input: stem 4x4/4 (3 -> dims[0]), then per stage a depthwise 7x7 pad 3
    and a 2x2/2 downsample to the next stage's width, ending with the last
    stage's depthwise conv."""
    layers = []
    c, hh, ww = dims[0], h // 4, w // 4
    layers.append(_layer(name_prefix + "stem", 3, c, 4, 4, 0, 1, (n, 3, h, w), (n, c, hh, ww)))
    for st, cn in enumerate(dims):
        layers.append(_layer(f"{name_prefix}dw{st + 1}", cn, cn, 7, 1, 3, cn, (n, cn, hh, ww), (n, cn, hh, ww)))
        if st + 1 < len(dims):
            nxt = dims[st + 1]
            layers.append(_layer(f"{name_prefix}ds{st + 1}", cn, nxt, 2, 2, 0, 1, (n, cn, hh, ww),
                                 (n, nxt, hh // 2, ww // 2)))
            hh, ww = hh // 2, ww // 2
    return tuple(layers)


WORKLOADS = {
    "dense5x5_tiny": Workload(
        "dense5x5_tiny",
        (_layer("conv", 3, 8, 5, 1, 2, 1, (1, 3, 32, 64), (1, 8, 32, 64)),),
        num_shards=4, shard=1, seed=1001, dist="uniform",
        description="dense 5x5 s1 p2 conv 3->8 on (1,3,32,64), four 16-wide slices, 2-column halos"),
    "dw7_c256": Workload(
        "dw7_c256",
        (_layer("dw", 256, 256, 7, 1, 3, 256, (7, 256, 128, 256), (7, 256, 128, 256)),),
        num_shards=4, shard=1, seed=1002, dist="normal",
        description="depthwise 7x7 s1 p3 C=256: shard (7,256,128,64) of a (7,256,128,256) map, 3-column halos"),
    "dw7_c256_hshard": Workload(
        "dw7_c256_hshard",
        (_layer("dw", 256, 256, 7, 1, 3, 256, (7, 256, 128, 256), (7, 256, 128, 256)),),
        num_shards=4, shard=1, seed=1002, dist="normal",
        description="depthwise 7x7 s1 p3 C=256 split along H: shard (7,256,32,256) of the same (7,256,128,256) "
                    "map, 3-row halos", axis=2),
    "convnext_block_c256": Workload(
        "convnext_block_c256",
        (_layer("dw", 256, 256, 7, 1, 3, 256, (7, 256, 128, 256), (7, 256, 128, 256)),
         _layer("pw1", 256, 1024, 1, 1, 0, 1, (7, 256, 128, 256), (7, 1024, 128, 256)),
         _layer("pw2", 1024, 256, 1, 1, 0, 1, (7, 1024, 128, 256), (7, 256, 128, 256))),
        num_shards=4, shard=1, seed=1006, dist="normal",
        description="ConvNeXt block at C=256 (dw 7x7, LayerNorm, 1x1 256->1024, GELU, 1x1 1024->256, layer "
                    "scale, DropPath 0.1, residual): shard (7,256,128,64) of a (7,256,128,256) map",
        kind="block"),
    "dw7_c256_grid": Workload(
        "dw7_c256_grid",
        (_layer("dw", 256, 256, 7, 1, 3, 256, (7, 256, 128, 256), (7, 256, 128, 256)),),
        num_shards=4, shard=3, seed=1002, dist="normal",
        description="depthwise 7x7 s1 p3 C=256 on a 2x2 grid of blocks: block (1,1), (7,256,64,128), of the same "
                    "(7,256,128,256) map, 3-row and 3-column halos with corners", kind="grid"),
    "dense5x5_c256": Workload(
        "dense5x5_c256",
        (_layer("conv", 256, 256, 5, 1, 2, 1, (7, 256, 128, 512), (7, 256, 128, 512)),),
        num_shards=4, shard=1, seed=1003, dist="normal",
        description="dense 5x5 s1 p2 conv 256->256: shard (7,256,128,128) of a (7,256,128,512) map, 2-column halos"),
    "dense5x5_c256_hshard": Workload(
        "dense5x5_c256_hshard",
        (_layer("conv", 256, 256, 5, 1, 2, 1, (7, 256, 128, 512), (7, 256, 128, 512)),),
        num_shards=4, shard=1, seed=1003, dist="normal",
        description="dense 5x5 s1 p2 conv 256->256 split along H: shard (7,256,32,512) of a (7,256,128,512) "
                    "map, 2-row halos", axis=2),
    "dense5x5_c256_grid": Workload(
        "dense5x5_c256_grid",
        (_layer("conv", 256, 256, 5, 1, 2, 1, (7, 256, 128, 512), (7, 256, 128, 512)),),
        num_shards=4, shard=3, seed=1003, dist="normal",
        description="dense 5x5 s1 p2 conv 256->256 on a 2x2 grid of blocks: block (1,1), (7,256,64,256), of a "
                    "(7,256,128,512) map, 2-row and 2-column halos with corners", kind="grid"),
    "convnext_xl_w2048": Workload(
        "convnext_xl_w2048", convnext_stack(7, 2048),
        num_shards=4, shard=1, seed=1004, dist="normal",
        description="ConvNeXt-XL conv stack on shard (7,3,512,512) of a (7,3,512,2048) input"),
    "convnext_xl_w4096": Workload(
        "convnext_xl_w4096", convnext_stack(7, 4096),
        num_shards=4, shard=1, seed=1005, dist="normal",
        description="ConvNeXt-XL conv stack on shard (7,3,512,1024) of a (7,3,512,4096) input"),
}


@dataclasses.dataclass
class Tensors:
    x: np.ndarray                  # global input (N, Ci, H, W)
    weights: List[np.ndarray]      # per layer (Co, Ci/groups, K, K)
    biases: List[np.ndarray]       # per layer (Co,)
    g: np.ndarray                  # global grad of the last output


def _draw(rng, shape, dist, scale=1.0):
    if dist == "uniform":
        return rng.uniform(-1.0, 1.0, size=shape).astype(np.float32)
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return a


def generate(wl: Workload, seed: Optional[int] = None) -> Tensors:
    """Draw the workload's tensors (host, float32) from its seed."""
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    act_scale, par_scale = (1.0, 1.0) if wl.dist == "uniform" else (1.0, 0.02)
    x = _draw(rng, wl.x_shape, wl.dist, act_scale)
    ws, bs = [], []
    for L in wl.layers:
        ws.append(_draw(rng, (L.co, L.ci // L.groups, L.k, L.k), wl.dist, par_scale))
        bs.append(_draw(rng, (L.co,), wl.dist, par_scale))
    g = _draw(rng, wl.g_shape, wl.dist, act_scale)
    return Tensors(x, ws, bs, g)


def stack(name, layers, num_shards, shard=1, seed=11, dist="normal") -> Workload:
    """A multi-layer workload (e.g. a smaller ConvNeXt-style stack)."""
    return Workload(name, tuple(layers), num_shards, shard, seed, dist, name)


def custom(name, n, ci, co, h, w, k, stride, pad, groups, ho, wo, num_shards,
           shard=1, seed=7, dist="normal") -> Workload:
    """A one-layer workload with explicit shapes (for parity cases that span
    several tiles and ragged tails)."""
    L = _layer("conv", ci, co, k, stride, pad, groups, (n, ci, h, w), (n, co, ho, wo))
    return Workload(name, (L,), num_shards, shard, seed, dist, name)
