"""Autograd layer over the W-sharded convolution ABI.

The pages train ConvNeXt with every activation sharded along W and the
parameters replicated (NVIDIA blog "Perception Model Training for Autonomous
Vehicles with Tensor Parallelism", DTensor section: activations Shard(3),
weights Replicate; the kwkr.cn retelling, section 3.2, wraps the halo exchange
in an autograd function).  Here an activation is a list of S contiguous
(N, C, H, W/S) float32 tensors on one device, one per shard, as they would sit
on S GPUs, and `ShardedConv2d` is a module over such lists:

* forward: each shard gathers its halo columns from its two neighbours, then
  convolves its slice (output: the shard's own columns);
* backward: grad_output halos are gathered the same way; each shard computes
  its grad_input slice and its partial grad_weight / grad_bias over its own
  output columns; the partials are summed in shard order (the reduction that
  turns the _Partial gradients into replicated ones).

With dim=2 the shards are slices of rows instead (Shard(2), the height split
of kwkr.cn retelling, section 5.2): the same steps with row halos.

This file only marshals tensors and calls the C ABI (`sscnn`); every step runs
in the library's kernels, and there is no fallback when the library is
missing.
"""
from __future__ import annotations

import math
from typing import List, Sequence

import torch

from . import sscnn


def shard(x: torch.Tensor, num_shards: int, dim: int = 3) -> List[torch.Tensor]:
    """Split an (N, C, H, W) tensor into num_shards contiguous slices along W
    (dim=3) or H (dim=2)."""
    if x.dim() != 4 or dim not in (2, 3) or x.shape[dim] % num_shards:
        raise ValueError(f"cannot split {tuple(x.shape)} into {num_shards} shards along dim {dim}")
    w = x.shape[dim] // num_shards
    return [x.narrow(dim, s * w, w).contiguous() for s in range(num_shards)]


def unshard(xs: Sequence[torch.Tensor], dim: int = 3) -> torch.Tensor:
    """Concatenate shards back into one tensor."""
    return torch.cat(list(xs), dim=dim)


class _WCalls:
    """The ABI calls of a W-split layer."""
    halo_gather = staticmethod(sscnn.halo_gather)
    conv_fwd = staticmethod(sscnn.conv_fwd)
    conv_bwd = staticmethod(sscnn.conv_bwd)
    conv_bwd_weight_partial = staticmethod(sscnn.conv_bwd_weight_partial)
    new_workspace = staticmethod(sscnn.new_workspace)
    init = staticmethod(sscnn.conv_init)


class _HCalls:
    """The ABI calls of an H-split layer (row halos)."""
    halo_gather = staticmethod(sscnn.row_halo_gather)
    conv_fwd = staticmethod(sscnn.hconv_fwd)
    conv_bwd = staticmethod(sscnn.hconv_bwd)
    conv_bwd_weight_partial = staticmethod(sscnn.hconv_bwd_weight_partial)
    new_workspace = staticmethod(sscnn.new_hworkspace)
    init = staticmethod(sscnn.hconv_init)


class _ShardedConv(torch.autograd.Function):
    """Arguments: (layer, weight, bias or None, *x_shards) -> tuple of y shards."""

    @staticmethod
    def forward(ctx, layer, weight, bias, *xs):
        S = len(xs)
        convs = layer._descriptors(xs)
        A = layer._calls
        dev = xs[0].device
        halos = []
        for s, c in enumerate(convs):
            h = torch.empty(c.halo_shape(sscnn.HALO_INPUT), device=dev, dtype=torch.float32)
            A.halo_gather(c, sscnn.HALO_INPUT, xs[s - 1] if s > 0 else None, xs[s + 1] if s + 1 < S else None, h)
            halos.append(h)
        ys = []
        for s, c in enumerate(convs):
            y = torch.empty(c.y_shape, device=dev, dtype=torch.float32)
            A.conv_fwd(c, xs[s], halos[s], weight, bias, y)
            ys.append(y)
        ctx.convs = convs
        ctx.calls = A
        ctx.has_bias = bias is not None
        ctx.save_for_backward(weight, *xs, *halos)
        return tuple(ys)

    @staticmethod
    def backward(ctx, *gys):
        convs = ctx.convs
        A = ctx.calls
        S = len(convs)
        saved = ctx.saved_tensors
        weight, xs, halos = saved[0], saved[1:1 + S], saved[1 + S:1 + 2 * S]
        dev = weight.device
        gys = [torch.zeros(c.y_shape, device=dev, dtype=torch.float32) if g is None else g.contiguous()
               for g, c in zip(gys, convs)]
        need_dx = any(ctx.needs_input_grad[3:])
        ghalos = []
        for s, c in enumerate(convs):
            h = torch.empty(c.halo_shape(sscnn.HALO_GRAD_OUTPUT), device=dev, dtype=torch.float32)
            A.halo_gather(c, sscnn.HALO_GRAD_OUTPUT, gys[s - 1] if s > 0 else None,
                          gys[s + 1] if s + 1 < S else None, h)
            ghalos.append(h)
        nw, co = weight.numel(), weight.shape[0]
        parts = [torch.empty(nw + co, device=dev, dtype=torch.float32) for _ in range(S)]
        workspace = A.new_workspace(convs[0], device=dev)   # shards share a geometry; calls run in order
        dxs = []
        for s, c in enumerate(convs):
            gw_part, gb_part = parts[s][:nw].view(weight.shape), parts[s][nw:]
            if need_dx:
                dx = torch.empty(c.x_shape, device=dev, dtype=torch.float32)
                A.conv_bwd(c, xs[s], halos[s], gys[s], ghalos[s], weight, dx, gw_part, gb_part, workspace)
                dxs.append(dx)
            else:
                A.conv_bwd_weight_partial(c, xs[s], halos[s], gys[s], gw_part, gb_part, workspace)
                dxs.append(None)
        reduced = torch.empty(nw + co, device=dev, dtype=torch.float32)
        sscnn.partial_reduce(parts, reduced)
        grad_w = reduced[:nw].view(weight.shape)
        grad_b = reduced[nw:] if ctx.has_bias else None
        return (None, grad_w, grad_b, *dxs)


class ShardedConv2d(torch.nn.Module):
    """A 2-D convolution (cross-correlation, zero padding, square kernel) on
    sharded activations: forward(list of S shards) -> list of S shards, the
    shards being slices along W (dim=3, the default) or H (dim=2).

    Parameters are replicated (one weight / bias tensor); their gradients are
    the reduced sums of the shards' partials.  Initialisation matches
    torch.nn.Conv2d's defaults."""

    def __init__(self, in_channels: int, out_channels: int, kernel_size: int, stride: int = 1,
                 padding: int = 0, groups: int = 1, bias: bool = True, device="cuda", dim: int = 3):
        super().__init__()
        if dim not in (2, 3):
            raise ValueError("dim must be 2 (H) or 3 (W)")
        self.dim = dim
        self._calls = _HCalls if dim == 2 else _WCalls
        if in_channels % groups or out_channels % groups:
            raise ValueError("groups must divide in_channels and out_channels")
        self.in_channels, self.out_channels = in_channels, out_channels
        self.kernel_size, self.stride, self.padding, self.groups = kernel_size, stride, padding, groups
        self.weight = torch.nn.Parameter(torch.empty(out_channels, in_channels // groups, kernel_size, kernel_size,
                                                     device=device, dtype=torch.float32))
        self.bias = (torch.nn.Parameter(torch.empty(out_channels, device=device, dtype=torch.float32))
                     if bias else None)
        self.reset_parameters()
        self._cache = {}

    def reset_parameters(self):
        torch.nn.init.kaiming_uniform_(self.weight, a=math.sqrt(5))
        if self.bias is not None:
            fan_in = self.weight.shape[1] * self.kernel_size * self.kernel_size
            bound = 1.0 / math.sqrt(fan_in)
            torch.nn.init.uniform_(self.bias, -bound, bound)

    def _descriptors(self, xs):
        shapes = tuple(tuple(x.shape) for x in xs)
        if len(set(shapes)) != 1:
            raise ValueError(f"shards must have one shape, got {shapes}")
        key = shapes[0] + (len(xs),)
        if key not in self._cache:
            n, c, h, w = shapes[0]
            if c != self.in_channels:
                raise ValueError(f"expected {self.in_channels} channels, got {c}")
            self._cache[key] = [self._calls.init(n, c, self.out_channels, h, w, self.kernel_size, self.stride,
                                                 self.padding, self.groups, s, len(xs)) for s in range(len(xs))]
        return self._cache[key]

    def forward(self, xs: Sequence[torch.Tensor]) -> List[torch.Tensor]:
        xs = list(xs)
        if not xs:
            raise ValueError("no shards")
        return list(_ShardedConv.apply(self, self.weight, self.bias, *xs))

    def extra_repr(self):
        return (f"{self.in_channels}, {self.out_channels}, kernel_size={self.kernel_size}, stride={self.stride}, "
                f"padding={self.padding}, groups={self.groups}, bias={self.bias is not None}, dim={self.dim}")


# --- the ConvNeXt block on sharded activations ---------------------------------------
#
# The block (depthwise 7x7 -> LayerNorm over channels -> 1x1 expansion -> GELU
# -> 1x1 projection -> layer scale -> DropPath -> residual) with every step in
# the library: the convolutions through ShardedConv2d, the rest through the
# per-pixel block calls, which need no halo.  Weight gradients of the per-pixel
# steps are partial sums per shard, reduced like the convolutions'.  DropPath
# draws its per-sample factors from a counter-based generator keyed by (seed,
# call counter), so every shard drops the same samples (kwkr.cn retelling,
# sections 3.1 and 6.1; NVIDIA blog, ConvNeXt-XL paragraph).

def _zeros_if_none(gs, like):
    return [torch.zeros_like(x) if g is None else g.contiguous() for g, x in zip(gs, like)]


class _ChannelLayerNorm(torch.autograd.Function):
    @staticmethod
    def forward(ctx, weight, bias, eps, *xs):
        ys, stats = [], []
        for x in xs:
            n, c, h, w = x.shape
            y = torch.empty_like(x)
            mean = torch.empty((n, h, w), device=x.device, dtype=torch.float32)
            rstd = torch.empty((n, h, w), device=x.device, dtype=torch.float32)
            sscnn.layernorm_fwd(x, weight, bias, y, mean, rstd, eps)
            ys.append(y)
            stats += [mean, rstd]
        ctx.save_for_backward(weight, *xs, *stats)
        ctx.nshards = len(xs)
        return tuple(ys)

    @staticmethod
    def backward(ctx, *gys):
        S = ctx.nshards
        saved = ctx.saved_tensors
        weight, xs, stats = saved[0], saved[1:1 + S], saved[1 + S:]
        gys = _zeros_if_none(gys, xs)
        c = weight.shape[0]
        need_dx = any(ctx.needs_input_grad[3:])
        dxs, parts = [], []
        for s, x in enumerate(xs):
            part = torch.empty(2 * c, device=x.device, dtype=torch.float32)
            dx = torch.empty_like(x) if need_dx else None
            sscnn.layernorm_bwd(x, gys[s], weight, stats[2 * s], stats[2 * s + 1], dx, part[:c], part[c:])
            dxs.append(dx)
            parts.append(part)
        red = torch.empty(2 * c, device=weight.device, dtype=torch.float32)
        sscnn.partial_reduce(parts, red)
        return (red[:c], red[c:], None, *dxs)


class _Gelu(torch.autograd.Function):
    @staticmethod
    def forward(ctx, *xs):
        ys = []
        for x in xs:
            y = torch.empty_like(x)
            sscnn.gelu_fwd(x, y)
            ys.append(y)
        ctx.save_for_backward(*xs)
        return tuple(ys)

    @staticmethod
    def backward(ctx, *gys):
        xs = ctx.saved_tensors
        gys = _zeros_if_none(gys, xs)
        dxs = []
        for x, g in zip(xs, gys):
            dx = torch.empty_like(x)
            sscnn.gelu_bwd(x, g, dx)
            dxs.append(dx)
        return tuple(dxs)


def _pointwise_desc(x, c_out):
    """A 1x1 layer over one shard, described as one whole slice: a pointwise
    layer needs no halo, so W-, H- and 2-D shards are alike to it."""
    n, c, h, w = x.shape
    return sscnn.conv_init(n, c, c_out, h, w, 1, 1, 0, 1, 0, 1)


def _mlp_fusable(xs, c_in, c_hidden, c_out):
    """Whether the fused pointwise calls take these shards (the matrix-core
    path's conditions: channels and slice width multiples of 16)."""
    return all(c % 16 == 0 for c in (c_in, c_hidden, c_out)) and \
        all(x.shape[3] % 16 == 0 and x.numel() // c_in * c_hidden < 2 ** 31 for x in xs)


class _PointwiseMLP(torch.autograd.Function):
    """pw2(GELU(pw1(x))) on every shard, with GELU inside pw1's kernel: its
    forward writes the pre-activation h and GELU(h) together (h is kept for
    GELU's gradient in the backward).
    Arguments: (w1, b1, w2, b2, *x_shards) -> tuple of output shards."""

    @staticmethod
    def forward(ctx, w1, b1, w2, b2, *xs):
        hs, acts, outs, convs = [], [], [], []
        for x in xs:
            c1, c2 = _pointwise_desc(x, w1.shape[0]), None
            h = torch.empty(c1.y_shape, device=x.device, dtype=torch.float32)
            a = torch.empty_like(h)
            sscnn.pointwise_gelu_fwd(c1, x, w1, b1, h, a)
            c2 = _pointwise_desc(a, w2.shape[0])
            out = torch.empty(c2.y_shape, device=x.device, dtype=torch.float32)
            sscnn.conv_fwd(c2, a, None, w2, b2, out)
            hs.append(h)
            acts.append(a)
            outs.append(out)
            convs.append((c1, c2))
        ctx.convs = convs
        ctx.has_bias = (b1 is not None, b2 is not None)
        ctx.save_for_backward(w1, w2, *xs, *hs, *acts)
        return tuple(outs)

    @staticmethod
    def backward(ctx, *gos):
        S = len(ctx.convs)
        saved = ctx.saved_tensors
        w1, w2 = saved[0], saved[1]
        xs, hs, acts = saved[2:2 + S], saved[2 + S:2 + 2 * S], saved[2 + 2 * S:2 + 3 * S]
        dev = w1.device
        gos = [torch.zeros(c2.y_shape, device=dev, dtype=torch.float32) if g is None else g.contiguous()
               for g, (_, c2) in zip(gos, ctx.convs)]
        need_dx = any(ctx.needs_input_grad[4:])
        n1, n2 = w1.numel(), w2.numel()
        parts1 = [torch.empty(n1 + w1.shape[0], device=dev, dtype=torch.float32) for _ in range(S)]
        parts2 = [torch.empty(n2 + w2.shape[0], device=dev, dtype=torch.float32) for _ in range(S)]
        dxs = []
        for s, (c1, c2) in enumerate(ctx.convs):
            # pw2's grad_input, then GELU's gradient as a pass of its own: measured
            # faster than the fused sscnn_pointwise_bwd_input_gelu, whose epilogue
            # transcendentals run at the matrix kernel's low occupancy
            da, dh = torch.empty_like(hs[s]), torch.empty_like(hs[s])
            sscnn.conv_bwd(c2, acts[s], None, gos[s], None, w2, da, parts2[s][:n2].view(w2.shape),
                           parts2[s][n2:], sscnn.new_workspace(c2, device=dev))
            sscnn.gelu_bwd(hs[s], da, dh)
            del da
            gw1, gb1 = parts1[s][:n1].view(w1.shape), parts1[s][n1:]
            if need_dx:
                dx = torch.empty(c1.x_shape, device=dev, dtype=torch.float32)
                sscnn.conv_bwd(c1, xs[s], None, dh, None, w1, dx, gw1, gb1, sscnn.new_workspace(c1, device=dev))
                dxs.append(dx)
            else:
                sscnn.conv_bwd_weight_partial(c1, xs[s], None, dh, gw1, gb1, sscnn.new_workspace(c1, device=dev))
                dxs.append(None)
        red1 = torch.empty(n1 + w1.shape[0], device=dev, dtype=torch.float32)
        red2 = torch.empty(n2 + w2.shape[0], device=dev, dtype=torch.float32)
        sscnn.partial_reduce(parts1, red1)
        sscnn.partial_reduce(parts2, red2)
        return (red1[:n1].view(w1.shape), red1[n1:] if ctx.has_bias[0] else None,
                red2[:n2].view(w2.shape), red2[n2:] if ctx.has_bias[1] else None, *dxs)


class _LayerScaleResidual(torch.autograd.Function):
    """out_s = x_s + scales[n] * (gamma[c] * h_s) for every shard s."""

    @staticmethod
    def forward(ctx, gamma, scales, *xs_hs):
        S = len(xs_hs) // 2
        xs, hs = xs_hs[:S], xs_hs[S:]
        outs = []
        for x, h in zip(xs, hs):
            out = torch.empty_like(x)
            sscnn.layer_scale_residual_fwd(x, h, gamma, scales, out)
            outs.append(out)
        ctx.save_for_backward(gamma, *hs)
        ctx.scales = scales
        ctx.nshards = S
        return tuple(outs)

    @staticmethod
    def backward(ctx, *gos):
        S = ctx.nshards
        saved = ctx.saved_tensors
        gamma, hs = saved[0], saved[1:]
        gos = _zeros_if_none(gos, hs)
        c = gamma.shape[0]
        dhs, parts = [], []
        for h, go in zip(hs, gos):
            dh = torch.empty_like(h)
            part = torch.empty(c, device=h.device, dtype=torch.float32)
            sscnn.layer_scale_residual_bwd(h, go, gamma, ctx.scales, dh, part)
            dhs.append(dh)
            parts.append(part)
        dgamma = torch.empty(c, device=gamma.device, dtype=torch.float32)
        sscnn.partial_reduce(parts, dgamma)
        dxs = list(gos) if any(ctx.needs_input_grad[2:2 + S]) else [None] * S
        return (dgamma, None, *dxs, *dhs)


class ShardedConvNeXtBlock(torch.nn.Module):
    """One ConvNeXt block over a list of S shards (W slices, or H slices with
    dim=2): x + DropPath(gamma * pw2(GELU(pw1(LN(dw7x7(x)))))).  When the
    channel counts and slice width are multiples of 16, the forward GELU runs
    inside the 1x1 expansion's kernel (_PointwiseMLP); otherwise as a pass of
    its own.

    DropPath is active in training mode when drop_path > 0; its per-sample
    factors come from sscnn_droppath_scales with this block's seed and a call
    counter.  They depend on those two numbers and the sample index only, so a
    shard on a GPU of its own would compute the same factors; here they are
    computed once per call and used by every shard."""

    def __init__(self, dim: int, drop_path: float = 0.0, layer_scale_init: float = 1e-6, eps: float = 1e-6,
                 seed: int = 0, device="cuda", shard_dim: int = 3):
        super().__init__()
        if not 0.0 <= drop_path < 1.0:
            raise ValueError("drop_path must be in [0, 1)")
        self.dim, self.drop_path, self.eps, self.seed = dim, drop_path, eps, seed
        self.dwconv = ShardedConv2d(dim, dim, 7, padding=3, groups=dim, device=device, dim=shard_dim)
        self.norm_weight = torch.nn.Parameter(torch.ones(dim, device=device))
        self.norm_bias = torch.nn.Parameter(torch.zeros(dim, device=device))
        self.pwconv1 = ShardedConv2d(dim, 4 * dim, 1, device=device, dim=shard_dim)
        self.pwconv2 = ShardedConv2d(4 * dim, dim, 1, device=device, dim=shard_dim)
        self.gamma = torch.nn.Parameter(torch.full((dim,), layer_scale_init, device=device))
        self.calls = 0      # DropPath call counter: the generator's offset

    def forward(self, xs: Sequence[torch.Tensor]) -> List[torch.Tensor]:
        xs = list(xs)
        h = self.dwconv(xs)
        h = list(_ChannelLayerNorm.apply(self.norm_weight, self.norm_bias, self.eps, *h))
        p1, p2 = self.pwconv1, self.pwconv2
        if _mlp_fusable(h, self.dim, p1.out_channels, p2.out_channels):
            h = list(_PointwiseMLP.apply(p1.weight, p1.bias, p2.weight, p2.bias, *h))
        else:
            h = p2(list(_Gelu.apply(*p1(h))))
        scales = None
        if self.training and self.drop_path > 0.0:
            scales = torch.empty(xs[0].shape[0], device=xs[0].device, dtype=torch.float32)
            sscnn.droppath_scales(self.seed, self.calls, 1.0 - self.drop_path, scales)
            self.calls += 1
        return list(_LayerScaleResidual.apply(self.gamma, scales, *xs, *h))
