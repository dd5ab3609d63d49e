"""CPU oracle for the ConvNeXt block's non-convolution steps -- TEST INFRASTRUCTURE ONLY.

Only ``tests/`` may import this module; the product library never does, and
this module imports nothing from the product.  Everything is float64 numpy,
written from the definitions:

* ``philox4x32_10`` -- the counter-based generator Philox4x32 with 10 rounds
  (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2,
  3", SC'11): each round multiplies two counter words by the constants
  0xD2511F53 and 0xCD9E8D57, and mixes the high halves with the other words
  and the key; the key is bumped by the Weyl constants 0x9E3779B9 and
  0xBB67AE85 between rounds.
* ``droppath_scales`` -- per-sample DropPath (stochastic depth) factors.  The
  NVIDIA blog "Perception Model Training for Autonomous Vehicles with Tensor
  Parallelism" (its ConvNeXt-XL paragraph) says the Bernoulli draws of
  DropPath must be the same on every GPU, and the kwkr.cn retelling (sections
  3.1 and 6.1) asks for the same seed in every DropPath layer.  Reading: a
  sample is kept with probability keep and then scaled by 1/keep; its draw is
  Philox4x32-10 of the counter (sample, offset low, offset high, 0) under the
  key (seed low, seed high), first word, kept when below floor(keep * 2^32).
  The draw depends on the sample index and not on the shard, so every shard
  makes the same decision.
* ``layernorm_channels_fwd`` / ``_bwd`` -- LayerNorm over the channel axis of
  an NCHW tensor (each pixel normalised over its C values, then scaled and
  shifted per channel), the ConvNeXt block's normalisation; mean and
  population variance, rstd = 1 / sqrt(var + eps).  The per-channel weight and
  bias gradients of a shard are partial sums over its own pixels.
* ``gelu_fwd`` / ``_bwd`` -- GELU, x * Phi(x) with Phi the standard normal
  CDF, written with the error function (scipy.special.erf).
* ``layer_scale_residual_fwd`` / ``_bwd`` -- the block's tail,
  out = x + s[n] * (gamma[c] * h), with s the DropPath factors (1 without
  DropPath) and gamma the per-channel layer scale.
"""
from __future__ import annotations

import math

import numpy as np
import scipy.special

_M0, _M1 = 0xD2511F53, 0xCD9E8D57
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
_MASK = 0xFFFFFFFF


def philox4x32_10(counter, key):
    """Philox4x32-10 of one 4-word counter under a 2-word key (Python ints)."""
    c = [int(v) & _MASK for v in counter]
    k0, k1 = int(key[0]) & _MASK, int(key[1]) & _MASK
    for r in range(10):
        if r:
            k0, k1 = (k0 + _W0) & _MASK, (k1 + _W1) & _MASK
        p0, p1 = _M0 * c[0], _M1 * c[2]
        hi0, lo0 = p0 >> 32, p0 & _MASK
        hi1, lo1 = p1 >> 32, p1 & _MASK
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
    return c


def keep_threshold(keep_prob: float) -> int:
    """The integer a draw must stay below to keep its sample: floor(keep * 2^32), at most 2^32 - 1."""
    return min(int(math.floor(keep_prob * 4294967296.0)), 0xFFFFFFFF)


def droppath_scales(seed: int, offset: int, n: int, keep_prob: float) -> np.ndarray:
    """Per-sample factors: 1/keep for a kept sample, 0 for a dropped one (float32).
    keep >= 1 keeps every sample (factor 1) without drawing."""
    if keep_prob >= 1.0:
        return np.ones(n, dtype=np.float32)
    thr = keep_threshold(keep_prob)
    inv = np.float32(1.0 / keep_prob)
    out = np.zeros(n, dtype=np.float32)
    for i in range(n):
        word = philox4x32_10((i, offset & _MASK, (offset >> 32) & _MASK, 0), (seed & _MASK, (seed >> 32) & _MASK))[0]
        out[i] = inv if word < thr else np.float32(0.0)
    return out


def layernorm_channels_fwd(x, gamma, beta, eps: float):
    """y[n,c,i,j] = (x - mean_c) * rstd * gamma[c] + beta[c]; returns (y, mean, rstd) with mean/rstd (N, H, W)."""
    x = np.asarray(x, dtype=np.float64)
    mean = x.mean(axis=1)
    var = ((x - mean[:, None]) ** 2).mean(axis=1)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (x - mean[:, None]) * rstd[:, None]
    g = np.asarray(gamma, dtype=np.float64)[None, :, None, None]
    b = np.asarray(beta, dtype=np.float64)[None, :, None, None]
    return xhat * g + b, mean, rstd


def layernorm_channels_bwd(x, dy, gamma, eps: float):
    """Gradients of layernorm_channels_fwd: (dx, dgamma, dbeta), the last two summed over every pixel given."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    c = x.shape[1]
    mean = x.mean(axis=1, keepdims=True)
    rstd = 1.0 / np.sqrt(((x - mean) ** 2).mean(axis=1, keepdims=True) + eps)
    xhat = (x - mean) * rstd
    dxhat = dy * np.asarray(gamma, dtype=np.float64)[None, :, None, None]
    a = dxhat.sum(axis=1, keepdims=True)
    b = (dxhat * xhat).sum(axis=1, keepdims=True)
    dx = rstd * (dxhat - a / c - xhat * b / c)
    return dx, (dy * xhat).sum(axis=(0, 2, 3)), dy.sum(axis=(0, 2, 3))


_SQRT1_2 = 1.0 / math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)
# erf by scipy's vectorised double-precision routine (math.erf element by
# element is too slow for the 2.3e8-element activations of a full-size shard)
_erf = scipy.special.erf


def gelu_fwd(x):
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + _erf(x * _SQRT1_2))


def gelu_bwd(x, dy):
    """dx = dy * (Phi(x) + x * phi(x))."""
    x = np.asarray(x, dtype=np.float64)
    cdf = 0.5 * (1.0 + _erf(x * _SQRT1_2))
    pdf = _INV_SQRT_2PI * np.exp(-0.5 * x * x)
    return np.asarray(dy, dtype=np.float64) * (cdf + x * pdf)


def layer_scale_residual_fwd(x, h, gamma, scales=None):
    """out = x + s[n] * (gamma[c] * h)."""
    h = np.asarray(h, dtype=np.float64)
    s = np.ones(h.shape[0]) if scales is None else np.asarray(scales, dtype=np.float64)
    g = np.asarray(gamma, dtype=np.float64)[None, :, None, None]
    return np.asarray(x, dtype=np.float64) + s[:, None, None, None] * (g * h)


def layer_scale_residual_bwd(h, dout, gamma, scales=None):
    """(dh, dgamma) of layer_scale_residual_fwd; d(x) is dout itself."""
    h = np.asarray(h, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    s = np.ones(h.shape[0]) if scales is None else np.asarray(scales, dtype=np.float64)
    g = np.asarray(gamma, dtype=np.float64)[None, :, None, None]
    sd = s[:, None, None, None] * dout
    return sd * g, (sd * h).sum(axis=(0, 2, 3))
