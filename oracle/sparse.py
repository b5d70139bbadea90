"""Per-vector dense-and-sparse group quantization (oracle; test infrastructure only).

synthetic.wiki "KV cache quantization: putting the bits in the cached vectors, not the weights",
section "What they report", KVQuant's list of methods: per-vector dense-and-sparse quantization isolates outliers separately for each
vector, so that they do not skew the quantization ranges.

Readings taken where the page is silent:
- a vector is one quantization group of 32 elements (keys: 32 tokens of one channel; values: 32 channels of one
  token), so the outlier handling follows the grouping the rest of the cache uses;
- the number of outliers is a fixed fraction chosen here, one per group (1/32), with no calibration: the element of
  largest magnitude |x|, the lowest index on ties;
- the outlier keeps its float16 value exactly, stored with its index within the group; the other 31 elements (the
  dense part) are quantized by the ordinary group quantizer (``quant.quantize_groups``) over their own minimum and
  maximum; the outlier's code slot holds 0 and is ignored when decoding.

The largest-magnitude element is always the group maximum or minimum, so the dense range never exceeds the full
range: dense-and-sparse never enlarges the scale.
"""
from __future__ import annotations

import numpy as np

from . import quant


def quantize_groups_sparse(x: np.ndarray, bits: int):
    """Groups along the last axis of float16 ``x`` ``[..., g]`` (g >= 2).

    Returns ``codes`` uint8 ``[..., g]`` (the outlier's slot 0), ``scale``, ``zero`` float16 ``[...]`` of the dense
    part, the outlier value float16 ``[...]`` and its index uint8 ``[...]``.
    """
    x = np.asarray(x)
    if x.dtype != np.float16:
        raise TypeError("quantize_groups_sparse expects float16 input")
    if x.shape[-1] < 2:
        raise ValueError("a group needs at least two elements")
    idx = np.argmax(np.abs(x.astype(np.float64)), axis=-1)          # first occurrence on ties
    out = np.take_along_axis(x, idx[..., None], axis=-1)[..., 0]
    # the dense part: the outlier's slot takes the smallest dense value, which leaves the dense minimum and maximum
    # (all the quantizer looks at besides each element itself) unchanged
    xf = x.astype(np.float64)
    is_out = np.arange(x.shape[-1]) == idx[..., None]
    dense_min = np.where(is_out, np.inf, xf).min(axis=-1)
    filled = np.where(is_out, dense_min[..., None], xf).astype(np.float16)
    codes, scale, zero = quant.quantize_groups(filled, bits)
    codes = np.where(is_out, 0, codes).astype(np.uint8)
    return codes, scale, zero, out.astype(np.float16), idx.astype(np.uint8)


def dequantize_groups_sparse(codes, scale, zero, out, idx) -> np.ndarray:
    """Decoded values float64: dense ``q * s + z``, with each group's outlier restored at its index."""
    x = quant.dequantize_groups(codes, scale, zero)
    is_out = np.arange(codes.shape[-1]) == np.asarray(idx, np.int64)[..., None]
    return np.where(is_out, np.asarray(out, np.float64)[..., None], x)


def quantize_keys_per_channel_sparse(k: np.ndarray, group: int = 32, bits: int = 4):
    """Per-channel key groups (32 tokens of one channel) with one outlier each. ``k`` float16 ``[..., T, D]``.

    Returns codes ``[..., T, D]``, scale, zero ``[..., T // group, D]``, outlier values float16 and their token
    indices within the group uint8 ``[..., T // group, D]``.
    """
    *lead, t, d = k.shape
    if t % group:
        raise ValueError("token count must be a multiple of the group size")
    g = np.swapaxes(k.reshape(*lead, t // group, group, d), -1, -2)     # [..., tiles, D, group]
    codes, scale, zero, out, idx = quantize_groups_sparse(g, bits)
    return np.swapaxes(codes, -1, -2).reshape(*lead, t, d), scale, zero, out, idx


def quantize_values_per_token_sparse(v: np.ndarray, group: int = 32, bits: int = 4):
    """Per-token value groups (32 channels of one token) with one outlier each. ``v`` float16 ``[..., T, D]``.

    Returns codes ``[..., T, D]``, scale, zero ``[..., T, D // group]``, outlier values float16 and their channel
    indices within the group uint8 ``[..., T, D // group]``.
    """
    *lead, t, d = v.shape
    if d % group:
        raise ValueError("head_dim must be a multiple of the group size")
    codes, scale, zero, out, idx = quantize_groups_sparse(v.reshape(*lead, t, d // group, group), bits)
    return codes.reshape(*lead, t, d), scale, zero, out, idx


def dequantize_keys_sparse(codes, scale, zero, out, idx, group: int = 32) -> np.ndarray:
    """Decoded keys float64 ``[..., T, D]``: per-channel dense decode, each group's outlier token restored."""
    x = quant.dequantize_keys(codes, scale, zero, group)
    *lead, t, d = x.shape
    g = x.reshape(*lead, t // group, group, d)
    is_out = np.arange(group)[:, None] == np.asarray(idx, np.int64)[..., None, :]     # [..., tiles, group, D]
    g = np.where(is_out, np.asarray(out, np.float64)[..., None, :], g)
    return g.reshape(*lead, t, d)


def dequantize_values_sparse(codes, scale, zero, out, idx, group: int = 32) -> np.ndarray:
    """Decoded values float64 ``[..., T, D]``: per-token dense decode, each group's outlier channel restored."""
    *lead, t, d = codes.shape
    g = dequantize_groups_sparse(codes.reshape(*lead, t, d // group, group), scale, zero, out, idx)
    return g.reshape(*lead, t, d)
