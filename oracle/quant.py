"""Asymmetric min/max group quantizer (oracle; test infrastructure only).

What the pages fix: KIVI is an asymmetric quantizer (title of the KIVI page; synthetic.wiki "Sources"), keys are
grouped per channel over 32 tokens and values per token (KIVI page, paragraph on the cache contents;
synthetic.wiki "Keys are harder than values"), and 2 bits is the width on the hot path.

What the pages leave open, and the reading taken here:
- form: uniform levels between the group minimum and maximum, zero-point z = min, scale s = (max - min) / L with
  L = 2**bits - 1, decoded value x_hat = q * s + z;
- precision: s and z are stored as binary16; the code arithmetic is binary32 with round-to-nearest-even at every
  operation and a correctly rounded division; the final rounding to an integer level is half-to-even;
- coverage guard: if rounding s to binary16 left (L + 1/2) * s < max - min (only possible when s is a binary16
  subnormal), s is raised to the next binary16 value, so every element stays within s/2 of its decoded value;
- a zero minimum is stored as +0;
- a constant group stores s = 0 and all codes 0, and never divides.
"""
from __future__ import annotations

import numpy as np


def _rn32(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest binary32 (ties to even), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def quantize_groups(x: np.ndarray, bits: int = 2):
    """Quantize groups laid out along the last axis.

    ``x``: float16 array ``[..., g]`` (finite). Returns ``codes`` uint8 ``[..., g]`` in ``0..2**bits-1``,
    ``scale`` float16 ``[...]`` and ``zero`` float16 ``[...]``.
    """
    x = np.asarray(x)
    if x.dtype != np.float16:
        raise TypeError("quantize_groups expects float16 input")
    xf = x.astype(np.float64)
    if not np.all(np.isfinite(xf)):
        raise ValueError("non-finite input: the quantizer is defined for finite values only")
    levels = (1 << bits) - 1

    # step 1: group minimum and maximum (exact: they are float16 values)
    mn = xf.min(axis=-1)
    mx = xf.max(axis=-1)
    # step 2: range in binary32
    r = _rn32(mx - mn)
    # step 3: scale = range / L, rounded to binary32 then to binary16
    s32 = (r / levels).astype(np.float32)
    scale = np.asarray(s32.astype(np.float16))
    # coverage guard: keep (L + 1/2) * s >= range; the product is exact in float64
    short = (levels + 0.5) * scale.astype(np.float64) < r
    scale = np.where(short, np.nextafter(scale, np.float16(np.inf)), scale).astype(np.float16)
    # step 4: zero-point = minimum, with a zero minimum stored as +0
    zero = np.where(mn == 0, 0.0, mn).astype(np.float16)
    # step 5: codes = clamp(round_half_even(RN32(RN32(x - z) / s)), 0, L); constant groups get 0
    sf = scale.astype(np.float64)[..., None]
    d = _rn32(xf - zero.astype(np.float64)[..., None])
    with np.errstate(divide="ignore", invalid="ignore"):
        t = _rn32(d / np.where(sf == 0, 1.0, sf))
    codes = np.clip(np.rint(t), 0, levels)
    codes = np.where(sf == 0, 0, codes).astype(np.uint8)
    return codes, scale, zero


def dequantize_groups(codes: np.ndarray, scale: np.ndarray, zero: np.ndarray) -> np.ndarray:
    """Decoded values ``q * s + z`` in float64 (exact), groups along the last axis of ``codes``."""
    return codes.astype(np.float64) * scale.astype(np.float64)[..., None] + zero.astype(np.float64)[..., None]


def quantize_keys_per_channel(k: np.ndarray, group: int = 32, bits: int = 2):
    """Per-channel key quantization: each group is ``group`` consecutive tokens of one channel.

    KIVI page, paragraph on the cache contents (a group is 32 tokens of one channel). ``k``: float16
    ``[..., T, D]`` with ``T`` a multiple of ``group``. Returns codes uint8 ``[..., T, D]``, scale and zero float16
    ``[..., T // group, D]``.
    """
    *lead, t, d = k.shape
    if t % group:
        raise ValueError("token count must be a multiple of the group size")
    g = k.reshape(*lead, t // group, group, d)
    g = np.swapaxes(g, -1, -2)                    # [..., tiles, D, group]: the group axis last
    codes, scale, zero = quantize_groups(g, bits)
    codes = np.swapaxes(codes, -1, -2).reshape(*lead, t, d)
    return codes, scale, zero


def quantize_values_per_token(v: np.ndarray, group: int = 32, bits: int = 2):
    """Per-token value quantization: each group is ``group`` consecutive channels of one token.

    KIVI page and synthetic.wiki "Keys are harder than values" (values per token); the group of 32 channels is the
    reading taken for the value group size. ``v``: float16 ``[..., T, D]``. Returns codes uint8 ``[..., T, D]``,
    scale and zero float16 ``[..., T, D // group]``.
    """
    *lead, t, d = v.shape
    if d % group:
        raise ValueError("head_dim must be a multiple of the group size")
    g = v.reshape(*lead, t, d // group, group)
    codes, scale, zero = quantize_groups(g, bits)
    return codes.reshape(*lead, t, d), scale, zero


def dequantize_keys(codes: np.ndarray, scale: np.ndarray, zero: np.ndarray, group: int = 32) -> np.ndarray:
    """Decoded keys float64 ``[..., T, D]`` from per-channel groups."""
    s = np.repeat(scale.astype(np.float64), group, axis=-2)
    z = np.repeat(zero.astype(np.float64), group, axis=-2)
    return codes.astype(np.float64) * s + z


def dequantize_values(codes: np.ndarray, scale: np.ndarray, zero: np.ndarray, group: int = 32) -> np.ndarray:
    """Decoded values float64 ``[..., T, D]`` from per-token groups."""
    s = np.repeat(scale.astype(np.float64), group, axis=-1)
    z = np.repeat(zero.astype(np.float64), group, axis=-1)
    return codes.astype(np.float64) * s + z
