"""Rotary position embedding, as the KVQuant variant applies it to dequantized pre-RoPE keys (oracle).

TEST INFRASTRUCTURE ONLY.

synthetic.wiki "KV cache quantization: putting the bits in the cached vectors, not the weights",
section "Keys are harder than values", on pre-RoPE key quantization (KVQuant): the keys are quantized before the rotary embedding is applied, and
the rotation (which turns pairs of channels by a position-dependent angle) is applied after dequantization.

Readings taken where the page is silent: the pairs are adjacent channels (2i, 2i+1)
(the RoFormer form); the angle of pair i at position m is m * theta_i with theta_i = base ** (-2 i / D) and base
10000 unless given; the position of a cached token is its absolute index in the sequence (the first token is
position 0). The stored query is already rotated for its own position, so a score is q . R(m) k for the key of
token m.

Everything here is float64.
"""
from __future__ import annotations

import numpy as np


def frequencies(head_dim: int, base: float = 10000.0) -> np.ndarray:
    """theta_i = base ** (-2 i / D) for the D / 2 channel pairs, float64 ``[D / 2]``."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / head_dim)


def rotate(x: np.ndarray, positions, base: float = 10000.0) -> np.ndarray:
    """R(m) x for vectors ``x`` ``[..., T, D]`` at positions ``m`` ``[T]`` (or a scalar): pair (2i, 2i+1) becomes
    (x0 cos a - x1 sin a, x0 sin a + x1 cos a) with a = m * theta_i."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    m = np.asarray(positions, np.float64)
    ang = m[..., None] * frequencies(d, base) if m.ndim else m * frequencies(d, base)   # [T, D/2] or [D/2]
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out
