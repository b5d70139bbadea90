"""The packed tile record of the 2-bit cache, packed and unpacked independently of the library (oracle).

TEST INFRASTRUCTURE ONLY.

A tile is 32 consecutive quantized tokens of one (batch row, KV head) slice. Each tile is one 3072-byte record:

    bytes    0..1023  key codes,   256 little-endian uint32 words
    bytes 1024..2047  value codes, 256 little-endian uint32 words
    bytes 2048..2303  key scale   s_K[c],      c = 0..127          (binary16)
    bytes 2304..2559  key zero    z_K[c]                           (binary16)
    bytes 2560..2815  value scale s_V[g][t],   g = 0..3, t = 0..31  (binary16, index 32*g + t)
    bytes 2816..3071  value zero  z_V[g][t]                        (binary16)

With dense-and-sparse groups (one outlier per 32-element group, see ``oracle.sparse``) a record is 3840 bytes: the
3072 above, then the outlier section

    bytes 3072..3327  key outlier value   o_K[c],  c = 0..127          (binary16)
    bytes 3328..3455  key outlier token   u_K[c]                       (uint8, 0..31)
    bytes 3456..3711  value outlier value o_V[g][t]                    (binary16, index 32*g + t)
    bytes 3712..3839  value outlier channel i_V[g][t] within group g   (uint8, 0..31)

and the outlier's own code is 0. 3840 = 15 * 256 keeps records 256-byte aligned.

A word holds 16 codes of 2 bits. Word w of a code region is read by lane w // 4 of a 64-lane wavefront and the
code placement is fixed by the functions below (a layout of this library, not of the pages; it is defined so
each lane reads 16 contiguous bytes and expands them with byte-wise fp4 conversions).

Key code of token t (0..31), channel c (0..127):
    m = t // 16, n = t % 16, ks = c // 32, kc = (c % 32) // 8, e = c % 8
    word = 4 * (n + 16 * kc) + 2 * m + ks // 2,   bit = 4 * e + 2 * (ks % 2)
Value code of channel c, token t:
    j = c // 16, cc = c % 16
    (kc, e) = (t // 4, t % 4) if t < 16 else ((t - 16) // 4, 4 + (t - 16) % 4)
    word = 4 * (cc + 16 * kc) + j // 2,           bit = 4 * e + 2 * (j % 2)
"""
from __future__ import annotations

import numpy as np

TILE_TOKENS = 32
HEAD_DIM = 128
RECORD_BYTES = 3072
K_CODES_OFF, V_CODES_OFF = 0, 1024
K_SCALE_OFF, K_ZERO_OFF = 2048, 2304
V_SCALE_OFF, V_ZERO_OFF = 2560, 2816
RECORD_BYTES_SPARSE = 3840
K_OUT_OFF, K_IDX_OFF, V_OUT_OFF, V_IDX_OFF = 3072, 3328, 3456, 3712


def key_code_position(t: int, c: int) -> tuple[int, int]:
    """(word, bit) of the key code of token ``t`` and channel ``c`` within the key-code region."""
    m, n = t // 16, t % 16
    ks, kc, e = c // 32, (c % 32) // 8, c % 8
    return 4 * (n + 16 * kc) + 2 * m + ks // 2, 4 * e + 2 * (ks % 2)


def value_code_position(t: int, c: int) -> tuple[int, int]:
    """(word, bit) of the value code of channel ``c`` and token ``t`` within the value-code region."""
    j, cc = c // 16, c % 16
    if t < 16:
        kc, e = t // 4, t % 4
    else:
        kc, e = (t - 16) // 4, 4 + (t - 16) % 4
    return 4 * (cc + 16 * kc) + j // 2, 4 * e + 2 * (j % 2)


def _tables():
    kw = np.empty((TILE_TOKENS, HEAD_DIM), np.int64)
    kb = np.empty_like(kw)
    vw = np.empty_like(kw)
    vb = np.empty_like(kw)
    for t in range(TILE_TOKENS):
        for c in range(HEAD_DIM):
            kw[t, c], kb[t, c] = key_code_position(t, c)
            vw[t, c], vb[t, c] = value_code_position(t, c)
    return kw, kb, vw, vb


_KW, _KB, _VW, _VB = _tables()


def _word_sources(words: np.ndarray, bits: np.ndarray):
    """For each of the 256 words, the 16 flat code indices it holds and their bit offsets."""
    idx = np.full((256, 16), -1, np.int64)
    sh = np.zeros((256, 16), np.int64)
    fill = np.zeros(256, np.int64)
    for i, (w, b) in enumerate(zip(words.reshape(-1), bits.reshape(-1))):
        idx[w, fill[w]] = i
        sh[w, fill[w]] = b
        fill[w] += 1
    if not np.all(fill == 16):
        raise AssertionError("code placement is not a bijection onto 256 words x 16 slots")
    return idx, sh


_KSRC = _word_sources(_KW, _KB)
_VSRC = _word_sources(_VW, _VB)


def _pack_words(codes: np.ndarray, src) -> np.ndarray:
    """codes [..., 32, 128] (0..3) -> uint32 [..., 256] with each code at its (word, bit)."""
    idx, sh = src
    lead = codes.shape[:-2]
    flat = codes.reshape(lead + (-1,)).astype(np.uint64)
    parts = flat[..., idx] << sh.astype(np.uint64)           # [..., 256, 16]
    return np.bitwise_or.reduce(parts, axis=-1).astype(np.uint32)


def _unpack_words(words32: np.ndarray, words: np.ndarray, bits: np.ndarray) -> np.ndarray:
    lead = words32.shape[:-1]
    w = words32.astype(np.uint64)
    vals = (w[..., words.reshape(-1)] >> bits.reshape(-1).astype(np.uint64)) & np.uint64(3)
    return vals.reshape(lead + (TILE_TOKENS, HEAD_DIM)).astype(np.uint8)


def pack_tiles(k_codes, k_scale, k_zero, v_codes, v_scale, v_zero) -> np.ndarray:
    """Build tile records.

    Inputs per tile (leading dims ``...`` shared): ``k_codes``/``v_codes`` uint8 ``[..., 32, 128]``;
    ``k_scale``/``k_zero`` float16 ``[..., 128]``; ``v_scale``/``v_zero`` float16 ``[..., 32, 4]``
    (per token, per 32-channel group). Returns uint8 ``[..., 3072]``.
    """
    lead = k_codes.shape[:-2]
    rec = np.zeros(lead + (RECORD_BYTES,), dtype=np.uint8)
    rec[..., K_CODES_OFF:K_CODES_OFF + 1024] = np.ascontiguousarray(_pack_words(k_codes, _KSRC), '<u4').view(np.uint8).reshape(lead + (1024,))
    rec[..., V_CODES_OFF:V_CODES_OFF + 1024] = np.ascontiguousarray(_pack_words(v_codes, _VSRC), '<u4').view(np.uint8).reshape(lead + (1024,))
    rec[..., K_SCALE_OFF:K_SCALE_OFF + 256] = np.ascontiguousarray(np.broadcast_to(k_scale, lead + (128,)), np.float16).view(np.uint8).reshape(lead + (256,))
    rec[..., K_ZERO_OFF:K_ZERO_OFF + 256] = np.ascontiguousarray(np.broadcast_to(k_zero, lead + (128,)), np.float16).view(np.uint8).reshape(lead + (256,))
    vs = np.ascontiguousarray(np.swapaxes(np.asarray(v_scale, np.float16), -1, -2))   # [..., 4, 32]
    vz = np.ascontiguousarray(np.swapaxes(np.asarray(v_zero, np.float16), -1, -2))
    rec[..., V_SCALE_OFF:V_SCALE_OFF + 256] = vs.view(np.uint8).reshape(lead + (256,))
    rec[..., V_ZERO_OFF:V_ZERO_OFF + 256] = vz.view(np.uint8).reshape(lead + (256,))
    return rec


def unpack_tiles(rec: np.ndarray):
    """Inverse of :func:`pack_tiles`: returns (k_codes, k_scale, k_zero, v_codes, v_scale, v_zero)."""
    rec = np.ascontiguousarray(rec, dtype=np.uint8)
    lead = rec.shape[:-1]
    kwords = rec[..., K_CODES_OFF:K_CODES_OFF + 1024].copy().view("<u4").reshape(lead + (256,))
    vwords = rec[..., V_CODES_OFF:V_CODES_OFF + 1024].copy().view("<u4").reshape(lead + (256,))
    k_codes = _unpack_words(kwords, _KW, _KB)
    v_codes = _unpack_words(vwords, _VW, _VB)
    k_scale = rec[..., K_SCALE_OFF:K_SCALE_OFF + 256].copy().view(np.float16).reshape(lead + (128,))
    k_zero = rec[..., K_ZERO_OFF:K_ZERO_OFF + 256].copy().view(np.float16).reshape(lead + (128,))
    v_scale = np.swapaxes(rec[..., V_SCALE_OFF:V_SCALE_OFF + 256].copy().view(np.float16).reshape(lead + (4, 32)), -1, -2)
    v_zero = np.swapaxes(rec[..., V_ZERO_OFF:V_ZERO_OFF + 256].copy().view(np.float16).reshape(lead + (4, 32)), -1, -2)
    return k_codes, k_scale, k_zero, v_codes, np.ascontiguousarray(v_scale), np.ascontiguousarray(v_zero)


def pack_tiles_sparse(k_codes, k_scale, k_zero, v_codes, v_scale, v_zero, k_out, k_idx, v_out, v_idx) -> np.ndarray:
    """3840-byte records: :func:`pack_tiles` plus the outlier section. Key outliers float16 / uint8 ``[..., 128]``
    (one per channel: value and token), value outliers ``[..., 32, 4]`` (one per token and channel group: value and
    channel within the group)."""
    base = pack_tiles(k_codes, k_scale, k_zero, v_codes, v_scale, v_zero)
    lead = base.shape[:-1]
    rec = np.zeros(lead + (RECORD_BYTES_SPARSE,), dtype=np.uint8)
    rec[..., :RECORD_BYTES] = base
    rec[..., K_OUT_OFF:K_OUT_OFF + 256] = np.ascontiguousarray(
        np.broadcast_to(np.asarray(k_out, np.float16), lead + (128,))).view(np.uint8).reshape(lead + (256,))
    rec[..., K_IDX_OFF:K_IDX_OFF + 128] = np.broadcast_to(np.asarray(k_idx, np.uint8), lead + (128,))
    vo = np.ascontiguousarray(np.swapaxes(np.asarray(v_out, np.float16), -1, -2))          # [..., 4, 32]
    rec[..., V_OUT_OFF:V_OUT_OFF + 256] = vo.view(np.uint8).reshape(lead + (256,))
    rec[..., V_IDX_OFF:V_IDX_OFF + 128] = np.ascontiguousarray(
        np.swapaxes(np.asarray(v_idx, np.uint8), -1, -2)).reshape(lead + (128,))
    return rec


def unpack_tiles_sparse(rec: np.ndarray):
    """Inverse of :func:`pack_tiles_sparse`: the six dense fields, then (k_out, k_idx, v_out, v_idx)."""
    rec = np.ascontiguousarray(rec, dtype=np.uint8)
    lead = rec.shape[:-1]
    dense = unpack_tiles(rec[..., :RECORD_BYTES])
    k_out = rec[..., K_OUT_OFF:K_OUT_OFF + 256].copy().view(np.float16).reshape(lead + (128,))
    k_idx = rec[..., K_IDX_OFF:K_IDX_OFF + 128].copy()
    v_out = np.swapaxes(rec[..., V_OUT_OFF:V_OUT_OFF + 256].copy().view(np.float16).reshape(lead + (4, 32)), -1, -2)
    v_idx = np.swapaxes(rec[..., V_IDX_OFF:V_IDX_OFF + 128].copy().reshape(lead + (4, 32)), -1, -2)
    return dense + (k_out, k_idx, np.ascontiguousarray(v_out), np.ascontiguousarray(v_idx))
