"""Packed records of the 4-bit (KVQuant-style) cache, packed and unpacked independently of the library (oracle).

TEST INFRASTRUCTURE ONLY.

A tile is 32 consecutive quantized tokens of one (batch row, KV head) slice; with 4-bit codes (levels 0..15) each
tile is one 5120-byte record:

    bytes    0..2047  key codes,   512 little-endian uint32 words, 8 codes of 4 bits per word
    bytes 2048..4095  value codes, 512 words
    bytes 4096..4351  key scale   s_K[c],      c = 0..127          (binary16)
    bytes 4352..4607  key zero    z_K[c]                           (binary16)
    bytes 4608..4863  value scale s_V[g][t],   g = 0..3, t = 0..31  (binary16, index 32*g + t)
    bytes 4864..5119  value zero  z_V[g][t]                        (binary16)

The code placement is a layout of this library (the pages fix only the code width). Lane l of a 64-lane wavefront
reads the 32 contiguous bytes of words 8 l .. 8 l + 7 of a region:

    key code of token t, channel c:   word = 8 * (c // 8 + 16 * (t // 8)) + t % 8,   bit = 4 * (c % 8)
    value code of channel c, token t: word = 8 * (c // 2) + 4 * (c % 2) + t // 8,    bit = 4 * (t % 8)

so a key word holds 8 channels of one token and a lane owns 8 channels of 8 tokens; a value word holds 8 tokens of
one channel and a lane owns 2 channels of all 32 tokens.

The sink record (one per slice, 512 bytes) holds token 0 when the first token's keys are kept in full precision:

    bytes   0..255  its key, binary16 [128]
    bytes 256..319  its value codes, 4 bits each: channel c at byte 256 + c // 2, bit 4 * (c % 2)
    bytes 320..327  its value scales s_V[g], g = 0..3 (binary16)
    bytes 328..335  its value zeros z_V[g] (binary16)
    bytes 336..511  zero

With per-vector dense-and-sparse quantization (``oracle.sparse``), each tile record grows to 5888 bytes with a
section after the metadata, and the sink record keeps its value outliers in its padding:

    bytes 5120..5375  key outlier values   o_K[c],    c = 0..127          (binary16)
    bytes 5376..5503  key outlier tokens   i_K[c]     (uint8, 0..31, the token within the tile)
    bytes 5504..5759  value outlier values o_V[g][t]  (binary16, index 32*g + t)
    bytes 5760..5887  value outlier channels i_V[g][t] (uint8, 0..31, the channel within group g)
    sink: bytes 336..343 value outlier values o_V[g] (binary16), bytes 344..347 their channels i_V[g] (uint8)
"""
from __future__ import annotations

import numpy as np

TILE_TOKENS = 32
HEAD_DIM = 128
RECORD_BYTES = 5120
K_CODES_OFF, V_CODES_OFF = 0, 2048
K_SCALE_OFF, K_ZERO_OFF = 4096, 4352
V_SCALE_OFF, V_ZERO_OFF = 4608, 4864
SINK_BYTES = 512
RECORD_BYTES_SPARSE = 5888
K_OUT_OFF, K_IDX_OFF, V_OUT_OFF, V_IDX_OFF = 5120, 5376, 5504, 5760


def key_code_position(t: int, c: int) -> tuple[int, int]:
    """(word, bit) of the key code of token ``t`` (0..31) and channel ``c`` within the key-code region."""
    return 8 * (c // 8 + 16 * (t // 8)) + t % 8, 4 * (c % 8)


def value_code_position(t: int, c: int) -> tuple[int, int]:
    """(word, bit) of the value code of channel ``c`` and token ``t`` within the value-code region."""
    return 8 * (c // 2) + 4 * (c % 2) + t // 8, 4 * (t % 8)


def _tables():
    t = np.arange(TILE_TOKENS)[:, None]
    c = np.arange(HEAD_DIM)[None, :]
    kw = 8 * (c // 8 + 16 * (t // 8)) + t % 8
    kb = 4 * (c % 8) + 0 * t
    vw = 8 * (c // 2) + 4 * (c % 2) + t // 8
    vb = 4 * (t % 8) + 0 * c
    return kw, kb, vw, vb


_KW, _KB, _VW, _VB = _tables()


def _pack(codes: np.ndarray, words: np.ndarray, bits: np.ndarray) -> np.ndarray:
    """codes [..., 32, 128] (0..15) -> uint32 [..., 512]; each code OR-ed into its (word, bit)."""
    lead = codes.shape[:-2]
    out = np.zeros(lead + (512,), np.uint64)
    c64 = codes.astype(np.uint64)
    for t in range(TILE_TOKENS):
        for ch in range(HEAD_DIM):
            out[..., words[t, ch]] |= c64[..., t, ch] << np.uint64(bits[t, ch])
    return out.astype(np.uint32)


def _unpack(words32: np.ndarray, words: np.ndarray, bits: np.ndarray) -> np.ndarray:
    w = words32.astype(np.uint64)
    vals = (w[..., words] >> bits.astype(np.uint64)) & np.uint64(15)
    return vals.astype(np.uint8)


def pack_tiles(k_codes, k_scale, k_zero, v_codes, v_scale, v_zero) -> np.ndarray:
    """Build 4-bit tile records. Shapes as for the 2-bit record: codes uint8 ``[..., 32, 128]`` (0..15), key scale
    and zero float16 ``[..., 128]``, value scale and zero float16 ``[..., 32, 4]``. Returns uint8 ``[..., 5120]``."""
    if np.any(np.asarray(k_codes) > 15) or np.any(np.asarray(v_codes) > 15):
        raise ValueError("4-bit codes are 0..15")
    lead = k_codes.shape[:-2]
    rec = np.zeros(lead + (RECORD_BYTES,), dtype=np.uint8)
    rec[..., K_CODES_OFF:K_CODES_OFF + 2048] = np.ascontiguousarray(_pack(k_codes, _KW, _KB), '<u4').view(np.uint8).reshape(lead + (2048,))
    rec[..., V_CODES_OFF:V_CODES_OFF + 2048] = np.ascontiguousarray(_pack(v_codes, _VW, _VB), '<u4').view(np.uint8).reshape(lead + (2048,))
    rec[..., K_SCALE_OFF:K_SCALE_OFF + 256] = np.ascontiguousarray(np.broadcast_to(k_scale, lead + (128,)), np.float16).view(np.uint8).reshape(lead + (256,))
    rec[..., K_ZERO_OFF:K_ZERO_OFF + 256] = np.ascontiguousarray(np.broadcast_to(k_zero, lead + (128,)), np.float16).view(np.uint8).reshape(lead + (256,))
    vs = np.ascontiguousarray(np.swapaxes(np.asarray(v_scale, np.float16), -1, -2))   # [..., 4, 32]
    vz = np.ascontiguousarray(np.swapaxes(np.asarray(v_zero, np.float16), -1, -2))
    rec[..., V_SCALE_OFF:V_SCALE_OFF + 256] = vs.view(np.uint8).reshape(lead + (256,))
    rec[..., V_ZERO_OFF:V_ZERO_OFF + 256] = vz.view(np.uint8).reshape(lead + (256,))
    return rec


def pack_tiles_sparse(k_codes, k_scale, k_zero, v_codes, v_scale, v_zero, k_out, k_idx, v_out, v_idx) -> np.ndarray:
    """5888-byte records: :func:`pack_tiles` plus the outlier section. Key outliers float16 / uint8 ``[..., 128]``
    (one per channel), value outliers ``[..., 32, 4]`` (one per token and channel group)."""
    base = pack_tiles(k_codes, k_scale, k_zero, v_codes, v_scale, v_zero)
    lead = base.shape[:-1]
    rec = np.zeros(lead + (RECORD_BYTES_SPARSE,), dtype=np.uint8)
    rec[..., :RECORD_BYTES] = base
    rec[..., K_OUT_OFF:K_OUT_OFF + 256] = np.ascontiguousarray(np.broadcast_to(np.asarray(k_out, np.float16), lead + (128,))).view(np.uint8).reshape(lead + (256,))
    rec[..., K_IDX_OFF:K_IDX_OFF + 128] = np.broadcast_to(np.asarray(k_idx, np.uint8), lead + (128,))
    vo = np.ascontiguousarray(np.swapaxes(np.asarray(v_out, np.float16), -1, -2))          # [..., 4, 32]
    rec[..., V_OUT_OFF:V_OUT_OFF + 256] = vo.view(np.uint8).reshape(lead + (256,))
    rec[..., V_IDX_OFF:V_IDX_OFF + 128] = np.ascontiguousarray(np.swapaxes(np.asarray(v_idx, np.uint8), -1, -2)).reshape(lead + (128,))
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


def unpack_tiles(rec: np.ndarray):
    """Inverse of :func:`pack_tiles`: (k_codes, k_scale, k_zero, v_codes, v_scale, v_zero)."""
    rec = np.ascontiguousarray(rec, dtype=np.uint8)
    lead = rec.shape[:-1]
    kwords = rec[..., K_CODES_OFF:K_CODES_OFF + 2048].copy().view("<u4").reshape(lead + (512,))
    vwords = rec[..., V_CODES_OFF:V_CODES_OFF + 2048].copy().view("<u4").reshape(lead + (512,))
    k_codes = _unpack(kwords, _KW, _KB)
    v_codes = _unpack(vwords, _VW, _VB)
    k_scale = rec[..., K_SCALE_OFF:K_SCALE_OFF + 256].copy().view(np.float16).reshape(lead + (128,))
    k_zero = rec[..., K_ZERO_OFF:K_ZERO_OFF + 256].copy().view(np.float16).reshape(lead + (128,))
    v_scale = np.swapaxes(rec[..., V_SCALE_OFF:V_SCALE_OFF + 256].copy().view(np.float16).reshape(lead + (4, 32)), -1, -2)
    v_zero = np.swapaxes(rec[..., V_ZERO_OFF:V_ZERO_OFF + 256].copy().view(np.float16).reshape(lead + (4, 32)), -1, -2)
    return k_codes, k_scale, k_zero, v_codes, np.ascontiguousarray(v_scale), np.ascontiguousarray(v_zero)


def pack_sink(k_sink, v_codes, v_scale, v_zero, v_out=None, v_idx=None) -> np.ndarray:
    """Sink records uint8 ``[..., 512]`` from the fp16 key ``[..., 128]``, value codes uint8 ``[..., 128]`` (0..15)
    and value scale / zero float16 ``[..., 4]``; with dense-and-sparse values also the outlier values float16 and
    channels uint8 ``[..., 4]``."""
    k_sink = np.asarray(k_sink, np.float16)
    lead = k_sink.shape[:-1]
    rec = np.zeros(lead + (SINK_BYTES,), np.uint8)
    rec[..., 0:256] = np.ascontiguousarray(k_sink).view(np.uint8).reshape(lead + (256,))
    vc = np.asarray(v_codes, np.uint8)
    rec[..., 256:320] = (vc[..., 0::2] | (vc[..., 1::2] << 4)).astype(np.uint8)
    rec[..., 320:328] = np.ascontiguousarray(np.asarray(v_scale, np.float16)).view(np.uint8).reshape(lead + (8,))
    rec[..., 328:336] = np.ascontiguousarray(np.asarray(v_zero, np.float16)).view(np.uint8).reshape(lead + (8,))
    if v_out is not None:
        rec[..., 336:344] = np.ascontiguousarray(np.asarray(v_out, np.float16)).view(np.uint8).reshape(lead + (8,))
        rec[..., 344:348] = np.asarray(v_idx, np.uint8)
    return rec


def unpack_sink(rec: np.ndarray):
    """Inverse of :func:`pack_sink`: (k_sink float16 [..., 128], v_codes uint8 [..., 128], v_scale, v_zero)."""
    rec = np.ascontiguousarray(rec, dtype=np.uint8)
    lead = rec.shape[:-1]
    k = rec[..., 0:256].copy().view(np.float16).reshape(lead + (128,))
    b = rec[..., 256:320]
    vc = np.empty(lead + (128,), np.uint8)
    vc[..., 0::2] = b & 15
    vc[..., 1::2] = b >> 4
    vs = rec[..., 320:328].copy().view(np.float16).reshape(lead + (4,))
    vz = rec[..., 328:336].copy().view(np.float16).reshape(lead + (4,))
    return k, vc, vs, vz
