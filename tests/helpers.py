"""Test-side glue: oracle expectations for GPU results (imports the oracle; test infrastructure only)."""
from __future__ import annotations

import numpy as np

import kvsynth
from oracle import attention as oa
from oracle import cache as oc
from oracle import layout


def oracle_records(cache: oc.SliceCache) -> np.ndarray:
    """Tile records [S, n_quant / 32, 3072 (3840 with dense-and-sparse groups)] of the oracle's quantized part,
    packed by the oracle."""
    kq, ks, kz, vq, vs, vz = cache.quantized()
    S, nq, D = kq.shape
    nt = nq // 32
    dense = (kq.reshape(S, nt, 32, D), ks, kz, vq.reshape(S, nt, 32, D), vs.reshape(S, nt, 32, 4),
             vz.reshape(S, nt, 32, 4))
    if not cache.sparse:
        return layout.pack_tiles(*dense)
    ko, ki, vo, vi = cache.outliers()
    return layout.pack_tiles_sparse(*dense, ko, ki, vo.reshape(S, nt, 32, 4), vi.reshape(S, nt, 32, 4))


def records_from_device(tiles, n_tiles: int, slices=None) -> np.ndarray:
    """GPU tile array [B, H, max_tiles, record] -> numpy [S, n_tiles, record] (optionally only slice indices)."""
    B, H = tiles.shape[:2]
    t = tiles[:, :, :n_tiles].reshape(B * H, n_tiles, tiles.shape[-1])
    if slices is not None:
        t = t[list(slices)]
    return t.cpu().numpy()


def first_mismatch(a: np.ndarray, b: np.ndarray) -> str:
    """Describe the first differing byte of two record arrays (slice, tile, field, byte)."""
    idx = np.argwhere(a != b)
    if len(idx) == 0:
        return "identical"
    s, t, off = idx[0][0], idx[0][1], idx[0][-1]
    bounds = [(0, "k_codes"), (1024, "v_codes"), (2048, "k_scale"), (2304, "k_zero"), (2560, "v_scale"),
              (2816, "v_zero"), (3072, "k_outlier"), (3328, "k_outlier_token"), (3456, "v_outlier"),
              (3712, "v_outlier_channel")]
    field = [name for start, name in bounds if off >= start][-1]
    return f"{len(idx)} bytes differ; first at slice {s} tile {t} byte {off} ({field}): gpu {a[tuple(idx[0])]} oracle {b[tuple(idx[0])]}"


def oracle_out(cache: oc.SliceCache, q: np.ndarray, batch: int, kv_heads: int, sm_scale=None) -> np.ndarray:
    return oa.decode_attention(cache, q, batch, kv_heads, sm_scale)


def workload_tokens(w: kvsynth.Workload, tensor_id: int, t0: int, t1: int, b=None, h=None, threads=None):
    """Synthetic K (tensor_id 0, with the workload's outlier channels) or V (1) for tokens [t0, t1)."""
    n_out, factor = (w.k_outliers, w.k_factor) if tensor_id == kvsynth.K_ID else (0, 1.0)
    if b is not None:
        return kvsynth.slice_tokens(w.seed, tensor_id, b, h, t0, t1, w.head_dim, n_out, factor)
    return kvsynth.kv_tensor(w.seed, tensor_id, w.batch, w.kv_heads, t0, t1, w.head_dim, n_out, factor,
                             threads=threads)


def oracle_records4(cache: oc.SliceCache) -> np.ndarray:
    """4-bit tile records [S, n_quant / 32, 5120 (5888 with dense-and-sparse groups)] of the oracle's quantized
    part, packed by the oracle."""
    from oracle import layout4
    kq, ks, kz, vq, vs, vz = cache.quantized()
    S, nq, D = kq.shape
    nt = nq // 32
    dense = (kq.reshape(S, nt, 32, D), ks, kz, vq.reshape(S, nt, 32, D), vs.reshape(S, nt, 32, 4),
             vz.reshape(S, nt, 32, 4))
    if not cache.sparse:
        return layout4.pack_tiles(*dense)
    ko, ki, vo, vi = cache.outliers()
    return layout4.pack_tiles_sparse(*dense, ko, ki, vo.reshape(S, nt, 32, 4), vi.reshape(S, nt, 32, 4))


def oracle_sink(cache: oc.SliceCache) -> np.ndarray:
    """Sink records [S, 512] of the oracle's sink token, packed by the oracle."""
    from oracle import layout4
    vq, vs, vz = cache.v_sink
    if cache.sparse:
        return layout4.pack_sink(cache.k_sink, vq, vs, vz, *cache.v_sink_out)
    return layout4.pack_sink(cache.k_sink, vq, vs, vz)


def records4_from_device(tiles, n_tiles: int, slices=None) -> np.ndarray:
    """GPU 4-bit tile array [B, H, max_tiles, record] -> numpy [S, n_tiles, record]."""
    B, H = tiles.shape[:2]
    t = tiles[:, :, :n_tiles].reshape(B * H, n_tiles, tiles.shape[-1])
    if slices is not None:
        t = t[list(slices)]
    return t.cpu().numpy()


def first_mismatch4(a: np.ndarray, b: np.ndarray) -> str:
    """First differing byte of two 4-bit record arrays (slice, tile, field, byte)."""
    idx = np.argwhere(a != b)
    if len(idx) == 0:
        return "identical"
    off = idx[0][-1]
    bounds = [(0, "k_codes"), (2048, "v_codes"), (4096, "k_scale"), (4352, "k_zero"), (4608, "v_scale"),
              (4864, "v_zero"), (5120, "k_outlier"), (5376, "k_outlier_token"), (5504, "v_outlier"),
              (5760, "v_outlier_channel")]
    field = [name for start, name in bounds if off >= start][-1]
    return f"{len(idx)} bytes differ; first at {tuple(idx[0])} ({field}): gpu {a[tuple(idx[0])]} oracle {b[tuple(idx[0])]}"


def tie_groups_sparse(rng, n_groups: int, levels: int) -> np.ndarray:
    """float16 [n_groups, 32]: a :func:`tie_groups` group with one of its half-level values dropped, plus one
    element of strictly largest magnitude (the outlier) at a random position. The 31 dense elements keep the range
    levels * 2^e, so their quotients land on or beside half levels."""
    base = tie_groups(rng, n_groups, levels).astype(np.float32)
    out = np.empty((n_groups, 32), np.float32)
    for gi in range(n_groups):
        row = base[gi]
        lo, hi = row.min(), row.max()
        inner = np.flatnonzero((row != lo) & (row != hi))
        rest = np.delete(row, inner[int(rng.integers(0, len(inner)))])
        o = (max(abs(lo), abs(hi)) + 4 * (hi - lo) / levels) * (1.0 if rng.integers(0, 2) else -1.0)
        out[gi] = np.insert(rest, int(rng.integers(0, 32)), o)
    h = out.astype(np.float16)
    assert np.array_equal(h.astype(np.float32), out), "sparse tie groups must be exact binary16 values"
    return h


def tie_groups(rng, n_groups: int, levels: int) -> np.ndarray:
    """float16 [n_groups, 32]: groups whose quotients (x - min) / s land exactly on a half level k + 1/2 or one
    binary16 ulp beside it. The scale is a power of two 2^e and the minimum c a multiple of it, with max - min =
    levels * 2^e, so the quantizer's s is exactly 2^e (r / L is exact and a binary16 value); every value is exactly
    representable. Used to exercise the rounding-boundary path of the kernels' quotient."""
    out = np.empty((n_groups, 32), np.float32)
    for gi in range(n_groups):
        e = int(rng.integers(-10, 4))
        s = 2.0 ** e
        c = s * int(rng.integers(-6, 7))
        k = rng.integers(0, levels, 30)
        x = c + (k + 0.5) * s
        ulp = np.spacing(np.abs(x).astype(np.float16)).astype(np.float32)
        x = x + rng.integers(-1, 2, 30) * ulp
        x = np.clip(x, c, c + levels * s)
        row = np.concatenate([[c, c + levels * s], x])
        out[gi] = rng.permutation(row)
    h = out.astype(np.float16)
    assert np.array_equal(h.astype(np.float32), out), "tie groups must be exact binary16 values"
    return h
