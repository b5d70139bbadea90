"""Decode attention over the decoded grouped + residual cache (oracle; test infrastructure only).

synthetic.wiki "Keys are harder than values", last bullet: attention scores combine the grouped key part and the
residual key part. Decoding reaches exactly (up to rounding order) plain softmax attention over the decoded cache,
so this module writes that definition out in float64:

    K_hat[t, c] = code_K[t, c] * s_K[c, t // 32] + z_K[c, t // 32]      (t < n_quant)
    V_hat[t, c] = code_V[t, c] * s_V[t, c // 32] + z_V[t, c // 32]      (t < n_quant)
    K_hat[t], V_hat[t] = the float16 residual tokens, widened              (n_quant <= t < N)
    score_t = sigma * sum_c q_c K_hat[t, c],  out = sum_t softmax(score)_t V_hat[t]

Readings taken where the pages are silent: sigma = 1/sqrt(head_dim) unless the caller gives another scale; query
head hq uses KV head hq // G with G = Hq / Hkv (consecutive query heads share a KV head); the output is float64
here and float32 in the library.

KVQuant variant: with a sink, token 0 is the sink (its float16 key, its value decoded from per-token codes); with
``rope_base`` set the cached keys are pre-RoPE and every decoded key is rotated by its absolute position before the
dot product (see ``rope``): score_t = sigma * sum_c q_c (R(t) K_hat[t])_c. With dense-and-sparse groups the decoded
keys and values hold each group's outlier at its index (``oracle.sparse``).

Long caches are processed in token chunks (two passes: the global maximum first, then the exponential sums), so
a million-token slice never materializes in float64 all at once.
"""
from __future__ import annotations

import numpy as np

from . import quant, rope, sparse as dsq
from .cache import SliceCache

CHUNK = 65536


def decoded_range(cache: SliceCache, t0: int, t1: int):
    """Decoded keys and values of tokens ``[t0, t1)`` (absolute indices, the sink first) of every slice, float64
    ``[S, t1 - t0, D]``."""
    g = cache.group
    ns = cache.n_sink
    S, D = cache.slices, cache.head_dim
    K = np.empty((S, t1 - t0, D), np.float64)
    V = np.empty((S, t1 - t0, D), np.float64)
    if ns and t0 == 0 and t1 > 0:      # token 0 is the sink
        vq, vs, vz = cache.v_sink
        K[:, 0] = cache.k_sink.astype(np.float64)
        if cache.sparse:
            vo, vi = cache.v_sink_out
            V[:, 0] = dsq.dequantize_values_sparse(vq[:, None], vs[:, None], vz[:, None], vo[:, None], vi[:, None],
                                                   g)[:, 0]
        else:
            V[:, 0] = quant.dequantize_values(vq[:, None], vs[:, None], vz[:, None], g)[:, 0]
    a0, b0 = max(t0, ns), t1            # absolute range after the sink
    if b0 <= a0:
        return K, V
    kq, ks, kz, vq, vs, vz = cache.quantized()
    nq = cache.n_quant
    a, b = a0 - ns, min(b0 - ns, nq)    # indices into the quantized part
    off = a0 - t0
    if b > a:
        # expand to whole key groups so the per-channel scale of each token is indexed by its group
        ga, gb = a // g, (b + g - 1) // g
        if cache.sparse:
            ko, ki, vo, vi = cache.outliers()
            kh = dsq.dequantize_keys_sparse(kq[:, ga * g:gb * g], ks[:, ga:gb], kz[:, ga:gb], ko[:, ga:gb],
                                            ki[:, ga:gb], g)
            V[:, off:off + b - a] = dsq.dequantize_values_sparse(vq[:, a:b], vs[:, a:b], vz[:, a:b], vo[:, a:b],
                                                                 vi[:, a:b], g)
        else:
            kh = quant.dequantize_keys(kq[:, ga * g:gb * g], ks[:, ga:gb], kz[:, ga:gb], g)
            V[:, off:off + b - a] = quant.dequantize_values(vq[:, a:b], vs[:, a:b], vz[:, a:b], g)
        K[:, off:off + b - a] = kh[:, a - ga * g:b - ga * g]
    a2 = max(a0 - ns, nq)
    if b0 - ns > a2:
        o2 = a2 + ns - t0
        K[:, o2:] = cache.k_res[:, a2 - nq:b0 - ns - nq].astype(np.float64)
        V[:, o2:] = cache.v_res[:, a2 - nq:b0 - ns - nq].astype(np.float64)
    return K, V


def _q_for_slices(q: np.ndarray, batch: int, kv_heads: int) -> np.ndarray:
    """float16 [B, Hq, D] -> float64 [S = B*Hkv, G, D] (query heads grouped by the KV head they use)."""
    B, Hq, D = q.shape
    G = Hq // kv_heads
    return q.astype(np.float64).reshape(B, kv_heads, G, D).reshape(B * kv_heads, G, D)


def decode_attention(cache: SliceCache, q: np.ndarray, batch: int, kv_heads: int, sm_scale: float | None = None,
                     chunk: int = CHUNK, rope_base: float | None = None) -> np.ndarray:
    """Attention output float64 ``[B, Hq, D]`` of query ``q`` (float16 ``[B, Hq, D]``) over the whole cache.

    Slice index of (b, hkv) is ``b * kv_heads + hkv``. With ``rope_base`` the decoded keys are rotated by their
    absolute positions (pre-RoPE key cache).
    """
    def keys(t0, t1):
        K, V = decoded_range(cache, t0, t1)
        if rope_base is not None:
            K = rope.rotate(K, np.arange(t0, t1), rope_base)
        return K, V

    B, Hq, D = q.shape
    if cache.slices != batch * kv_heads or Hq % kv_heads:
        raise ValueError("cache slices must be batch * kv_heads and Hq a multiple of kv_heads")
    if cache.n_tokens == 0:
        raise ValueError("attention over an empty cache is undefined")
    sigma = 1.0 / np.sqrt(D) if sm_scale is None or sm_scale <= 0 else float(sm_scale)
    qs = _q_for_slices(q, batch, kv_heads)                       # [S, G, D]
    N = cache.n_tokens
    S, G = qs.shape[0], qs.shape[1]
    # pass 1: global maximum of the scores
    m = np.full((S, G), -np.inf)
    for t0 in range(0, N, chunk):
        K, _ = keys(t0, min(N, t0 + chunk))
        sc = sigma * np.matmul(qs, np.swapaxes(K, 1, 2))
        m = np.maximum(m, sc.max(axis=-1))
    # pass 2: exponential sums and the weighted sum of values
    l = np.zeros((S, G))
    acc = np.zeros((S, G, D))
    for t0 in range(0, N, chunk):
        K, V = keys(t0, min(N, t0 + chunk))
        sc = sigma * np.matmul(qs, np.swapaxes(K, 1, 2))
        p = np.exp(sc - m[..., None])
        l += p.sum(axis=-1)
        acc += np.matmul(p, V)
    out = acc / l[..., None]
    return out.reshape(batch, kv_heads, G, D).reshape(batch, Hq, D)


def refolded_scores(cache: SliceCache, q: np.ndarray, batch: int, kv_heads: int, sm_scale: float | None = None):
    """Scores over the quantized part computed with scales and zero-points folded into the query.

    score_t = sigma * (sum_c (q_c * s_K[c, j]) * code_K[t, c] + sum_c q_c * z_K[c, j]),  j = t // 32.
    This is the algebra a fused kernel uses instead of decoding the keys; float64 ``[S, G, n_quant]``.
    """
    D = q.shape[-1]
    sigma = 1.0 / np.sqrt(D) if sm_scale is None or sm_scale <= 0 else float(sm_scale)
    qs = _q_for_slices(q, batch, kv_heads)
    kq, ks, kz, _, _, _ = cache.quantized()
    nt = kq.shape[1] // cache.group
    codes = kq.astype(np.float64).reshape(cache.slices, nt, cache.group, D)
    qt = qs[:, :, None, :] * ks.astype(np.float64)[:, None, :, :]          # [S, G, tiles, D]
    beta = np.einsum("sgd,sjd->sgj", qs, kz.astype(np.float64))            # [S, G, tiles]
    sc = np.einsum("sgjd,sjtd->sgjt", qt, codes) + beta[..., None]
    return sigma * sc.reshape(cache.slices, qs.shape[1], nt * cache.group)


def refolded_values(cache: SliceCache, p: np.ndarray) -> np.ndarray:
    """sum_t p_t V_hat[t] over the quantized part with value scales folded into p.

    sum_t (p_t * s_V[t, g]) * code_V[t, c] + sum_t p_t * z_V[t, g],  g = c // 32.  ``p``: ``[S, G, n_quant]``.
    """
    _, _, _, vq, vs, vz = cache.quantized()
    S, nq, D = vq.shape
    gsz = cache.group
    ng = D // gsz
    codes = vq.astype(np.float64).reshape(S, nq, ng, gsz)
    pt = p[..., None] * vs.astype(np.float64)[:, None, :, :]               # [S, G, nq, ng]
    main = np.einsum("sgtk,stkc->sgkc", pt, codes)
    zterm = np.einsum("sgt,stk->sgk", p, vz.astype(np.float64))
    return (main + zterm[..., None]).reshape(S, p.shape[1], D)


def split_partials(cache: SliceCache, q: np.ndarray, batch: int, kv_heads: int, bounds, sm_scale=None):
    """Per-split (m, l, o) over token ranges ``bounds`` = [(t0, t1), ...]; empty ranges give (-inf, 0, 0).

    m is the maximum score of the range, l = sum exp(score - m), o = sum exp(score - m) V_hat (unnormalized).
    """
    D = q.shape[-1]
    sigma = 1.0 / np.sqrt(D) if sm_scale is None or sm_scale <= 0 else float(sm_scale)
    qs = _q_for_slices(q, batch, kv_heads)
    S, G = qs.shape[:2]
    ms, ls, os_ = [], [], []
    for t0, t1 in bounds:
        if t1 <= t0:
            ms.append(np.full((S, G), -np.inf)); ls.append(np.zeros((S, G))); os_.append(np.zeros((S, G, D)))
            continue
        K, V = decoded_range(cache, t0, t1)
        sc = sigma * np.matmul(qs, np.swapaxes(K, 1, 2))
        m = sc.max(axis=-1)
        p = np.exp(sc - m[..., None])
        ms.append(m); ls.append(p.sum(-1)); os_.append(np.matmul(p, V))
    return np.stack(ms), np.stack(ls), np.stack(os_)


def merge_partials(m: np.ndarray, l: np.ndarray, o: np.ndarray) -> np.ndarray:
    """Second pass: out = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s with M = max_s m_s; -inf splits drop out."""
    M = m.max(axis=0)
    w = np.where(np.isneginf(m), 0.0, np.exp(m - M))
    return (w[..., None] * o).sum(0) / (w * l).sum(0)[..., None]
