"""Pins of the oracle's decode attention over the grouped + residual cache.

- all-residual caches (N <= R) reduce to textbook attention: ``torch.nn.functional.scaled_dot_product_attention``
  in float64 on the CPU over the float16 keys and values;
- special cases with closed forms: one token gives its value row; a zero query gives the mean of the decoded
  values; identical value rows give that row; grid-exact keys/values give textbook attention over the inputs;
- the chunked two-pass evaluation equals a dense softmax (``scipy.special.softmax``) over the fully materialized
  decoded cache, and any split of the tokens merged by the second pass equals it too;
- the refolded algebra (scales and zero-points folded into the query and the probabilities) is the same function;
- the GQA head map (consecutive query heads share a KV head) equals multi-head attention over a cache whose KV
  heads are repeated.
"""
import numpy as np
import pytest
import scipy.special
import torch

from oracle import attention as oa
from oracle import cache as oc
from oracle import quant


def _cache(rng, B, Hkv, N, D=128, outliers=(3, 50), factor=20.0):
    k = rng.standard_normal((B * Hkv, N, D)).astype(np.float32)
    k[:, :, list(outliers)] *= factor
    v = rng.standard_normal((B * Hkv, N, D)).astype(np.float32)
    k, v = k.astype(np.float16), v.astype(np.float16)
    c = oc.SliceCache(B * Hkv, D)
    oc.append_block(c, k, v)
    return c, k, v


def _sdpa64(q, k, v, G):
    """q [B,Hq,D] f16, k/v [B*Hkv, N, D] f16 -> [B,Hq,D] float64 via torch SDPA on the CPU."""
    B, Hq, D = q.shape
    Hkv = k.shape[0] // B
    kk = torch.from_numpy(k.astype(np.float64)).reshape(B, Hkv, -1, D).repeat_interleave(G, dim=1)
    vv = torch.from_numpy(v.astype(np.float64)).reshape(B, Hkv, -1, D).repeat_interleave(G, dim=1)
    qq = torch.from_numpy(q.astype(np.float64)).reshape(B, Hq, 1, D)
    return torch.nn.functional.scaled_dot_product_attention(qq, kk, vv).reshape(B, Hq, D).numpy()


@pytest.mark.parametrize("N,G", [(1, 1), (17, 1), (128, 1), (100, 4)])
def test_all_residual_equals_sdpa(N, G):
    rng = np.random.default_rng(N)
    B, Hkv = 2, 2
    c, k, v = _cache(rng, B, Hkv, N)
    assert c.n_quant == 0 and c.n_resid == N
    q = rng.standard_normal((B, Hkv * G, 128)).astype(np.float16)
    out = oa.decode_attention(c, q, B, Hkv)
    np.testing.assert_allclose(out, _sdpa64(q, k, v, G), rtol=1e-12, atol=1e-12)


def test_one_token_gives_its_value():
    rng = np.random.default_rng(0)
    c, k, v = _cache(rng, 1, 1, 1)
    q = rng.standard_normal((1, 1, 128)).astype(np.float16)
    np.testing.assert_array_equal(oa.decode_attention(c, q, 1, 1)[0, 0], v[0, 0].astype(np.float64))


def test_zero_query_gives_mean_of_decoded_values():
    rng = np.random.default_rng(1)
    c, k, v = _cache(rng, 1, 2, 1000)
    assert c.n_quant == 896
    q = np.zeros((1, 2, 128), np.float16)
    out = oa.decode_attention(c, q, 1, 2)
    # decoded values: codes * s + z per token group; the residual as is
    vq, vs, vz = c.quantized()[3:]
    vhat = np.concatenate([quant.dequantize_values(vq, vs, vz), c.v_res.astype(np.float64)], axis=1)
    np.testing.assert_allclose(out[0], vhat.mean(axis=1), rtol=0, atol=1e-13)
    # the decoded values differ from the inputs by at most half a scale step
    err = np.abs(vhat[:, :896] - v[:, :896].astype(np.float64))
    assert np.all(err <= np.repeat(vs.astype(np.float64), 32, axis=-1) * (0.5 + 2.0 ** -21))


def test_identical_value_rows():
    rng = np.random.default_rng(2)
    N = 700
    k = rng.standard_normal((1, N, 128)).astype(np.float16)
    row = rng.standard_normal(128).astype(np.float16)
    v = np.broadcast_to(row, (1, N, 128)).copy()
    c = oc.SliceCache(1)
    oc.append_block(c, k, v)
    q = rng.standard_normal((1, 1, 128)).astype(np.float16)
    vhat_row = quant.dequantize_values(*quant.quantize_values_per_token(row[None]))[0]
    out = oa.decode_attention(c, q, 1, 1)[0, 0]
    # quantized tokens decode to vhat_row, residual tokens are the row itself: the output lies between them
    lo, hi = np.minimum(vhat_row, row.astype(np.float64)), np.maximum(vhat_row, row.astype(np.float64))
    assert np.all(out >= lo - 1e-12) and np.all(out <= hi + 1e-12)
    # and with a grid-exact row both coincide
    row2 = (np.arange(128) % 4 * 0.5 - 1.0).astype(np.float16)
    v2 = np.broadcast_to(row2, (1, N, 128)).copy()
    c2 = oc.SliceCache(1)
    oc.append_block(c2, k, v2)
    np.testing.assert_allclose(oa.decode_attention(c2, q, 1, 1)[0, 0], row2.astype(np.float64), atol=1e-13)


def test_grid_exact_cache_equals_textbook_attention():
    """Keys and values on an exact 2-bit grid per group decode to themselves, so attention over the quantized
    cache equals textbook attention over the float16 inputs."""
    rng = np.random.default_rng(3)
    N, D = 600, 128
    # keys: per channel and 32-token group, values z + k * s with s a power of two and both ends present
    kc = rng.integers(0, 4, (1, N, D))
    kc[:, ::32, :] = 0
    kc[:, 1::32, :] = 3
    ks = 2.0 ** rng.integers(-4, 2, (1, N // 32 + 1, D))
    kz = rng.integers(-8, 8, (1, N // 32 + 1, D)) * ks
    k = kz.repeat(32, 1)[:, :N] + kc * ks.repeat(32, 1)[:, :N]
    vc = rng.integers(0, 4, (1, N, D))
    vc[:, :, ::32] = 0
    vc[:, :, 1::32] = 3
    vs = 2.0 ** rng.integers(-4, 2, (1, N, D // 32))
    vz = rng.integers(-8, 8, (1, N, D // 32)) * vs
    v = vz.repeat(32, -1) + vc * vs.repeat(32, -1)
    k16, v16 = k.astype(np.float16), v.astype(np.float16)
    assert np.array_equal(k16.astype(np.float64), k) and np.array_equal(v16.astype(np.float64), v)
    c = oc.SliceCache(1)
    oc.append_block(c, k16, v16)
    q = rng.standard_normal((1, 1, D)).astype(np.float16)
    np.testing.assert_allclose(oa.decode_attention(c, q, 1, 1), _sdpa64(q, k16, v16, 1), rtol=1e-12, atol=1e-12)


def _dense(c, q, B, Hkv, sigma=None):
    D = q.shape[-1]
    sigma = 1 / np.sqrt(D) if sigma is None else sigma
    K, V = oa.decoded_range(c, 0, c.n_tokens)
    G = q.shape[1] // Hkv
    out = np.empty(q.shape, np.float64)
    for b in range(B):
        for hq in range(q.shape[1]):
            s = b * Hkv + hq // G
            w = scipy.special.softmax(sigma * (K[s] @ q[b, hq].astype(np.float64)))
            out[b, hq] = w @ V[s]
    return out


def test_chunked_equals_dense_softmax_and_splits_merge():
    rng = np.random.default_rng(4)
    B, Hkv, G, N = 2, 2, 2, 1000
    c, _, _ = _cache(rng, B, Hkv, N)
    q = rng.standard_normal((B, Hkv * G, 128)).astype(np.float16)
    dense = _dense(c, q, B, Hkv)
    np.testing.assert_allclose(oa.decode_attention(c, q, B, Hkv), dense, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oa.decode_attention(c, q, B, Hkv, chunk=37), dense, rtol=1e-12, atol=1e-12)
    for bounds in ([(0, N)], [(0, 300), (300, 301), (301, N)], [(0, 0), (0, 896), (896, N), (N, N)],
                   [(i, min(N, i + 96)) for i in range(0, N, 96)]):
        m, l, o = oa.split_partials(c, q, B, Hkv, bounds)
        merged = oa.merge_partials(m, l, o).reshape(B, Hkv * G, 128)
        np.testing.assert_allclose(merged, dense, rtol=1e-12, atol=1e-12)
    # a caller-given scale
    np.testing.assert_allclose(oa.decode_attention(c, q, B, Hkv, sm_scale=0.3), _dense(c, q, B, Hkv, 0.3),
                               rtol=1e-12, atol=1e-12)


def test_refolded_algebra_is_the_same_function():
    rng = np.random.default_rng(5)
    B, Hkv, G, N = 1, 2, 4, 640
    c, _, _ = _cache(rng, B, Hkv, N)
    q = rng.standard_normal((B, Hkv * G, 128)).astype(np.float16)
    nq = c.n_quant
    K, V = oa.decoded_range(c, 0, nq)
    qs = q.astype(np.float64).reshape(B * Hkv, G, 128)
    direct = np.einsum("sgd,std->sgt", qs, K) / np.sqrt(128)
    np.testing.assert_allclose(oa.refolded_scores(c, q, B, Hkv), direct, rtol=1e-12, atol=1e-10)
    p = np.exp(direct - direct.max(-1, keepdims=True))
    np.testing.assert_allclose(oa.refolded_values(c, p), np.einsum("sgt,std->sgd", p, V), rtol=1e-12, atol=1e-10)


def test_gqa_head_map_consecutive_heads():
    rng = np.random.default_rng(6)
    B, Hkv, G, N = 2, 2, 4, 300
    c, k, v = _cache(rng, B, Hkv, N)
    q = rng.standard_normal((B, Hkv * G, 128)).astype(np.float16)
    out = oa.decode_attention(c, q, B, Hkv)
    # multi-head cache with every KV head repeated G times in a row
    rep = oc.SliceCache(B * Hkv * G)
    kr = np.repeat(k.reshape(B, Hkv, N, 128), G, axis=1).reshape(B * Hkv * G, N, 128)
    vr = np.repeat(v.reshape(B, Hkv, N, 128), G, axis=1).reshape(B * Hkv * G, N, 128)
    oc.append_block(rep, kr, vr)
    np.testing.assert_allclose(out, oa.decode_attention(rep, q, B, Hkv * G), rtol=1e-13, atol=1e-13)


def test_empty_cache_rejected():
    c = oc.SliceCache(1)
    with pytest.raises(ValueError):
        oa.decode_attention(c, np.zeros((1, 1, 128), np.float16), 1, 1)
