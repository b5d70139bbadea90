"""Pins of the KVQuant-style oracle pieces: rotary embedding, 4-bit tile and sink records, the sink cache, and
attention over a pre-RoPE 4-bit cache with a sink.

Sources: synthetic.wiki "KV cache quantization: putting the bits in the cached vectors, not the weights": section
"Keys are harder than values" (keys quantized before RoPE with the rotation applied after dequantization) and
section "What they report" (the first token's keys kept in full precision); 4-bit codes. Each pin checks the oracle against something other than its own formula:
closed forms, group laws of rotations, a brute-force per-token loop with explicit 2x2 rotation matrices, and
special cases that reduce to the plain (already pinned) attention path.
"""
import numpy as np
import pytest

from oracle import attention as oa
from oracle import cache as oc
from oracle import layout4
from oracle import quant
from oracle import rope


# ------------------------------------------------------------------ rotary embedding
def test_frequencies_endpoints():
    th = rope.frequencies(128, 10000.0)
    assert th.shape == (64,)
    assert th[0] == 1.0
    assert np.isclose(th[-1], 10000.0 ** (-126.0 / 128.0), rtol=1e-15)
    assert np.all(np.diff(th) < 0)
    assert np.array_equal(rope.frequencies(2, 10000.0), [1.0])


def test_basis_vectors_closed_form():
    # pair 0 turns by m radians (theta_0 = 1): e0 -> (cos m, sin m), e1 -> (-sin m, cos m)
    for m in [0, 1, 3, 17, 1000]:
        e0 = np.zeros(8); e0[0] = 1.0
        e1 = np.zeros(8); e1[1] = 1.0
        r0, r1 = rope.rotate(e0, m), rope.rotate(e1, m)
        assert np.allclose(r0, [np.cos(m), np.sin(m), 0, 0, 0, 0, 0, 0], atol=1e-15)
        assert np.allclose(r1, [-np.sin(m), np.cos(m), 0, 0, 0, 0, 0, 0], atol=1e-15)


def test_pairs_are_adjacent_channels():
    # energy in channels (2i, 2i+1) stays there; the split-halves convention (i, i + D/2) would move it
    rng = np.random.default_rng(1)
    for i in [0, 5, 31, 63]:
        x = np.zeros(128)
        x[2 * i], x[2 * i + 1] = rng.standard_normal(2)
        y = rope.rotate(x, 12345)
        mask = np.ones(128, bool); mask[[2 * i, 2 * i + 1]] = False
        assert np.all(y[mask] == 0)
        assert np.isclose(np.hypot(y[2 * i], y[2 * i + 1]), np.hypot(x[2 * i], x[2 * i + 1]), rtol=1e-14)


def test_block_rotation_matrix():
    # the same map as an explicit block-diagonal matrix built from 2x2 rotations
    D, base = 16, 500.0
    th = base ** (-2.0 * np.arange(D // 2) / D)
    x = np.random.default_rng(2).standard_normal((5, D))
    pos = np.array([0, 1, 7, 100, 4095])
    for t in range(5):
        M = np.zeros((D, D))
        for i in range(D // 2):
            a = pos[t] * th[i]
            M[2 * i:2 * i + 2, 2 * i:2 * i + 2] = [[np.cos(a), -np.sin(a)], [np.sin(a), np.cos(a)]]
        assert np.allclose(rope.rotate(x[t], pos[t], base), M @ x[t], atol=1e-13)
    assert np.allclose(rope.rotate(x, pos, base)[3], rope.rotate(x[3], pos[3], base), atol=0)


def test_group_laws():
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal((2, 128))
    assert np.array_equal(rope.rotate(q, 0), q)
    a, b = 37, 2048
    assert np.allclose(rope.rotate(rope.rotate(q, a), b), rope.rotate(q, a + b), atol=1e-12)
    # relative position: <R(m) q, R(n) k> depends on m - n only
    lhs = rope.rotate(q, 900) @ rope.rotate(k, 650)
    rhs = rope.rotate(q, 250) @ k
    assert np.isclose(lhs, rhs, rtol=1e-11)
    assert np.isclose(np.linalg.norm(rope.rotate(q, 999)), np.linalg.norm(q), rtol=1e-14)


# ------------------------------------------------------------------ 4-bit records
def test_4bit_code_placement_is_a_bijection():
    seen = set()
    for t in range(32):
        for c in range(128):
            for w, b in (layout4.key_code_position(t, c),):
                assert 0 <= w < 512 and b in range(0, 32, 4)
                assert ("k", w, b) not in seen
                seen.add(("k", w, b))
            w, b = layout4.value_code_position(t, c)
            assert 0 <= w < 512 and b in range(0, 32, 4)
            assert ("v", w, b) not in seen
            seen.add(("v", w, b))
    assert len(seen) == 2 * 32 * 128


def test_4bit_lane_ownership():
    # lane l reads words 8l..8l+7: keys of channels 8 (l % 16) .. and tokens 8 (l // 16) ..; values of channels 2l, 2l+1
    for t in range(32):
        for c in range(128):
            lane = layout4.key_code_position(t, c)[0] // 8
            assert lane == c // 8 + 16 * (t // 8)
            lane = layout4.value_code_position(t, c)[0] // 8
            assert lane == c // 2


def test_4bit_record_round_trip_and_offsets():
    rng = np.random.default_rng(4)
    kc = rng.integers(0, 16, (3, 32, 128)).astype(np.uint8)
    vc = rng.integers(0, 16, (3, 32, 128)).astype(np.uint8)
    ks, kz = rng.standard_normal((2, 3, 128)).astype(np.float16)
    vs, vz = rng.standard_normal((2, 3, 32, 4)).astype(np.float16)
    rec = layout4.pack_tiles(kc, ks, kz, vc, vs, vz)
    assert rec.shape == (3, 5120)
    for a, b in zip(layout4.unpack_tiles(rec), (kc, ks, kz, vc, vs, vz)):
        assert np.array_equal(a, b)
    # a single code lands in exactly one nibble of the record
    one = np.zeros((32, 128), np.uint8)
    one[9, 77] = 0xB
    r = layout4.pack_tiles(one, np.zeros(128, np.float16), np.zeros(128, np.float16), np.zeros_like(one),
                           np.zeros((32, 4), np.float16), np.zeros((32, 4), np.float16))
    w, b = layout4.key_code_position(9, 77)
    byte = 4 * w + b // 8
    assert np.flatnonzero(r).tolist() == [byte] and r[byte] == (0xB << (b % 8))
    with pytest.raises(ValueError):
        layout4.pack_tiles(one + 16, ks[0], kz[0], one, vs[0], vz[0])


def test_sink_record_round_trip():
    rng = np.random.default_rng(5)
    k = rng.standard_normal((4, 128)).astype(np.float16)
    vc = rng.integers(0, 16, (4, 128)).astype(np.uint8)
    vs, vz = rng.standard_normal((2, 4, 4)).astype(np.float16)
    rec = layout4.pack_sink(k, vc, vs, vz)
    assert rec.shape == (4, 512) and not rec[:, 336:].any()
    for a, b in zip(layout4.unpack_sink(rec), (k, vc, vs, vz)):
        assert np.array_equal(a, b)


# ------------------------------------------------------------------ sink cache
def _kv(rng, S, N):
    k = rng.standard_normal((S, N, 128)).astype(np.float32)
    k[..., [3, 40, 77, 120]] *= 20
    return k.astype(np.float16), rng.standard_normal((S, N, 128)).astype(np.float16)


@pytest.mark.parametrize("N", [1, 2, 129, 130, 300])
def test_sink_prefill_equals_token_by_token(N):
    rng = np.random.default_rng(N)
    k, v = _kv(rng, 2, N)
    a = oc.SliceCache(2, bits=4, sink=True)
    for i in range(N):
        a.append_token(k[:, i], v[:, i])
    b = oc.SliceCache(2, bits=4, sink=True)
    oc.append_block(b, k[:, :N // 3], v[:, :N // 3])
    oc.append_block(b, k[:, N // 3:], v[:, N // 3:])
    assert a.n_sink == b.n_sink == 1
    assert (a.n_quant, a.n_resid) == (b.n_quant, b.n_resid)
    assert a.n_quant == oc.flushed_tokens(0, N - 1)
    for x, y in zip(a.quantized(), b.quantized()):
        assert np.array_equal(x, y)
    assert np.array_equal(a.k_res, b.k_res) and np.array_equal(a.k_sink, k[:, 0])
    for x, y in zip(a.v_sink, b.v_sink):
        assert np.array_equal(x, y)
    # the sink's value is the per-token quantization of token 0's value; key groups start at token 1
    vq, vs, vz = quant.quantize_values_per_token(v[:, :1], 32, 4)
    assert np.array_equal(a.v_sink[0], vq[:, 0]) and np.array_equal(a.v_sink[1], vs[:, 0])
    if a.n_quant:
        kq, ks, kz = quant.quantize_keys_per_channel(k[:, 1:33], 32, 4)
        assert np.array_equal(a.quantized()[0][:, :32], kq) and np.array_equal(a.quantized()[1][:, :1], ks)


def test_decoded_range_positions_with_sink():
    rng = np.random.default_rng(6)
    k, v = _kv(rng, 1, 200)
    c = oc.SliceCache(1, bits=4, sink=True)
    oc.append_block(c, k, v)
    assert (c.n_sink, c.n_quant, c.n_resid) == (1, 128, 71)
    K, V = oa.decoded_range(c, 0, 200)
    assert np.array_equal(K[0, 0], k[0, 0].astype(np.float64))                   # the sink key is exact
    assert np.array_equal(K[0, 129:], k[0, 129:].astype(np.float64))             # the window is exact
    s = c.quantized()[1][0, 0]                                                    # key scales of tokens 1..32
    assert np.all(np.abs(K[0, 1:33] - k[0, 1:33]) <= s / 2 + 1e-3 * s + 1e-7)
    K2, V2 = oa.decoded_range(c, 100, 150)                                        # any sub-range agrees
    assert np.array_equal(K2, K[:, 100:150]) and np.array_equal(V2, V[:, 100:150])


# ------------------------------------------------------------------ attention with RoPE and a sink
def _brute_force(c, q, base, sigma):
    """Per-token loop: decode every key and value on its own, rotate the key pair by pair with an explicit 2x2
    matrix, plain softmax in float64."""
    S, N, D = c.slices, c.n_tokens, c.head_dim
    out = np.zeros((S, D))
    kq, ks, kz, vq, vs, vz = c.quantized()
    for s in range(S):
        keys, vals = [], []
        for t in range(N):
            if c.n_sink and t == 0:
                kt = c.k_sink[s].astype(np.float64)
                vt = np.array([c.v_sink[0][s, ch] * float(c.v_sink[1][s, ch // 32]) + float(c.v_sink[2][s, ch // 32])
                               for ch in range(D)])
            elif t - c.n_sink < c.n_quant:
                u = t - c.n_sink
                kt = np.array([kq[s, u, ch] * float(ks[s, u // 32, ch]) + float(kz[s, u // 32, ch]) for ch in range(D)])
                vt = np.array([vq[s, u, ch] * float(vs[s, u, ch // 32]) + float(vz[s, u, ch // 32]) for ch in range(D)])
            else:
                u = t - c.n_sink - c.n_quant
                kt, vt = c.k_res[s, u].astype(np.float64), c.v_res[s, u].astype(np.float64)
            kr = np.empty(D)
            for i in range(D // 2):
                a = t * base ** (-2.0 * i / D)
                R = np.array([[np.cos(a), -np.sin(a)], [np.sin(a), np.cos(a)]])
                kr[2 * i:2 * i + 2] = R @ kt[2 * i:2 * i + 2]
            keys.append(kr); vals.append(vt)
        sc = np.array([sigma * float(q[s].astype(np.float64) @ kk) for kk in keys])
        p = np.exp(sc - sc.max())
        out[s] = (p[:, None] * np.array(vals)).sum(0) / p.sum()
    return out


@pytest.mark.parametrize("N", [1, 40, 161])
def test_rope_sink_attention_equals_brute_force(N):
    rng = np.random.default_rng(10 + N)
    k, v = _kv(rng, 2, N)
    c = oc.SliceCache(2, bits=4, sink=True)
    oc.append_block(c, k, v)
    q = rng.standard_normal((2, 1, 128)).astype(np.float16)
    got = oa.decode_attention(c, q, 2, 1, rope_base=10000.0)[:, 0]
    want = _brute_force(c, q[:, 0], 10000.0, 1 / np.sqrt(128))
    assert np.allclose(got, want, rtol=1e-10, atol=1e-12)


def test_zero_query_ignores_rotation():
    # every score is 0 whatever the rotation: the output is the mean of the decoded values, sink included
    rng = np.random.default_rng(20)
    k, v = _kv(rng, 1, 300)
    c = oc.SliceCache(1, bits=4, sink=True)
    oc.append_block(c, k, v)
    q = np.zeros((1, 1, 128), np.float16)
    _, V = oa.decoded_range(c, 0, 300)
    assert np.allclose(oa.decode_attention(c, q, 1, 1, rope_base=10000.0)[0, 0], V[0].mean(0), rtol=1e-12)


def test_rope_scores_depend_on_relative_position():
    # a query rotated by d against keys at positions t equals the unrotated query against keys at t - d
    rng = np.random.default_rng(21)
    N, d = 64, 10
    kf = rng.standard_normal((1, N + d, 128)).astype(np.float16)
    vf = rng.standard_normal((1, N + d, 128)).astype(np.float16)
    q = rng.standard_normal((1, 1, 128)).astype(np.float16).astype(np.float64)
    big = oc.SliceCache(1, residual_cap=256)
    oc.append_block(big, kf, vf)            # all in the window (exact): keys at positions 0..N+d-1
    small = oc.SliceCache(1, residual_cap=256)
    oc.append_block(small, kf[:, d:], vf[:, d:])   # the same keys at positions 0..N-1
    K, V = oa.decoded_range(big, d, N + d)
    lhs = rope.rotate(K[0], np.arange(d, N + d)) @ rope.rotate(q[0, 0], d)
    K2, _ = oa.decoded_range(small, 0, N)
    rhs = rope.rotate(K2[0], np.arange(N)) @ q[0, 0]
    assert np.allclose(lhs, rhs, rtol=1e-10)
