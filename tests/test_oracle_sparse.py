"""Pins of the per-vector dense-and-sparse oracle (synthetic.wiki "KV cache quantization", section "What they
report", KVQuant's list of methods: outliers isolated separately for each vector so that they do not skew the
quantization ranges).

Each pin checks the oracle against something other than its own code: the dense part against the plain group
quantizer called on the 31 remaining elements (np.delete, a different path from the oracle's slot filling),
explicit small groups with known outliers, the bound that removing the largest-magnitude element cannot widen the
range, record round trips, prefill against token-by-token appends, and attention against a per-token loop that
decodes every key and value from the packed records.
"""
import numpy as np
import pytest

from oracle import attention as oa
from oracle import cache as oc
from oracle import layout4
from oracle import quant
from oracle import sparse as dsq


def _groups(rng, n, outlier=20.0):
    x = rng.standard_normal((n, 32)).astype(np.float32)
    pos = rng.integers(0, 32, n)
    x[np.arange(n), pos] *= outlier
    return x.astype(np.float16)


def test_outlier_is_the_largest_magnitude_first_on_ties():
    g = np.zeros((4, 32), np.float16)
    g[0, 5] = -7.0                                   # a negative extreme
    g[1, 3], g[1, 9] = 4.0, -4.0                     # tie in magnitude: the lower index
    g[2, :] = 1.5                                    # constant group: index 0
    g[3, 31] = 65504.0
    codes, s, z, out, idx = dsq.quantize_groups_sparse(g, 4)
    assert idx.tolist() == [5, 3, 0, 31]
    assert out.astype(np.float64).tolist() == [-7.0, 4.0, 1.5, 65504.0]
    assert np.all(codes[np.arange(4), idx] == 0)
    # group 2: the other 31 are constant -> scale 0, zero 1.5; group 1: dense range [-4, 0]
    assert s[2] == 0 and z[2] == np.float16(1.5)
    assert z[1] == np.float16(-4.0) and s[1] == np.float16(4.0 / 15)


@pytest.mark.parametrize("bits", [2, 4])
def test_dense_part_equals_plain_quantizer_on_the_other_31(bits):
    rng = np.random.default_rng(bits)
    g = _groups(rng, 3000)
    g[:100] = np.round(g[:100])                      # repeated values, ties in magnitude
    codes, s, z, out, idx = dsq.quantize_groups_sparse(g, bits)
    dense = np.stack([np.delete(g[i], idx[i]) for i in range(len(g))])
    c31, s31, z31 = quant.quantize_groups(dense, bits)
    assert np.array_equal(s.view(np.uint16), s31.view(np.uint16))
    assert np.array_equal(z.view(np.uint16), z31.view(np.uint16))
    got = np.stack([np.delete(codes[i], idx[i]) for i in range(len(g))])
    assert np.array_equal(got, c31)
    assert np.array_equal(np.abs(out.astype(np.float64)), np.abs(g.astype(np.float64)).max(1))


@pytest.mark.parametrize("bits", [2, 4])
def test_decode_restores_the_outlier_and_bounds_the_rest(bits):
    rng = np.random.default_rng(10 + bits)
    g = _groups(rng, 2000)
    codes, s, z, out, idx = dsq.quantize_groups_sparse(g, bits)
    x = dsq.dequantize_groups_sparse(codes, s, z, out, idx)
    xf = g.astype(np.float64)
    assert np.array_equal(x[np.arange(len(g)), idx], xf[np.arange(len(g)), idx])
    err = np.abs(x - xf)
    bound = s.astype(np.float64)[:, None] * (0.5 + 2.0 ** -21)
    assert np.all(err <= bound)


@pytest.mark.parametrize("bits", [2, 4])
def test_dense_scale_never_exceeds_the_plain_scale(bits):
    """The largest-magnitude element is the group maximum or minimum: removing it cannot widen the range."""
    rng = np.random.default_rng(20 + bits)
    g = np.concatenate([_groups(rng, 2000), rng.standard_normal((500, 32)).astype(np.float16)])
    _, s, _, _, _ = dsq.quantize_groups_sparse(g, bits)
    _, sp, _ = quant.quantize_groups(g, bits)
    assert np.all(s.astype(np.float64) <= sp.astype(np.float64))
    # on groups with one x20 element the dense scale is several times smaller
    assert np.median(sp[:2000].astype(np.float64) / np.maximum(s[:2000].astype(np.float64), 1e-30)) > 3


def test_key_and_value_axes():
    """Keys: the outlier of (tile, channel) is the token of largest |k| in that channel's 32 tokens; values: the
    channel of largest |v| in each 32-channel group of a token (brute force over the tensors)."""
    rng = np.random.default_rng(3)
    k = rng.standard_normal((2, 64, 128)).astype(np.float16)
    v = rng.standard_normal((2, 64, 128)).astype(np.float16)
    kq, ks, kz, ko, ki = dsq.quantize_keys_per_channel_sparse(k)
    vq, vs, vz, vo, vi = dsq.quantize_values_per_token_sparse(v)
    for b in range(2):
        for j in range(2):
            for c in range(0, 128, 7):
                col = k[b, 32 * j:32 * j + 32, c].astype(np.float64)
                assert ki[b, j, c] == np.argmax(np.abs(col)) and ko[b, j, c] == k[b, 32 * j + ki[b, j, c], c]
        for t in range(0, 64, 5):
            for gg in range(4):
                row = v[b, t, 32 * gg:32 * gg + 32].astype(np.float64)
                assert vi[b, t, gg] == np.argmax(np.abs(row)) and vo[b, t, gg] == v[b, t, 32 * gg + vi[b, t, gg]]
    kd = dsq.dequantize_keys_sparse(kq, ks, kz, ko, ki)
    vd = dsq.dequantize_values_sparse(vq, vs, vz, vo, vi)
    for b in range(2):
        for j in range(2):
            for c in range(128):
                assert kd[b, 32 * j + ki[b, j, c], c] == k[b, 32 * j + ki[b, j, c], c]
    assert np.all(np.abs(kd - k) <= np.repeat(ks.astype(np.float64), 32, axis=1) * 0.5000005)
    assert np.all(np.abs(vd - v) <= np.repeat(vs.astype(np.float64), 32, axis=2) * 0.5000005)


def test_sparse_record_and_sink_round_trip():
    rng = np.random.default_rng(4)
    kq = rng.integers(0, 16, (3, 32, 128)).astype(np.uint8)
    vq = rng.integers(0, 16, (3, 32, 128)).astype(np.uint8)
    ks, kz = (rng.standard_normal((3, 128)).astype(np.float16) for _ in range(2))
    vs, vz = (rng.standard_normal((3, 32, 4)).astype(np.float16) for _ in range(2))
    ko = rng.standard_normal((3, 128)).astype(np.float16)
    ki = rng.integers(0, 32, (3, 128)).astype(np.uint8)
    vo = rng.standard_normal((3, 32, 4)).astype(np.float16)
    vi = rng.integers(0, 32, (3, 32, 4)).astype(np.uint8)
    rec = layout4.pack_tiles_sparse(kq, ks, kz, vq, vs, vz, ko, ki, vo, vi)
    assert rec.shape == (3, layout4.RECORD_BYTES_SPARSE)
    assert np.array_equal(rec[:, :layout4.RECORD_BYTES], layout4.pack_tiles(kq, ks, kz, vq, vs, vz))
    back = layout4.unpack_tiles_sparse(rec)
    for a, b in zip(back, (kq, ks, kz, vq, vs, vz, ko, ki, vo, vi)):
        assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))
    # value outlier of token 5, group 2 sits at index 32*2 + 5 of the section
    assert rec[1, layout4.V_IDX_OFF + 64 + 5] == vi[1, 5, 2]
    sink = layout4.pack_sink(ks[:, :128], kq[:, 0], vs[:, 0], vz[:, 0], vo[:, 0], vi[:, 0])
    assert np.array_equal(sink[:, 336:344].copy().view(np.float16), vo[:, 0])
    assert np.array_equal(sink[:, 344:348], vi[:, 0]) and not sink[:, 348:].any()


def test_sparse_prefill_equals_token_by_token():
    rng = np.random.default_rng(5)
    S, N = 3, 450
    k = rng.standard_normal((S, N, 128)).astype(np.float32)
    k[:, :, [3, 70]] *= 20
    k = k.astype(np.float16)
    v = rng.standard_normal((S, N, 128)).astype(np.float16)
    a = oc.SliceCache(S, bits=4, sink=True, sparse=True)
    oc.append_block(a, k, v)
    b = oc.SliceCache(S, bits=4, sink=True, sparse=True)
    for t in range(N):
        b.append_token(k[:, t], v[:, t])
    assert (a.n_sink, a.n_quant, a.n_resid) == (b.n_sink, b.n_quant, b.n_resid) == (1, 384, 65)
    for x, y in zip(a.quantized() + a.outliers(), b.quantized() + b.outliers()):
        assert np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8))
    for x, y in zip(a.v_sink + a.v_sink_out, b.v_sink + b.v_sink_out):
        assert np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8))


@pytest.mark.parametrize("N,rope_base", [(300, 10000.0), (161, None)])
def test_sparse_attention_equals_a_loop_over_packed_records(N, rope_base):
    """Attention of the oracle over a sparse, sink, (pre-RoPE) cache equals a per-token loop that decodes every key
    and value from the packed 5888-byte records and the sink record, rotates each key with an explicit 2x2 matrix
    per channel pair, and runs a float64 softmax."""
    rng = np.random.default_rng(N)
    S = 2
    k = rng.standard_normal((S, N, 128)).astype(np.float32)
    k[:, :, [9, 100]] *= 20
    k = k.astype(np.float16)
    v = rng.standard_normal((S, N, 128)).astype(np.float16)
    q = rng.standard_normal((1, S, 128)).astype(np.float16)
    c = oc.SliceCache(S, bits=4, sink=True, sparse=True)
    oc.append_block(c, k, v)
    want = oa.decode_attention(c, q.reshape(1, S, 128), 1, S, rope_base=rope_base)[0]

    kq, ks, kz, vq, vs, vz = c.quantized()
    ko, ki, vo, vi = c.outliers()
    nt = c.n_quant // 32
    rec = layout4.pack_tiles_sparse(kq.reshape(S, nt, 32, 128), ks, kz, vq.reshape(S, nt, 32, 128),
                                    vs.reshape(S, nt, 32, 4), vz.reshape(S, nt, 32, 4), ko, ki,
                                    vo.reshape(S, nt, 32, 4), vi.reshape(S, nt, 32, 4))
    sink = layout4.pack_sink(c.k_sink, *c.v_sink, *c.v_sink_out)
    th = 10000.0 ** (-np.arange(64) / 64.0) if rope_base else np.zeros(64)
    for s in range(S):
        keys, vals = [], []
        sk, svc, svs, svz, svo, svi = layout4.unpack_sink(sink[s])[0], *layout4.unpack_sink(sink[s])[1:], \
            sink[s, 336:344].copy().view(np.float16), sink[s, 344:348]
        val = np.array([svc[ch] * float(svs[ch // 32]) + float(svz[ch // 32]) for ch in range(128)])
        for gg in range(4):
            val[32 * gg + svi[gg]] = float(svo[gg])
        keys.append(sk.astype(np.float64))
        vals.append(val)
        for j in range(nt):
            f = layout4.unpack_tiles_sparse(rec[s, j])
            tkq, tks, tkz, tvq, tvs, tvz, tko, tki, tvo, tvi = f
            for t in range(32):
                key = np.array([tkq[t, ch] * float(tks[ch]) + float(tkz[ch]) for ch in range(128)])
                for ch in range(128):
                    if tki[ch] == t:
                        key[ch] = float(tko[ch])
                val = np.array([tvq[t, ch] * float(tvs[t, ch // 32]) + float(tvz[t, ch // 32]) for ch in range(128)])
                for gg in range(4):
                    val[32 * gg + tvi[t, gg]] = float(tvo[t, gg])
                keys.append(key)
                vals.append(val)
        for r in range(c.n_resid):
            keys.append(c.k_res[s, r].astype(np.float64))
            vals.append(c.v_res[s, r].astype(np.float64))
        scores = []
        for m, key in enumerate(keys):
            rk = key.copy()
            for i in range(64):
                a = m * th[i]
                rot = np.array([[np.cos(a), -np.sin(a)], [np.sin(a), np.cos(a)]])
                rk[2 * i:2 * i + 2] = rot @ key[2 * i:2 * i + 2]
            scores.append(float(q[0, s].astype(np.float64) @ rk) / np.sqrt(128))
        scores = np.array(scores)
        p = np.exp(scores - scores.max())
        ref = (p[:, None] * np.array(vals)).sum(0) / p.sum()
        assert np.allclose(want[s], ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------------------------- 2-bit records
from oracle import layout  # noqa: E402


def test_sparse_record_2bit_round_trip():
    """3840-byte 2-bit records: the dense 3072 bytes are pack_tiles' own, the outlier section sits at the stated
    offsets in [group][token] order for values, and unpacking returns every field."""
    rng = np.random.default_rng(41)
    kq = rng.integers(0, 4, (3, 32, 128)).astype(np.uint8)
    vq = rng.integers(0, 4, (3, 32, 128)).astype(np.uint8)
    ks, kz = (rng.standard_normal((3, 128)).astype(np.float16) for _ in range(2))
    vs, vz = (rng.standard_normal((3, 32, 4)).astype(np.float16) for _ in range(2))
    ko = rng.standard_normal((3, 128)).astype(np.float16)
    ki = rng.integers(0, 32, (3, 128)).astype(np.uint8)
    vo = rng.standard_normal((3, 32, 4)).astype(np.float16)
    vi = rng.integers(0, 32, (3, 32, 4)).astype(np.uint8)
    rec = layout.pack_tiles_sparse(kq, ks, kz, vq, vs, vz, ko, ki, vo, vi)
    assert rec.shape == (3, layout.RECORD_BYTES_SPARSE) and layout.RECORD_BYTES_SPARSE % 256 == 0
    assert np.array_equal(rec[:, :layout.RECORD_BYTES], layout.pack_tiles(kq, ks, kz, vq, vs, vz))
    back = layout.unpack_tiles_sparse(rec)
    for a, b in zip(back, (kq, ks, kz, vq, vs, vz, ko, ki, vo, vi)):
        assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))
    # key outlier of channel 77: value at 3072 + 2*77, token at 3328 + 77; value outlier of token 5, group 2 at
    # entry 32*2 + 5 of each value array
    assert rec[2, 3072 + 154:3072 + 156].copy().view(np.float16)[0] == ko[2, 77]
    assert rec[2, 3328 + 77] == ki[2, 77]
    assert rec[1, 3456 + 2 * 69:3456 + 2 * 70].copy().view(np.float16)[0] == vo[1, 5, 2]
    assert rec[1, 3712 + 69] == vi[1, 5, 2]


def test_sparse_2bit_prefill_equals_token_by_token():
    rng = np.random.default_rng(42)
    S, N = 3, 417
    k = rng.standard_normal((S, N, 128)).astype(np.float32)
    k[:, :, [3, 70]] *= 20
    k = k.astype(np.float16)
    v = rng.standard_normal((S, N, 128)).astype(np.float16)
    a = oc.SliceCache(S, bits=2, sparse=True)
    oc.append_block(a, k, v)
    b = oc.SliceCache(S, bits=2, sparse=True)
    for t in range(N):
        b.append_token(k[:, t], v[:, t])
    assert (a.n_quant, a.n_resid) == (b.n_quant, b.n_resid) == (384, 33)
    for x, y in zip(a.quantized() + a.outliers(), b.quantized() + b.outliers()):
        assert np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8))
    kq = a.quantized()[0]
    assert kq.max() <= 3


def test_sparse_2bit_attention_equals_a_loop_over_packed_records():
    """Attention of the oracle over a 2-bit dense-and-sparse cache equals a per-token loop that decodes every key and
    value element from the packed 3840-byte records (q * s + z, the group's outlier put back at its index) and the
    window, then runs a float64 softmax."""
    rng = np.random.default_rng(43)
    S, N = 2, 230
    k = rng.standard_normal((S, N, 128)).astype(np.float32)
    k[:, :, [9, 100]] *= 20
    k[:, 17] *= 8                      # a spike token: the outlier of most of its channels' groups
    k = k.astype(np.float16)
    v = rng.standard_normal((S, N, 128)).astype(np.float32)
    v[:, :, 45] *= 30
    v = v.astype(np.float16)
    q = rng.standard_normal((1, S, 128)).astype(np.float16)
    c = oc.SliceCache(S, bits=2, sparse=True)
    oc.append_block(c, k, v)
    want = oa.decode_attention(c, q, 1, S)[0]

    kq, ks, kz, vq, vs, vz = c.quantized()
    ko, ki, vo, vi = c.outliers()
    nt = c.n_quant // 32
    rec = layout.pack_tiles_sparse(kq.reshape(S, nt, 32, 128), ks, kz, vq.reshape(S, nt, 32, 128),
                                   vs.reshape(S, nt, 32, 4), vz.reshape(S, nt, 32, 4), ko, ki,
                                   vo.reshape(S, nt, 32, 4), vi.reshape(S, nt, 32, 4))
    assert rec.shape == (S, nt, 3840)
    for s in range(S):
        keys, vals = [], []
        for j in range(nt):
            tkq, tks, tkz, tvq, tvs, tvz, tko, tki, tvo, tvi = layout.unpack_tiles_sparse(rec[s, j])
            for t in range(32):
                key = [float(tkq[t, ch]) * float(tks[ch]) + float(tkz[ch]) for ch in range(128)]
                for ch in range(128):
                    if tki[ch] == t:
                        key[ch] = float(tko[ch])
                val = [float(tvq[t, ch]) * float(tvs[t, ch // 32]) + float(tvz[t, ch // 32]) for ch in range(128)]
                for gg in range(4):
                    val[32 * gg + int(tvi[t, gg])] = float(tvo[t, gg])
                keys.append(key)
                vals.append(val)
        for r in range(c.n_resid):
            keys.append(c.k_res[s, r].astype(np.float64))
            vals.append(c.v_res[s, r].astype(np.float64))
        scores = np.array(keys) @ q[0, s].astype(np.float64) / np.sqrt(128)
        p = np.exp(scores - scores.max())
        ref = (p[:, None] * np.array(vals)).sum(0) / p.sum()
        assert np.allclose(want[s], ref, rtol=0, atol=1e-12)
    # the outliers matter: without them the spike token's and channel 45's contributions change the output
    dense_only = oc.SliceCache(S, bits=2)
    oc.append_block(dense_only, k, v)
    assert np.abs(oa.decode_attention(dense_only, q, 1, S)[0] - want).max() > 1e-2
