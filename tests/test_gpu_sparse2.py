"""GPU parity of 2-bit dense-and-sparse groups (synthetic.wiki "KV cache quantization", section "What they report":
per-vector dense-and-sparse quantization; KIVI page for the 2-bit grouping and the recent-token window): 3840-byte
records through the C ABI, against the fp64 CPU oracle.

Bars: codes, fp16 scales, zero points, outlier values and their indices, and the window bytes bit-exact; attention
outputs within max-abs 2e-3. The decode cases include a key whose outlier channels alone make its token dominate the
softmax and value outliers that dominate output channels, so a dropped or misplaced correction fails by far more than
the tolerance; they cover one query head per KV head, GQA groups of 2, 4 and 8 (two query-head chunks) and splits
from one to many.
"""
import sys
import zlib

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

from oracle import attention as oa  # noqa: E402
from oracle import cache as oc  # noqa: E402
from tests import helpers  # noqa: E402

ATOL = 2e-3
REC = 3840


@pytest.fixture(scope="module")
def kvq():
    import decode_attention_quant_amd as m
    return m


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _dev(x: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _keys(rng, shape):
    """N(0, 1) with four channels x20 and about 1% isolated spikes x30."""
    x = rng.standard_normal(shape).astype(np.float32)
    x[..., [5, 33, 90, 127]] *= 20
    x[rng.random(shape) < 0.01] *= 30
    return x.astype(np.float16)


def _values(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    x[rng.random(shape) < 0.01] *= 25
    return x.astype(np.float16)


def _shape(kvq, B, Hkv, Hq, max_tokens, R=128):
    return kvq.Shape(B, Hkv, Hq, max_tokens=max_tokens, residual_cap=R, bits=2, flags=kvq.FLAG_SPARSE)


def _oracle(k, v, R=128):
    S = k.shape[0] * k.shape[1]
    ref = oc.SliceCache(S, residual_cap=R, bits=2, sparse=True)
    oc.append_block(ref, k.reshape(S, -1, 128), v.reshape(S, -1, 128))
    return ref


def _check_state(cache, ref, B, H, what):
    assert (cache.n_quant, cache.n_resid) == (ref.n_quant, ref.n_resid), what
    nt = ref.n_quant // 32
    if nt:
        got = helpers.records_from_device(cache.tiles, nt)
        want = helpers.oracle_records(ref)
        assert got.shape[-1] == REC
        assert np.array_equal(got, want), f"{what}: " + helpers.first_mismatch(got, want)
    nr = ref.n_resid
    kr = cache.k_res[:, :, :nr].reshape(B * H, nr, 128).cpu().numpy()
    vr = cache.v_res[:, :, :nr].reshape(B * H, nr, 128).cpu().numpy()
    assert np.array_equal(kr.view(np.uint16), ref.k_res.view(np.uint16)), what
    assert np.array_equal(vr.view(np.uint16), ref.v_res.view(np.uint16)), what


def _family(rng, kind, shape):
    if kind == "spikes":
        return _keys(rng, shape)
    if kind == "wide":
        return rng.uniform(-65504, 65504, shape).astype(np.float16)
    if kind == "tiny":
        return (rng.integers(-30, 30, shape) * 2.0 ** -24).astype(np.float16)
    if kind == "equal_magnitudes":   # many |x| ties: the first index of largest magnitude is the outlier
        x = rng.choice(np.array([-2.0, -1.0, -0.5, 0.0, -0.0, 0.5, 1.0, 2.0]), size=shape)
        x[..., :32, :] = 1.5                # whole key groups equal (outlier token 0, dense range 0)
        x[..., 40, :] = -3.0                # one token: value groups with a unique largest element
        x[..., 41, 0:64] = np.tile([3.0, -3.0], 32)
        return x.astype(np.float16)
    if kind == "const_and_zero":
        x = rng.standard_normal(shape)
        x[..., :32, :] = 1.25
        x[..., 64:96, 0:32] = 0.0
        x[..., 70, 0:16] = -0.0
        x[..., :, 100] = 65504.0
        x[..., 3, 100] = -65504.0
        return x.astype(np.float16)
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["spikes", "wide", "tiny", "equal_magnitudes", "const_and_zero", "ties"])
def test_quantize_sparse2_entry_points_bit_exact(kvq, kind):
    say(f"[quant-sparse2] kind={kind}")
    rng = np.random.default_rng(zlib.crc32(kind.encode()) + 240)
    B, H, T, tile0 = 2, 3, 256, 2
    if kind == "ties":   # the 31 dense elements of every group on or beside half levels, plus one outlier
        k = helpers.tie_groups_sparse(rng, B * H * (T // 32) * 128, 3).reshape(B, H, T // 32, 128, 32)
        k = np.ascontiguousarray(k.transpose(0, 1, 2, 4, 3)).reshape(B, H, T, 128)
        v = helpers.tie_groups_sparse(rng, B * H * T * 4, 3).reshape(B, H, T, 128)
    else:
        k = _family(rng, kind, (B, H, T, 128))
        v = _family(rng, kind, (B, H, T, 128))
    shape = _shape(kvq, B, H, H, T + 32 * tile0 + 64)
    assert shape.record_bytes == REC
    tiles = torch.zeros((B, H, shape.max_tokens // 32, REC), dtype=torch.uint8, device="cuda")
    kvq.kv_quant_keys_per_channel(shape, _dev(k), tile0, tiles)
    torch.cuda.synchronize()
    got = tiles.cpu().numpy().reshape(B * H, -1, REC)
    assert not got[:, :, 1024:2048].any() and not got[:, :, 2560:3072].any() and not got[:, :, 3456:].any(), \
        "key call wrote value fields"
    kvq.kv_quant_values_per_token(shape, _dev(v), tile0, tiles)
    torch.cuda.synchronize()
    got = tiles.cpu().numpy().reshape(B * H, -1, REC)
    ref = oc.SliceCache(B * H, bits=2, sparse=True)
    ref._push_quantized(k.reshape(B * H, T, 128), v.reshape(B * H, T, 128))
    want = helpers.oracle_records(ref)
    assert not got[:, :tile0].any() and not got[:, tile0 + T // 32:].any(), "wrote outside the tile range"
    sel = got[:, tile0:tile0 + T // 32]
    assert np.array_equal(sel, want), helpers.first_mismatch(sel, want)
    # keys and values again through non-contiguous views ([B, T, H, D] storage): the same records
    tiles2 = torch.zeros_like(tiles)
    k_store = _dev(np.ascontiguousarray(k.transpose(0, 2, 1, 3)))
    v_store = _dev(np.ascontiguousarray(v.transpose(0, 2, 1, 3)))
    kvq.kv_quant_keys_per_channel(shape, k_store.permute(0, 2, 1, 3), tile0, tiles2)
    kvq.kv_quant_values_per_token(shape, v_store.permute(0, 2, 1, 3), tile0, tiles2)
    torch.cuda.synchronize()
    got2 = tiles2.cpu().numpy().reshape(B * H, -1, REC)
    assert np.array_equal(got2, got), helpers.first_mismatch(got2[:, tile0:tile0 + T // 32], want)


def test_append_stream_sparse2(kvq):
    """Prefill, single-token appends across two flushes, then a block append: 3840-byte tiles and window equal the
    oracle's token-by-token state, bit for bit."""
    rng = np.random.default_rng(2141)
    B, H, R = 2, 3, 128
    total = 300 + 200 + 77
    k = _keys(rng, (B, H, total, 128))
    v = _values(rng, (B, H, total, 128))
    cache = kvq.KVCache(_shape(kvq, B, H, H, 1024, R))
    assert cache.tiles.shape[-1] == REC
    ref = oc.SliceCache(B * H, residual_cap=R, bits=2, sparse=True)
    kd, vd = _dev(k), _dev(v)
    kvq.kv_append_and_flush(cache, kd[:, :, :300], vd[:, :, :300])
    ref.append(k[:, :, :300].reshape(B * H, 300, 128), v[:, :, :300].reshape(B * H, 300, 128))
    torch.cuda.synchronize()
    _check_state(cache, ref, B, H, "after prefill")
    for t in range(300, 500):
        kvq.kv_append_and_flush(cache, kd[:, :, t:t + 1], vd[:, :, t:t + 1])
        flushed = ref.n_resid == R
        ref.append_token(k[:, :, t].reshape(B * H, 128), v[:, :, t].reshape(B * H, 128))
        if flushed or t == 499:
            torch.cuda.synchronize()
            say(f"[stream-sparse2] token {t} flushed={flushed}")
            _check_state(cache, ref, B, H, f"token {t}")
    kvq.kv_append_and_flush(cache, kd[:, :, 500:], vd[:, :, 500:])
    ref.append(k[:, :, 500:].reshape(B * H, 77, 128), v[:, :, 500:].reshape(B * H, 77, 128))
    torch.cuda.synchronize()
    _check_state(cache, ref, B, H, "after block append")


CASES = [
    # (B, Hq, Hkv, N, note)
    (1, 1, 1, 33, "one full window tile"),
    (1, 1, 1, 1024, "896 quantized + 128 window"),
    (2, 8, 2, 1000, "GQA G=4"),
    (2, 8, 4, 2177, "GQA G=2"),
    (2, 16, 2, 1500, "GQA G=8: two query-head chunks"),
    (1, 4, 4, 1300, "one query head per KV head"),
    (3, 4, 4, 4226, "many tiles, window of 2"),
    (4, 32, 8, 10000, "GQA G=4, splits of ~30 tiles"),
]


@pytest.mark.parametrize("B,Hq,Hkv,N,note", CASES)
def test_decode_sparse2_matches_oracle(kvq, B, Hq, Hkv, N, note):
    say(f"[decode-sparse2] B={B} Hq={Hq} Hkv={Hkv} N={N} ({note})")
    rng = np.random.default_rng(N * 17 + Hq)
    k = _keys(rng, (B, Hkv, N, 128))
    v = _values(rng, (B, Hkv, N, 128))
    q = rng.standard_normal((B, Hq, 128)).astype(np.float16)
    cache = kvq.KVCache(_shape(kvq, B, Hkv, Hq, ((N + 31) // 32) * 32 + 32))
    kvq.kv_append_and_flush(cache, _dev(k), _dev(v))
    out = kvq.kv_decode_attention(cache, _dev(q))
    torch.cuda.synchronize()
    ref = _oracle(k, v)
    assert (cache.n_quant, cache.n_resid) == (ref.n_quant, ref.n_resid)
    want = oa.decode_attention(ref, q, B, Hkv)
    got = out.cpu().numpy().astype(np.float64)
    err = np.abs(got - want)
    say(f"    splits={kvq.kv_decode_attention_splits(cache)} max_abs={err.max():.3e} "
        f"p99.9={np.quantile(err, 0.999):.3e}")
    assert np.all(np.isfinite(got))
    assert err.max() <= ATOL


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (4, 4)])
def test_decode_sparse2_dominant_outliers(kvq, Hq, Hkv):
    """Outliers that decide the result: at quantized position 333 (token 13 of its tile) channels 6, 7 hold the
    direction of the first query head of each group in that pair (length 1000), each the outlier of its key group,
    so that token dominates the softmax through its outliers alone; its value has outliers of 300 and -200 in
    channels 77 and 2 (the outliers of their value groups)."""
    rng = np.random.default_rng(2333 + Hq)
    B, N = 2, 777
    G = Hq // Hkv
    k = _keys(rng, (B, Hkv, N, 128))
    v = _values(rng, (B, Hkv, N, 128))
    q = rng.standard_normal((B, Hq, 128)).astype(np.float16)
    pos = 333
    pair = np.zeros((B, Hkv, 128))
    qp = q[:, ::G, 6:8].astype(np.float64)
    pair[..., 6:8] = qp / np.linalg.norm(qp, axis=-1, keepdims=True) * 1000
    k[:, :, pos] = pair.astype(np.float16)
    v[:, :, pos, 77] = 300.0
    v[:, :, pos, 2] = -200.0
    cache = kvq.KVCache(_shape(kvq, B, Hkv, Hq, 1024))
    kvq.kv_append_and_flush(cache, _dev(k), _dev(v))
    assert cache.n_quant > 400
    out = kvq.kv_decode_attention(cache, _dev(q))
    torch.cuda.synchronize()
    ref = _oracle(k, v)
    ko, ki, vo, vi = ref.outliers()
    big = 6 + int(abs(float(k[0, 0, pos, 7])) > abs(float(k[0, 0, pos, 6])))
    assert ki[0, pos // 32, big] == pos % 32 and vi[0, pos, 2] == 77 - 64, "the planted elements are the outliers"
    want = oa.decode_attention(ref, q, B, Hkv)
    got = out.cpu().numpy().astype(np.float64)
    err = np.abs(got - want)
    say(f"    max_abs={err.max():.3e}; oracle channel 77 of head 0: {want[0, 0, 77]:.2f}")
    assert np.abs(want[:, ::G, 77]).max() > 30, "the outlier token should dominate"
    assert err.max() <= ATOL


def test_sparse2_changes_the_result(kvq):
    """The same tokens in a dense 2-bit cache and a dense-and-sparse one give different outputs, each matching its
    own oracle: the outliers reach the output (and the dense-and-sparse error is the smaller one)."""
    rng = np.random.default_rng(2777)
    B, Hq, Hkv, N = 2, 8, 2, 900
    k = _keys(rng, (B, Hkv, N, 128))
    v = _values(rng, (B, Hkv, N, 128))
    q = rng.standard_normal((B, Hq, 128)).astype(np.float16)
    outs = {}
    for sparse in (False, True):
        shape = kvq.Shape(B, Hkv, Hq, max_tokens=1024, bits=2, flags=kvq.FLAG_SPARSE if sparse else 0)
        cache = kvq.KVCache(shape)
        kvq.kv_append_and_flush(cache, _dev(k), _dev(v))
        out = kvq.kv_decode_attention(cache, _dev(q))
        torch.cuda.synchronize()
        S = B * Hkv
        ref = oc.SliceCache(S, bits=2, sparse=sparse)
        oc.append_block(ref, k.reshape(S, N, 128), v.reshape(S, N, 128))
        want = oa.decode_attention(ref, q, B, Hkv)
        got = out.cpu().numpy().astype(np.float64)
        assert np.abs(got - want).max() <= ATOL, f"sparse={sparse}"
        outs[sparse] = got
    # attention over the unquantized fp16 tokens, in float64
    G = Hq // Hkv
    kf = k.astype(np.float64).repeat(G, axis=1)
    vf = v.astype(np.float64).repeat(G, axis=1)
    sc = np.einsum("bhd,bhtd->bht", q.astype(np.float64), kf) / np.sqrt(128)
    pr = np.exp(sc - sc.max(-1, keepdims=True))
    exact = np.einsum("bht,bhtd->bhd", pr, vf) / pr.sum(-1)[..., None]
    assert np.abs(outs[True] - outs[False]).max() > 1e-2
    assert np.abs(outs[True] - exact).mean() < np.abs(outs[False] - exact).mean()
