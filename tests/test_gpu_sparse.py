"""GPU parity of dense-and-sparse groups (synthetic.wiki "KV cache quantization", section "What they report":
per-vector dense-and-sparse quantization): the 4-bit
records of 5888 bytes and the sink record with value outliers, through the C ABI, against the fp64 CPU oracle.

Bars: codes, fp16 scales, zero points, outlier values and their indices, the sink record and the window bytes
bit-exact; attention outputs within max-abs 2e-3. The decode cases include an outlier key that dominates its
softmax after the decode-time rotation and value outliers that dominate output channels, so a dropped or misplaced
correction fails by far more than the tolerance.
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
from oracle import rope  # noqa: E402
from tests import helpers  # noqa: E402

ATOL = 2e-3
BASE = 10000.0


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


def _shape(kvq, B, Hkv, Hq, max_tokens, flags, R=128):
    return kvq.Shape(B, Hkv, Hq, max_tokens=max_tokens, residual_cap=R, bits=4, flags=flags | kvq.FLAG_SPARSE,
                     rope_base=BASE if flags & kvq.FLAG_PRE_ROPE else 0.0)


def _oracle(kvq, k, v, flags, R=128):
    S = k.shape[0] * k.shape[1]
    ref = oc.SliceCache(S, residual_cap=R, bits=4, sink=bool(flags & kvq.FLAG_SINK), sparse=True)
    oc.append_block(ref, k.reshape(S, -1, 128), v.reshape(S, -1, 128))
    return ref


def _check_state(cache, ref, B, H, what):
    assert (cache.n_sink, cache.n_quant, cache.n_resid) == (ref.n_sink, ref.n_quant, ref.n_resid), what
    nt = ref.n_quant // 32
    if nt:
        got = helpers.records4_from_device(cache.tiles, nt)
        want = helpers.oracle_records4(ref)
        assert got.shape[-1] == 5888
        assert np.array_equal(got, want), f"{what}: " + helpers.first_mismatch4(got, want)
    if ref.n_sink:
        got = cache.sink.reshape(B * H, 512).cpu().numpy()
        want = helpers.oracle_sink(ref)
        assert np.array_equal(got, want), f"{what}: sink record differs at bytes {np.argwhere(got != want)[:4]}"
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
def test_quantize_sparse_entry_points_bit_exact(kvq, kind):
    say(f"[quant-sparse] kind={kind}")
    rng = np.random.default_rng(zlib.crc32(kind.encode()) + 40)
    B, H, T, tile0 = 2, 3, 256, 2
    if kind == "ties":   # the 31 dense elements of every group on or beside half levels, plus one outlier
        k = helpers.tie_groups_sparse(rng, B * H * (T // 32) * 128, 15).reshape(B, H, T // 32, 128, 32)
        k = np.ascontiguousarray(k.transpose(0, 1, 2, 4, 3)).reshape(B, H, T, 128)
        v = helpers.tie_groups_sparse(rng, B * H * T * 4, 15).reshape(B, H, T, 128)
    else:
        k = _family(rng, kind, (B, H, T, 128))
        v = _family(rng, kind, (B, H, T, 128))
    shape = _shape(kvq, B, H, H, T + 32 * tile0 + 64, 0)
    assert shape.record_bytes == 5888
    tiles = torch.zeros((B, H, shape.max_tokens // 32, 5888), dtype=torch.uint8, device="cuda")
    kvq.kv_quant_keys_per_channel(shape, _dev(k), tile0, tiles)
    torch.cuda.synchronize()
    got = tiles.cpu().numpy().reshape(B * H, -1, 5888)
    assert not got[:, :, 2048:4096].any() and not got[:, :, 4608:5120].any() and not got[:, :, 5504:].any(), \
        "key call wrote value fields"
    kvq.kv_quant_values_per_token(shape, _dev(v), tile0, tiles)
    torch.cuda.synchronize()
    got = tiles.cpu().numpy().reshape(B * H, -1, 5888)
    ref = oc.SliceCache(B * H, bits=4, sparse=True)
    ref._push_quantized(k.reshape(B * H, T, 128), v.reshape(B * H, T, 128))
    want = helpers.oracle_records4(ref)
    assert not got[:, :tile0].any() and not got[:, tile0 + T // 32:].any(), "wrote outside the tile range"
    sel = got[:, tile0:tile0 + T // 32]
    assert np.array_equal(sel, want), helpers.first_mismatch4(sel, want)
    # keys and values again through non-contiguous views ([B, T, H, D] storage): the same records
    tiles2 = torch.zeros_like(tiles)
    k_store = _dev(np.ascontiguousarray(k.transpose(0, 2, 1, 3)))
    v_store = _dev(np.ascontiguousarray(v.transpose(0, 2, 1, 3)))
    kvq.kv_quant_keys_per_channel(shape, k_store.permute(0, 2, 1, 3), tile0, tiles2)
    kvq.kv_quant_values_per_token(shape, v_store.permute(0, 2, 1, 3), tile0, tiles2)
    torch.cuda.synchronize()
    got2 = tiles2.cpu().numpy().reshape(B * H, -1, 5888)
    assert np.array_equal(got2, got), helpers.first_mismatch4(got2[:, tile0:tile0 + T // 32], want)


def test_append_stream_sparse_with_sink(kvq):
    """Prefill (token 0 to the sink), single-token appends across two flushes, then a block append: sink record
    (with its value outliers), 5888-byte tiles and window equal the oracle's token-by-token state, bit for bit."""
    rng = np.random.default_rng(141)
    B, H, R = 2, 3, 128
    total = 300 + 200 + 77
    k = _keys(rng, (B, H, total, 128))
    v = _values(rng, (B, H, total, 128))
    v[:, :, 0, 77] = 300.0          # a sink value outlier
    flags = kvq.FLAG_SINK | kvq.FLAG_PRE_ROPE
    cache = kvq.KVCache(_shape(kvq, B, H, H, 1024, flags, R))
    assert cache.tiles.shape[-1] == 5888
    ref = oc.SliceCache(B * H, residual_cap=R, bits=4, sink=True, sparse=True)
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
            say(f"[stream-sparse] token {t} flushed={flushed}")
            _check_state(cache, ref, B, H, f"token {t}")
    kvq.kv_append_and_flush(cache, kd[:, :, 500:], vd[:, :, 500:])
    ref.append(k[:, :, 500:].reshape(B * H, 77, 128), v[:, :, 500:].reshape(B * H, 77, 128))
    torch.cuda.synchronize()
    _check_state(cache, ref, B, H, "after block append")


S_R = 3   # FLAG_SINK | FLAG_PRE_ROPE
CASES = [
    # (B, Hq, Hkv, N, flags, note); FLAG_SPARSE is added to every case
    (1, 1, 1, 1, S_R, "sink only"),
    (1, 1, 1, 33, S_R, "sink + one full window tile"),
    (1, 1, 1, 1024, S_R, "896 quantized + 127 window"),
    (2, 8, 2, 1000, 2, "pre-RoPE, no sink, GQA G=4"),
    (2, 8, 4, 2177, 1, "sink, no RoPE, GQA G=2"),
    (1, 4, 4, 1300, 0, "sparse only"),
    (3, 4, 4, 4226, S_R, "many tiles, window of 1"),
    (4, 128, 4, 10000, S_R, "splits of ~80 tiles: rotation re-anchored inside a split"),
]


@pytest.mark.parametrize("B,Hq,Hkv,N,flags,note", CASES)
def test_decode_sparse_matches_oracle(kvq, B, Hq, Hkv, N, flags, note):
    say(f"[decode-sparse] B={B} Hq={Hq} Hkv={Hkv} N={N} flags={flags} ({note})")
    rng = np.random.default_rng(N * 13 + Hq + 100 * flags)
    k = _keys(rng, (B, Hkv, N, 128))
    v = _values(rng, (B, Hkv, N, 128))
    q = rng.standard_normal((B, Hq, 128)).astype(np.float16)
    cache = kvq.KVCache(_shape(kvq, B, Hkv, Hq, ((N + 31) // 32) * 32 + 32, flags))
    kvq.kv_append_and_flush(cache, _dev(k), _dev(v))
    out = kvq.kv_decode_attention(cache, _dev(q))
    torch.cuda.synchronize()
    ref = _oracle(kvq, k, v, flags)
    assert (cache.n_sink, cache.n_quant, cache.n_resid) == (ref.n_sink, ref.n_quant, ref.n_resid)
    want = oa.decode_attention(ref, q, B, Hkv, rope_base=BASE if flags & 2 else None)
    got = out.cpu().numpy().astype(np.float64)
    err = np.abs(got - want)
    say(f"    splits={kvq.kv_decode_attention_splits(cache)} max_abs={err.max():.3e} "
        f"p99.9={np.quantile(err, 0.999):.3e}")
    assert np.all(np.isfinite(got))
    assert err.max() <= ATOL


@pytest.mark.parametrize("flags", [S_R, 1])
def test_decode_sparse_dominant_outliers(kvq, flags):
    """Outliers that decide the result: at quantized position 333 (token 13 of its tile, after the sink) channels
    6, 7 hold the direction of the first query head of each group in that pair (length 1000), rotated back by the
    position, each the outlier of its key
    group, so after the decode-time rotation that token dominates the softmax through its outliers alone; its value
    has outliers of 300 and -200 in channels 77 and 2; the sink's value has an outlier of 250 in channel 100."""
    rng = np.random.default_rng(333 + flags)
    B, Hq, Hkv, N = 2, 8, 2, 777
    G = Hq // Hkv
    k = _keys(rng, (B, Hkv, N, 128))
    v = _values(rng, (B, Hkv, N, 128))
    q = rng.standard_normal((B, Hq, 128)).astype(np.float16)
    pos = 334 if flags & kvq.FLAG_SINK else 333     # cache index of absolute position 334 / 333
    pair = np.zeros((B, Hkv, 128))
    qp = q[:, ::G, 6:8].astype(np.float64)
    pair[..., 6:8] = qp / np.linalg.norm(qp, axis=-1, keepdims=True) * 1000
    k[:, :, pos] = (rope.rotate(pair, -float(pos), BASE) if flags & kvq.FLAG_PRE_ROPE else pair).astype(np.float16)
    k[:, :, pos, :6] = 0
    k[:, :, pos, 8:] = 0
    v[:, :, pos, 77] = 300.0
    v[:, :, pos, 2] = -200.0
    v[:, :, 0, 100] = 250.0
    cache = kvq.KVCache(_shape(kvq, B, Hkv, Hq, 1024, flags))
    kvq.kv_append_and_flush(cache, _dev(k), _dev(v))
    assert cache.n_quant > 400
    out = kvq.kv_decode_attention(cache, _dev(q))
    torch.cuda.synchronize()
    ref = _oracle(kvq, k, v, flags)
    want = oa.decode_attention(ref, q, B, Hkv, rope_base=BASE if flags & 2 else None)
    got = out.cpu().numpy().astype(np.float64)
    err = np.abs(got - want)
    say(f"    max_abs={err.max():.3e}; oracle channel 77 of head 0: {want[0, 0, 77]:.2f}")
    assert np.abs(want[:, ::G, 77]).max() > 30, "the outlier token should dominate"
    assert err.max() <= ATOL


def test_sparse_changes_the_result(kvq):
    """The same tokens in a dense 4-bit cache and a dense-and-sparse one give different outputs, each matching its
    own oracle (a kernel that ignored the outlier section would pass only the first)."""
    rng = np.random.default_rng(78)
    B, Hq, Hkv, N = 1, 4, 2, 600
    k = _keys(rng, (B, Hkv, N, 128))
    v = _values(rng, (B, Hkv, N, 128))
    q = rng.standard_normal((B, Hq, 128)).astype(np.float16)
    outs = {}
    for sparse in (False, True):
        flags = S_R | (kvq.FLAG_SPARSE if sparse else 0)
        shape = kvq.Shape(B, Hkv, Hq, max_tokens=640, bits=4, flags=flags, rope_base=BASE)
        cache = kvq.KVCache(shape)
        kvq.kv_append_and_flush(cache, _dev(k), _dev(v))
        outs[sparse] = kvq.kv_decode_attention(cache, _dev(q)).cpu().numpy().astype(np.float64)
        ref = oc.SliceCache(B * Hkv, bits=4, sink=True, sparse=sparse)
        oc.append_block(ref, k.reshape(B * Hkv, N, 128), v.reshape(B * Hkv, N, 128))
        want = oa.decode_attention(ref, q, B, Hkv, rope_base=BASE)
        assert np.abs(outs[sparse] - want).max() <= ATOL
    assert np.abs(outs[False] - outs[True]).max() > 0.01


def test_decode_sparse_is_deterministic(kvq):
    rng = np.random.default_rng(19)
    B, Hq, Hkv, N = 2, 8, 2, 3000
    k = _keys(rng, (B, Hkv, N, 128))
    v = _values(rng, (B, Hkv, N, 128))
    q = _dev(rng.standard_normal((B, Hq, 128)).astype(np.float16))
    cache = kvq.KVCache(_shape(kvq, B, Hkv, Hq, 3072, S_R))
    kvq.kv_append_and_flush(cache, _dev(k), _dev(v))
    a = kvq.kv_decode_attention(cache, q).clone()
    b = kvq.kv_decode_attention(cache, q)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_kvquant_4bit_sparse_16k_sampled(kvq):
    """The full-size dense-and-sparse workload (B16, 32 heads, 16384 tokens: sink + 16256 quantized + 127 window)
    in the benchmark's launch configuration: records and sink of sampled slices bit-exact, their heads' outputs within
    2e-3 of the oracle, every output finite."""
    import kvsynth
    from kvsynth import device as kdev
    w = kvsynth.WORKLOADS["kvquant_4bit_sparse_16k"]
    assert w.sparse
    say(f"[workload-sparse] {w.name}: B{w.batch} Hq{w.q_heads} Hkv{w.kv_heads} N{w.context}")
    cache = kvq.KVCache(_shape(kvq, w.batch, w.kv_heads, w.q_heads, ((w.context + 31) // 32) * 32, S_R,
                               w.residual))
    K = kdev.kv_to_device(w, kvsynth.K_ID, 0, w.context)
    V = kdev.kv_to_device(w, kvsynth.V_ID, 0, w.context)
    kvq.kv_append_and_flush(cache, K[:, :, :w.prefill], V[:, :, :w.prefill])
    t = w.prefill
    kvq.kv_append_and_flush(cache, K[:, :, t:t + 1], V[:, :, t:t + 1])
    q = kdev.queries_to_device(w, [1])[0]
    out = kvq.kv_decode_attention(cache, q)
    torch.cuda.synchronize()
    del K, V
    say(f"    splits={kvq.kv_decode_attention_splits(cache)} n=({cache.n_sink},{cache.n_quant},{cache.n_resid})")
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    qn = q.cpu().numpy()
    G = w.q_heads // w.kv_heads
    for b, h in [(0, 0), (9, 23), (15, 31)]:
        k = helpers.workload_tokens(w, kvsynth.K_ID, 0, w.context, b, h)
        v = helpers.workload_tokens(w, kvsynth.V_ID, 0, w.context, b, h)
        ref = oc.SliceCache(1, residual_cap=w.residual, bits=4, sink=True, sparse=True)
        oc.append_block(ref, k[None], v[None])
        assert (cache.n_sink, cache.n_quant, cache.n_resid) == (ref.n_sink, ref.n_quant, ref.n_resid)
        s = b * w.kv_heads + h
        g = helpers.records4_from_device(cache.tiles, ref.n_quant // 32, [s])
        want = helpers.oracle_records4(ref)
        assert np.array_equal(g, want), helpers.first_mismatch4(g, want)
        assert np.array_equal(cache.sink.reshape(-1, 512)[s].cpu().numpy(), helpers.oracle_sink(ref)[0])
        o = oa.decode_attention(ref, qn[b, h * G:(h + 1) * G][None], 1, 1, rope_base=w.rope_base)[0]
        err = np.abs(got[b, h * G:(h + 1) * G] - o).max()
        say(f"    slice ({b},{h}) max_abs={err:.3e}")
        assert err <= ATOL
