"""GPU parity of the 4-bit KVQuant-style variant: the HIP path (through the C ABI) against the fp64 CPU oracle.

Bars: 4-bit codes, fp16 scales and zero-points, the sink record and the window bytes bit-exact; attention outputs
within max-abs 2e-3 (fp32 accumulation and binary32 rotation factors on the GPU against float64 in the oracle).
Cases cover keys cached before RoPE (rotated at decode time by absolute position), the attention-sink token,
both together and neither, grouped-query layouts, ragged windows, caches holding only the sink, and splits long
enough that the per-tile rotation is re-anchored.
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
    x = rng.standard_normal(shape).astype(np.float32)
    x[..., [5, 33, 90, 127]] *= 20
    return x.astype(np.float16)


def _shape(kvq, B, Hkv, Hq, max_tokens, flags, R=128):
    return kvq.Shape(B, Hkv, Hq, max_tokens=max_tokens, residual_cap=R, bits=4, flags=flags,
                     rope_base=BASE if flags & kvq.FLAG_PRE_ROPE else 0.0)


def _oracle(kvq, k, v, flags, R=128):
    S = k.shape[0] * k.shape[1]
    ref = oc.SliceCache(S, residual_cap=R, bits=4, sink=bool(flags & kvq.FLAG_SINK))
    oc.append_block(ref, k.reshape(S, -1, 128), v.reshape(S, -1, 128))
    return ref


def _check_state(kvq, cache, ref, B, H, what):
    assert (cache.n_sink, cache.n_quant, cache.n_resid) == (ref.n_sink, ref.n_quant, ref.n_resid), what
    nt = ref.n_quant // 32
    if nt:
        got = helpers.records4_from_device(cache.tiles, nt)
        want = helpers.oracle_records4(ref)
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
    if kind == "normal_outliers":
        x = _keys(rng, shape)
    elif kind == "wide":
        x = rng.uniform(-65504, 65504, shape)
    elif kind == "tiny":
        x = rng.integers(-30, 30, shape) * 2.0 ** -24
    elif kind == "const_and_zero":
        x = rng.standard_normal(shape)
        x[..., :32, :] = 1.25
        x[..., 40, :] = -0.0
        x[..., 64:96, 0:32] = 0.0
        x[..., 70, 0:16] = -0.0
        x[..., :, 100] = 65504.0
        x[..., 3, 100] = -65504.0
    else:
        raise ValueError(kind)
    return np.asarray(x).astype(np.float16)


@pytest.mark.parametrize("kind", ["normal_outliers", "wide", "tiny", "const_and_zero", "ties"])
def test_quantize_4bit_entry_points_bit_exact(kvq, kind):
    say(f"[quant4] kind={kind}")
    rng = np.random.default_rng(zlib.crc32(kind.encode()) + 4)
    B, H, T, tile0 = 2, 3, 256, 2
    if kind == "ties":   # key groups along tokens, value groups along channels, all at or beside half levels
        k = helpers.tie_groups(rng, B * H * (T // 32) * 128, 15).reshape(B, H, T // 32, 128, 32)
        k = np.ascontiguousarray(k.transpose(0, 1, 2, 4, 3)).reshape(B, H, T, 128)
        v = helpers.tie_groups(rng, B * H * T * 4, 15).reshape(B, H, T, 128)
    else:
        k = _family(rng, kind, (B, H, T, 128))
        v = _family(rng, kind, (B, H, T, 128))
    shape = kvq.Shape(B, H, H, max_tokens=T + 32 * tile0 + 64, bits=4)
    tiles = torch.zeros((B, H, shape.max_tokens // 32, 5120), dtype=torch.uint8, device="cuda")
    k_store = _dev(np.ascontiguousarray(k.transpose(0, 2, 1, 3)))
    kvq.kv_quant_keys_per_channel(shape, k_store.permute(0, 2, 1, 3), tile0, tiles)
    torch.cuda.synchronize()
    got = tiles.cpu().numpy().reshape(B * H, -1, 5120)
    assert not got[:, :, 2048:4096].any() and not got[:, :, 4608:].any(), "key call wrote value fields"
    kvq.kv_quant_values_per_token(shape, _dev(v), tile0, tiles)
    torch.cuda.synchronize()
    got = tiles.cpu().numpy().reshape(B * H, -1, 5120)
    ref = oc.SliceCache(B * H, bits=4)
    ref._push_quantized(k.reshape(B * H, T, 128), v.reshape(B * H, T, 128))
    want = helpers.oracle_records4(ref)
    assert not got[:, :tile0].any() and not got[:, tile0 + T // 32:].any(), "wrote outside the tile range"
    sel = got[:, tile0:tile0 + T // 32]
    assert np.array_equal(sel, want), helpers.first_mismatch4(sel, want)
    # values again through a non-contiguous view ([B, T, H, D] storage): the same value fields
    tiles2 = torch.zeros_like(tiles)
    v_store = _dev(np.ascontiguousarray(v.transpose(0, 2, 1, 3)))
    kvq.kv_quant_values_per_token(shape, v_store.permute(0, 2, 1, 3), tile0, tiles2)
    torch.cuda.synchronize()
    got2 = tiles2.cpu().numpy().reshape(B * H, -1, 5120)
    for lo, hi in ((2048, 4096), (4608, 5120)):
        assert np.array_equal(got2[..., lo:hi], got[..., lo:hi]), f"strided values differ in bytes {lo}..{hi}"


def test_append_stream_with_sink(kvq):
    """Prefill (token 0 to the sink), single-token appends across two flushes, then a block append: the sink
    record, tiles and window equal the oracle's token-by-token state, bit for bit."""
    rng = np.random.default_rng(41)
    B, H, R = 2, 3, 128
    total = 300 + 200 + 77
    k = _keys(rng, (B, H, total, 128))
    v = rng.standard_normal((B, H, total, 128)).astype(np.float16)
    flags = kvq.FLAG_SINK | kvq.FLAG_PRE_ROPE
    cache = kvq.KVCache(_shape(kvq, B, H, H, 1024, flags, R))
    ref = oc.SliceCache(B * H, residual_cap=R, bits=4, sink=True)
    kd, vd = _dev(k), _dev(v)
    say("[stream4] prefill 300")
    kvq.kv_append_and_flush(cache, kd[:, :, :300], vd[:, :, :300])
    ref.append(k[:, :, :300].reshape(B * H, 300, 128), v[:, :, :300].reshape(B * H, 300, 128))
    torch.cuda.synchronize()
    _check_state(kvq, cache, ref, B, H, "after prefill")
    for t in range(300, 500):
        kvq.kv_append_and_flush(cache, kd[:, :, t:t + 1], vd[:, :, t:t + 1])
        flushed = ref.n_resid == R
        ref.append_token(k[:, :, t].reshape(B * H, 128), v[:, :, t].reshape(B * H, 128))
        if flushed or t in (301, 499):
            torch.cuda.synchronize()
            say(f"[stream4] token {t} flushed={flushed}")
            _check_state(kvq, cache, ref, B, H, f"token {t}")
    kvq.kv_append_and_flush(cache, kd[:, :, 500:], vd[:, :, 500:])
    ref.append(k[:, :, 500:].reshape(B * H, 77, 128), v[:, :, 500:].reshape(B * H, 77, 128))
    torch.cuda.synchronize()
    _check_state(kvq, cache, ref, B, H, "after block append")


def test_single_token_appends_from_empty(kvq):
    """The very first single-token append fills the sink and nothing else; the second opens the window."""
    rng = np.random.default_rng(42)
    B, H = 1, 2
    k = _keys(rng, (B, H, 3, 128))
    v = rng.standard_normal((B, H, 3, 128)).astype(np.float16)
    cache = kvq.KVCache(_shape(kvq, B, H, H, 256, kvq.FLAG_SINK))
    ref = oc.SliceCache(B * H, bits=4, sink=True)
    for t in range(3):
        kvq.kv_append_and_flush(cache, _dev(k[:, :, t:t + 1]), _dev(v[:, :, t:t + 1]))
        ref.append_token(k[:, :, t].reshape(B * H, 128), v[:, :, t].reshape(B * H, 128))
        torch.cuda.synchronize()
        _check_state(kvq, cache, ref, B, H, f"append {t}")


S_R = 3   # FLAG_SINK | FLAG_PRE_ROPE
CASES = [
    # (B, Hq, Hkv, N, flags, note)
    (1, 1, 1, 1, S_R, "sink only"),
    (1, 1, 1, 2, S_R, "sink + one window token"),
    (1, 1, 1, 33, S_R, "sink + one full window tile"),
    (2, 4, 4, 100, S_R, "all window, ragged"),
    (1, 1, 1, 1024, S_R, "896 quantized + 127 window"),
    (2, 8, 2, 1000, 2, "pre-RoPE, no sink, GQA G=4"),
    (2, 8, 4, 2177, 1, "sink, no RoPE, GQA G=2"),
    (1, 4, 4, 1300, 0, "plain 4-bit"),
    (3, 4, 4, 4226, S_R, "many tiles, window of 1"),
    (1, 6, 2, 3000, S_R, "G=3"),
    (4, 128, 4, 10000, S_R, "splits of ~80 tiles: rotation re-anchored inside a split"),
]


@pytest.mark.parametrize("B,Hq,Hkv,N,flags,note", CASES)
def test_decode_4bit_matches_oracle(kvq, B, Hq, Hkv, N, flags, note):
    say(f"[decode4] B={B} Hq={Hq} Hkv={Hkv} N={N} flags={flags} ({note})")
    rng = np.random.default_rng(N * 11 + Hq + 100 * flags)
    k = _keys(rng, (B, Hkv, N, 128))
    v = rng.standard_normal((B, Hkv, N, 128)).astype(np.float16)
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


def test_rope_changes_the_result(kvq):
    """The same cache contents attended with and without the pre-RoPE flag differ, and each matches its own oracle
    (a kernel that ignored the rotation would pass only the second)."""
    rng = np.random.default_rng(77)
    B, Hq, Hkv, N = 1, 4, 2, 600
    k = _keys(rng, (B, Hkv, N, 128))
    v = rng.standard_normal((B, Hkv, N, 128)).astype(np.float16)
    q = rng.standard_normal((B, Hq, 128)).astype(np.float16)
    outs = {}
    for flags in (kvq.FLAG_SINK, kvq.FLAG_SINK | kvq.FLAG_PRE_ROPE):
        cache = kvq.KVCache(_shape(kvq, B, Hkv, Hq, 640, flags))
        kvq.kv_append_and_flush(cache, _dev(k), _dev(v))
        outs[flags] = kvq.kv_decode_attention(cache, _dev(q)).cpu().numpy().astype(np.float64)
        ref = _oracle(kvq, k, v, flags)
        want = oa.decode_attention(ref, q, B, Hkv, rope_base=BASE if flags & 2 else None)
        assert np.abs(outs[flags] - want).max() <= ATOL
    assert np.abs(outs[1] - outs[3]).max() > 0.05


@pytest.mark.parametrize("variant", ["zero_query", "large_query", "sm_scale", "constant_values", "peaked_rotated"])
def test_decode_4bit_special_inputs(kvq, variant):
    say(f"[decode4-special] {variant}")
    rng = np.random.default_rng(6)
    B, Hq, Hkv, N = 2, 8, 2, 777
    flags = kvq.FLAG_SINK | kvq.FLAG_PRE_ROPE
    k = _keys(rng, (B, Hkv, N, 128))
    v = rng.standard_normal((B, Hkv, N, 128)).astype(np.float16)
    q = rng.standard_normal((B, Hq, 128)).astype(np.float16)
    sm = 0.0
    if variant == "zero_query":
        q[:] = 0
    elif variant == "large_query":
        q = (q.astype(np.float32) * 300).astype(np.float16)
        k = (k.astype(np.float32) / 20).astype(np.float16)
    elif variant == "sm_scale":
        sm = 0.021
    elif variant == "constant_values":
        v[:] = np.float16(0.7)
    elif variant == "peaked_rotated":
        # the pre-RoPE key at position 333 is the first query head of its group rotated back by 333 (x4): after
        # the decode-time rotation it points along that query and dominates its softmax
        G = Hq // Hkv
        k[:, :, 333] = rope.rotate(q[:, ::G].astype(np.float64) * 4, -333.0, BASE).astype(np.float16)
    cache = kvq.KVCache(_shape(kvq, B, Hkv, Hq, 1024, flags))
    kvq.kv_append_and_flush(cache, _dev(k), _dev(v))
    out = kvq.kv_decode_attention(cache, _dev(q), sm_scale=sm)
    torch.cuda.synchronize()
    ref = _oracle(kvq, k, v, flags)
    want = oa.decode_attention(ref, q, B, Hkv, sm if sm > 0 else None, rope_base=BASE)
    err = np.abs(out.cpu().numpy().astype(np.float64) - want)
    say(f"    max_abs={err.max():.3e}")
    assert err.max() <= ATOL


@pytest.mark.parametrize("N", [1000, 1102])
def test_4bit_window_rows_past_length_are_ignored(kvq, N):
    """Window rows past the cache's length hold NaN: the ragged last window tile must mask them."""
    say(f"[decode4-window-nan] N={N}")
    rng = np.random.default_rng(N + 4)
    B, Hq, Hkv = 2, 8, 2
    flags = kvq.FLAG_SINK | kvq.FLAG_PRE_ROPE
    k = _keys(rng, (B, Hkv, N, 128))
    v = rng.standard_normal((B, Hkv, N, 128)).astype(np.float16)
    q = rng.standard_normal((B, Hq, 128)).astype(np.float16)
    cache = kvq.KVCache(_shape(kvq, B, Hkv, Hq, 1280, flags))
    cache.k_res.fill_(float("nan"))
    cache.v_res.fill_(float("nan"))
    kvq.kv_append_and_flush(cache, _dev(k), _dev(v))
    assert cache.n_resid % 32 != 0
    out = kvq.kv_decode_attention(cache, _dev(q))
    torch.cuda.synchronize()
    ref = _oracle(kvq, k, v, flags)
    got = out.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    err = np.abs(got - oa.decode_attention(ref, q, B, Hkv, rope_base=BASE))
    say(f"    n_resid={cache.n_resid} max_abs={err.max():.3e}")
    assert err.max() <= ATOL


def test_decode_4bit_is_deterministic(kvq):
    rng = np.random.default_rng(9)
    B, Hq, Hkv, N = 2, 8, 2, 3000
    k = _keys(rng, (B, Hkv, N, 128))
    v = rng.standard_normal((B, Hkv, N, 128)).astype(np.float16)
    q = _dev(rng.standard_normal((B, Hq, 128)).astype(np.float16))
    cache = kvq.KVCache(_shape(kvq, B, Hkv, Hq, 3072, 3))
    kvq.kv_append_and_flush(cache, _dev(k), _dev(v))
    a = kvq.kv_decode_attention(cache, q).clone()
    b = kvq.kv_decode_attention(cache, q)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_kvquant_4bit_16k_sampled(kvq):
    """The full-size KVQuant-style workload (B16, 32 heads, 16384 tokens: sink + 16256 quantized + 127 window) in
    the benchmark's launch configuration: tiles and sink records of sampled slices bit-exact, their heads' outputs
    within 2e-3 of the oracle (pre-RoPE keys rotated by absolute position), every output finite."""
    import kvsynth
    from kvsynth import device as kdev
    w = kvsynth.WORKLOADS["kvquant_4bit_16k"]
    say(f"[workload4] {w.name}: B{w.batch} Hq{w.q_heads} Hkv{w.kv_heads} N{w.context}")
    flags = kvq.FLAG_SINK | kvq.FLAG_PRE_ROPE
    cache = kvq.KVCache(_shape(kvq, w.batch, w.kv_heads, w.q_heads, ((w.context + 31) // 32) * 32, flags,
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
    for b, h in [(0, 0), (7, 19), (15, 31)]:
        k = helpers.workload_tokens(w, kvsynth.K_ID, 0, w.context, b, h)
        v = helpers.workload_tokens(w, kvsynth.V_ID, 0, w.context, b, h)
        ref = oc.SliceCache(1, residual_cap=w.residual, bits=4, sink=True)
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
