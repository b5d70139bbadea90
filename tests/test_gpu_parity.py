"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle on the same seeded inputs.

Bars: packed codes, fp16 scales and zero-points, and residual-window bytes bit-exact; attention outputs within
max-abs 2e-3 (fp32 accumulation on the GPU against float64 in the oracle).
"""
import sys
import zlib

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import kvsynth  # noqa: E402
from oracle import cache as oc  # noqa: E402
from tests import helpers  # noqa: E402

ATOL = 2e-3


@pytest.fixture(scope="module")
def kvq():
    import decode_attention_quant_amd as m
    return m


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _dev(x: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _family(rng, kind, shape):
    if kind == "normal_outliers":
        x = rng.standard_normal(shape).astype(np.float32)
        x[..., [5, 33, 90, 127]] *= 20
    elif kind == "wide":
        x = rng.uniform(-65504, 65504, shape)
    elif kind == "tiny":
        x = rng.integers(-30, 30, shape) * 2.0 ** -24
    elif kind == "const_and_zero":
        x = rng.standard_normal(shape)
        x[..., :32, :] = 1.25                      # tile 0: every key group constant
        x[..., 40, :] = -0.0
        x[..., 64:96, 0:32] = 0.0                  # value groups of zeros (mixed signs below)
        x[..., 70, 0:16] = -0.0
        x[..., :, 100] = 65504.0
        x[..., 3, 100] = -65504.0
    else:
        raise ValueError(kind)
    return x.astype(np.float16)


@pytest.mark.parametrize("kind", ["normal_outliers", "wide", "tiny", "const_and_zero", "ties"])
def test_quantize_entry_points_bit_exact(kvq, kind):
    say(f"[quant] kind={kind}")
    rng = np.random.default_rng(zlib.crc32(kind.encode()))
    B, H, T, tile0 = 2, 3, 256, 2
    if kind == "ties":   # key groups along tokens, value groups along channels, all at or beside half levels
        k = helpers.tie_groups(rng, B * H * (T // 32) * 128, 3).reshape(B, H, T // 32, 128, 32)
        k = np.ascontiguousarray(k.transpose(0, 1, 2, 4, 3)).reshape(B, H, T, 128)
        v = helpers.tie_groups(rng, B * H * T * 4, 3).reshape(B, H, T, 128)
    else:
        k = _family(rng, kind, (B, H, T, 128))
        v = _family(rng, kind, (B, H, T, 128))
    shape = kvq.Shape(B, H, H, max_tokens=T + 32 * tile0 + 64)
    tiles = torch.zeros((B, H, shape.max_tokens // 32, 3072), dtype=torch.uint8, device="cuda")
    # keys through a non-contiguous view ([B, T, H, D] storage), values contiguous
    k_store = _dev(np.ascontiguousarray(k.transpose(0, 2, 1, 3)))
    kvq.kv_quant_keys_per_channel(shape, k_store.permute(0, 2, 1, 3), tile0, tiles)
    torch.cuda.synchronize()
    got = tiles.cpu().numpy().reshape(B * H, -1, 3072)
    assert not got[:, :, 1024:2048].any() and not got[:, :, 2560:].any(), "key call wrote value fields"
    kvq.kv_quant_values_per_token(shape, _dev(v), tile0, tiles)
    torch.cuda.synchronize()
    got = tiles.cpu().numpy().reshape(B * H, -1, 3072)
    ref = oc.SliceCache(B * H)
    ref._push_quantized(k.reshape(B * H, T, 128), v.reshape(B * H, T, 128))
    want = helpers.oracle_records(ref)
    assert not got[:, :tile0].any() and not got[:, tile0 + T // 32:].any(), "wrote outside the tile range"
    sel = got[:, tile0:tile0 + T // 32]
    assert np.array_equal(sel, want), helpers.first_mismatch(sel, want)
    # values again through a non-contiguous view ([B, T, H, D] storage): the same value fields
    tiles2 = torch.zeros_like(tiles)
    v_store = _dev(np.ascontiguousarray(v.transpose(0, 2, 1, 3)))
    kvq.kv_quant_values_per_token(shape, v_store.permute(0, 2, 1, 3), tile0, tiles2)
    torch.cuda.synchronize()
    got2 = tiles2.cpu().numpy().reshape(B * H, -1, 3072)
    for lo, hi in ((1024, 2048), (2560, 3072)):
        assert np.array_equal(got2[..., lo:hi], got[..., lo:hi]), f"strided values differ in bytes {lo}..{hi}"


def _check_state(kvq, cache, ref, B, H, what):
    assert (cache.n_quant, cache.n_resid) == (ref.n_quant, ref.n_resid), what
    nt = ref.n_quant // 32
    if nt:
        got = helpers.records_from_device(cache.tiles, nt)
        want = helpers.oracle_records(ref)
        assert np.array_equal(got, want), f"{what}: " + helpers.first_mismatch(got, want)
    nr = ref.n_resid
    kr = cache.k_res[:, :, :nr].reshape(B * H, nr, 128).cpu().numpy()
    vr = cache.v_res[:, :, :nr].reshape(B * H, nr, 128).cpu().numpy()
    assert np.array_equal(kr.view(np.uint16), ref.k_res.view(np.uint16)), what
    assert np.array_equal(vr.view(np.uint16), ref.v_res.view(np.uint16)), what


def test_append_and_flush_stream(kvq):
    """Prefill, single-token decode appends across two flushes, then a block append: state equals the oracle's
    token-by-token state machine, bit for bit, after every flush."""
    rng = np.random.default_rng(21)
    B, H, R = 2, 3, 128
    total = 300 + 200 + 77
    k = _family(rng, "normal_outliers", (B, H, total, 128))
    v = rng.standard_normal((B, H, total, 128)).astype(np.float16)
    shape = kvq.Shape(B, H, H, max_tokens=1024, residual_cap=R)
    cache = kvq.KVCache(shape)
    ref = oc.SliceCache(B * H, residual_cap=R)
    kd, vd = _dev(k), _dev(v)
    say("[stream] prefill 300")
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
            say(f"[stream] step token {t} flushed={flushed}")
            _check_state(kvq, cache, ref, B, H, f"token {t}")
    kvq.kv_append_and_flush(cache, kd[:, :, 500:], vd[:, :, 500:])
    ref.append(k[:, :, 500:].reshape(B * H, 77, 128), v[:, :, 500:].reshape(B * H, 77, 128))
    torch.cuda.synchronize()
    _check_state(kvq, cache, ref, B, H, "after block append")


CASES = [
    # (B, Hq, Hkv, N, note)
    (1, 1, 1, 1, "single token"),
    (1, 1, 1, 32, "one full residual tile"),
    (2, 4, 4, 100, "all residual, ragged"),
    (1, 1, 1, 1024, "tiny workload shape"),
    (2, 8, 2, 1000, "GQA G=4, ragged residual 104"),
    (2, 8, 4, 2177, "GQA G=2"),
    (1, 16, 2, 1300, "GQA G=8: two head chunks per KV head"),
    (1, 10, 2, 700, "GQA G=5: chunk of 4 and chunk of 1"),
    (3, 4, 4, 4225, "many tiles, residual of 1"),
    (1, 2, 1, 5000, "G=2 long"),
]


@pytest.mark.parametrize("B,Hq,Hkv,N,note", CASES)
def test_decode_attention_matches_oracle(kvq, B, Hq, Hkv, N, note):
    say(f"[decode] B={B} Hq={Hq} Hkv={Hkv} N={N} ({note})")
    rng = np.random.default_rng(N * 7 + Hq)
    k = _family(rng, "normal_outliers", (B, Hkv, N, 128))
    v = rng.standard_normal((B, Hkv, N, 128)).astype(np.float16)
    q = rng.standard_normal((B, Hq, 128)).astype(np.float16)
    shape = kvq.Shape(B, Hkv, Hq, max_tokens=((N + 31) // 32) * 32 + 32)
    cache = kvq.KVCache(shape)
    kvq.kv_append_and_flush(cache, _dev(k), _dev(v))
    out = kvq.kv_decode_attention(cache, _dev(q))
    torch.cuda.synchronize()
    ref = oc.SliceCache(B * Hkv)
    oc.append_block(ref, k.reshape(B * Hkv, N, 128), v.reshape(B * Hkv, N, 128))
    want = helpers.oracle_out(ref, q, B, Hkv)
    got = out.cpu().numpy().astype(np.float64)
    err = np.abs(got - want)
    say(f"    splits={kvq.kv_decode_attention_splits(cache)} max_abs={err.max():.3e} "
        f"p99.9={np.quantile(err, 0.999):.3e}")
    assert np.all(np.isfinite(got))
    assert err.max() <= ATOL


@pytest.mark.parametrize("variant", ["zero_query", "large_query", "sm_scale", "constant_values", "peaked"])
def test_decode_attention_special_inputs(kvq, variant):
    say(f"[decode-special] {variant}")
    rng = np.random.default_rng(5)
    B, Hq, Hkv, N = 2, 8, 2, 777
    k = _family(rng, "normal_outliers", (B, Hkv, N, 128))
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
    elif variant == "peaked":
        k[:, :, 333] = (q[:, ::Hq // Hkv].astype(np.float32) * 4).astype(np.float16)
    shape = kvq.Shape(B, Hkv, Hq, max_tokens=1024)
    cache = kvq.KVCache(shape)
    kvq.kv_append_and_flush(cache, _dev(k), _dev(v))
    out = kvq.kv_decode_attention(cache, _dev(q), sm_scale=sm)
    torch.cuda.synchronize()
    ref = oc.SliceCache(B * Hkv)
    oc.append_block(ref, k.reshape(B * Hkv, N, 128), v.reshape(B * Hkv, N, 128))
    want = helpers.oracle_out(ref, q, B, Hkv, sm if sm > 0 else None)
    err = np.abs(out.cpu().numpy().astype(np.float64) - want)
    say(f"    max_abs={err.max():.3e}")
    assert err.max() <= ATOL


def test_decode_is_deterministic(kvq):
    rng = np.random.default_rng(8)
    B, Hq, Hkv, N = 2, 8, 2, 3000
    k = _family(rng, "normal_outliers", (B, Hkv, N, 128))
    v = rng.standard_normal((B, Hkv, N, 128)).astype(np.float16)
    q = _dev(rng.standard_normal((B, Hq, 128)).astype(np.float16))
    cache = kvq.KVCache(kvq.Shape(B, Hkv, Hq, max_tokens=3072))
    kvq.kv_append_and_flush(cache, _dev(k), _dev(v))
    a = kvq.kv_decode_attention(cache, q).clone()
    b = kvq.kv_decode_attention(cache, q)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


FP16_CASES = [
    # (B, Hq, Hkv, N, window capacity, note)
    (1, 1, 1, 1, 64, "one token"),
    (2, 8, 2, 1000, 1024, "GQA G=4, ragged last tile"),
    (1, 4, 4, 4096, 4096, "MHA, window full"),
    (2, 16, 2, 2500, 2560, "G=8, two head chunks"),
]


@pytest.mark.parametrize("B,Hq,Hkv,N,cap,note", FP16_CASES)
def test_decode_all_fp16_cache(kvq, B, Hq, Hkv, N, cap, note):
    """A window as large as the context: nothing is quantized and the call is plain fp16 attention (the comparator
    the 2-bit cache is measured against)."""
    say(f"[decode-fp16] B={B} Hq={Hq} Hkv={Hkv} N={N} cap={cap} ({note})")
    rng = np.random.default_rng(N + 31 * Hq)
    k = _family(rng, "normal_outliers", (B, Hkv, N, 128))
    v = rng.standard_normal((B, Hkv, N, 128)).astype(np.float16)
    q = rng.standard_normal((B, Hq, 128)).astype(np.float16)
    shape = kvq.Shape(B, Hkv, Hq, residual_cap=cap, max_tokens=cap)
    cache = kvq.KVCache(shape)
    kvq.kv_append_and_flush(cache, _dev(k), _dev(v))
    assert (cache.n_quant, cache.n_resid) == (0, N)
    out = kvq.kv_decode_attention(cache, _dev(q))
    torch.cuda.synchronize()
    ref = oc.SliceCache(B * Hkv, residual_cap=cap)
    oc.append_block(ref, k.reshape(B * Hkv, N, 128), v.reshape(B * Hkv, N, 128))
    assert (ref.n_quant, ref.n_resid) == (0, N)
    want = helpers.oracle_out(ref, q, B, Hkv)
    got = out.cpu().numpy().astype(np.float64)
    err = np.abs(got - want)
    say(f"    splits={kvq.kv_decode_attention_splits(cache)} max_abs={err.max():.3e}")
    assert np.all(np.isfinite(got))
    assert err.max() <= ATOL


@pytest.mark.parametrize("N", [1000, 1101])
def test_window_rows_past_length_are_ignored(kvq, N):
    """Window rows past the cache's length hold arbitrary bytes (here NaN): the ragged last window tile must mask
    them in the scores and in P V."""
    say(f"[decode-window-nan] N={N}")
    rng = np.random.default_rng(N)
    B, Hq, Hkv = 2, 8, 2
    k = _family(rng, "normal_outliers", (B, Hkv, N, 128))
    v = rng.standard_normal((B, Hkv, N, 128)).astype(np.float16)
    q = rng.standard_normal((B, Hq, 128)).astype(np.float16)
    cache = kvq.KVCache(kvq.Shape(B, Hkv, Hq, max_tokens=1280))
    cache.k_res.fill_(float("nan"))
    cache.v_res.fill_(float("nan"))
    kvq.kv_append_and_flush(cache, _dev(k), _dev(v))
    assert cache.n_resid % 32 != 0
    out = kvq.kv_decode_attention(cache, _dev(q))
    torch.cuda.synchronize()
    ref = oc.SliceCache(B * Hkv)
    oc.append_block(ref, k.reshape(B * Hkv, N, 128), v.reshape(B * Hkv, N, 128))
    got = out.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    err = np.abs(got - helpers.oracle_out(ref, q, B, Hkv))
    say(f"    n_resid={cache.n_resid} max_abs={err.max():.3e}")
    assert err.max() <= ATOL
