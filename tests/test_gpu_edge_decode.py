"""GPU parity of decode attention on the quantizer's edge cases, 2-bit and 4-bit, through the C ABI against the fp64
CPU oracle.

The quantizer's degenerate groups reach attention here, not only the packed records (2-bit with and without
dense-and-sparse groups, 4-bit with three flag sets):
- constant key groups and all-zero (and -0) groups: s = 0, every code 0, a score is the zero-point term alone;
- keys offset by 1000 (fp16 steps of 0.5): the zero-point term dominates every score, and the scores of all tokens
  sit near one large common value;
- wide keys (|K| up to 1e4, and channels scaled by 5000): the folded query q * s_K reaches thousands, which
  stresses its fp16 high/low split, and the softmax is nearly one-hot;
- tiny-range groups (a per-channel constant plus integer multiples of 2^-24): binary16-subnormal scales;
- tiles of those families in turn along the tokens, so one split rescales its running maximum across them;
- values scaled by 100.

Bar: max-abs 2e-3 while the values are O(1) (|v| <= 8); for values scaled past that, the same relative precision,
2e-3 * max|v| / 8 (fp32 accumulation errors scale with the values).
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

BASE = 10000.0
KINDS = ["const_tiles", "zero_keys", "offset_1000", "wide_1e4", "wide_channels", "tiny_range", "tile_mix",
         "values_x100"]


@pytest.fixture(scope="module")
def kvq():
    import decode_attention_quant_amd as m
    return m


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _dev(x: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _normal_keys(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    x[..., [5, 33, 90, 127]] *= 20
    return x


def _family_keys(rng, kind, shape):
    """float32 keys of one family (exact binary16 values after the final cast)"""
    B, H, N, D = shape
    if kind == "const_tiles":
        x = _normal_keys(rng, shape)
        x[:, :, :64] = rng.standard_normal((B, H, 1, D)) * 3     # tiles 0 and 1: every key group constant
        x[:, :, 96:128] = 0.0                                       # tile 3: zeros, a few of them -0
        x[:, :, 100, :40] = -0.0
        return x
    if kind == "zero_keys":
        x = np.zeros(shape, np.float32)
        x[..., 1::3, 7] = -0.0
        return x
    if kind == "offset_1000":
        return 1000.0 + rng.standard_normal(shape)
    if kind == "wide_1e4":
        return rng.uniform(-1e4, 1e4, shape)
    if kind == "wide_channels":
        x = rng.standard_normal(shape).astype(np.float32)
        x[..., [3, 64, 65, 111]] *= 5000
        return x
    if kind == "tiny_range":
        c = rng.standard_normal((B, H, 1, D))
        return c + rng.integers(-40, 40, shape) * 2.0 ** -24
    raise ValueError(kind)


def _keys_values(rng, kind, shape):
    if kind == "tile_mix":
        fams = ["normal", "const_tiles", "wide_1e4", "tiny_range", "offset_1000", "zero_keys", "wide_channels"]
        x = np.empty(shape, np.float32)
        for t0 in range(0, shape[2], 32):
            f = fams[(t0 // 32) % len(fams)]
            n = min(32, shape[2] - t0)
            sub = (shape[0], shape[1], n, shape[3])
            if f == "normal":
                x[:, :, t0:t0 + n] = _normal_keys(rng, sub)
            elif f == "const_tiles":
                x[:, :, t0:t0 + n] = rng.standard_normal((shape[0], shape[1], 1, shape[3])) * 3
            else:
                x[:, :, t0:t0 + n] = _family_keys(rng, f, sub)
        k = x
    elif kind == "values_x100":
        k = _normal_keys(rng, shape)
    else:
        k = _family_keys(rng, kind, shape)
    v = rng.standard_normal(shape).astype(np.float32)
    if kind == "values_x100":
        v *= 100
    return k.astype(np.float16), v.astype(np.float16)


def _tolerance(v: np.ndarray) -> float:
    vmax = float(np.abs(v.astype(np.float32)).max())
    return 2e-3 * max(1.0, vmax / 8.0)


@pytest.mark.parametrize("sparse", [False, True], ids=["dense", "dense-and-sparse"])
@pytest.mark.parametrize("kind", KINDS)
def test_decode_2bit_edge_inputs(kvq, kind, sparse):
    B, Hq, Hkv, N = 2, 8, 2, 1187          # 1152 quantized tokens (36 tiles) and a ragged window of 35
    say(f"[edge2] {kind} sparse={sparse} B={B} Hq={Hq} Hkv={Hkv} N={N}")
    rng = np.random.default_rng(zlib.crc32(kind.encode()) + (100 if sparse else 0))
    k, v = _keys_values(rng, kind, (B, Hkv, N, 128))
    q = rng.standard_normal((B, Hq, 128)).astype(np.float16)
    cache = kvq.KVCache(kvq.Shape(B, Hkv, Hq, max_tokens=1280, flags=kvq.FLAG_SPARSE if sparse else 0))
    kvq.kv_append_and_flush(cache, _dev(k), _dev(v))
    out = kvq.kv_decode_attention(cache, _dev(q))
    torch.cuda.synchronize()
    ref = oc.SliceCache(B * Hkv, sparse=sparse)
    oc.append_block(ref, k.reshape(B * Hkv, N, 128), v.reshape(B * Hkv, N, 128))
    assert (cache.n_quant, cache.n_resid) == (ref.n_quant, ref.n_resid)
    want = oa.decode_attention(ref, q, B, Hkv)
    got = out.cpu().numpy().astype(np.float64)
    err = np.abs(got - want)
    tol = _tolerance(v)
    say(f"    splits={kvq.kv_decode_attention_splits(cache)} n_quant={cache.n_quant} n_resid={cache.n_resid} "
        f"max_abs={err.max():.3e} tol={tol:.1e} max|out|={np.abs(want).max():.2f}")
    assert np.all(np.isfinite(got))
    assert err.max() <= tol


FLAGS4 = [(3, "sink+pre-RoPE"), (0, "plain"), (7, "sink+pre-RoPE+sparse")]


@pytest.mark.parametrize("flags,fnote", FLAGS4)
@pytest.mark.parametrize("kind", KINDS)
def test_decode_4bit_edge_inputs(kvq, kind, flags, fnote):
    B, Hq, Hkv, N = 2, 8, 2, 1188
    say(f"[edge4] {kind} flags={flags} ({fnote}) B={B} Hq={Hq} Hkv={Hkv} N={N}")
    rng = np.random.default_rng(zlib.crc32(kind.encode()) + flags)
    k, v = _keys_values(rng, kind, (B, Hkv, N, 128))
    q = rng.standard_normal((B, Hq, 128)).astype(np.float16)
    rope_base = BASE if flags & kvq.FLAG_PRE_ROPE else 0.0
    cache = kvq.KVCache(kvq.Shape(B, Hkv, Hq, max_tokens=1280, bits=4, flags=flags, rope_base=rope_base))
    kvq.kv_append_and_flush(cache, _dev(k), _dev(v))
    out = kvq.kv_decode_attention(cache, _dev(q))
    torch.cuda.synchronize()
    S = B * Hkv
    ref = oc.SliceCache(S, bits=4, sink=bool(flags & kvq.FLAG_SINK), sparse=bool(flags & kvq.FLAG_SPARSE))
    oc.append_block(ref, k.reshape(S, N, 128), v.reshape(S, N, 128))
    assert (cache.n_sink, cache.n_quant, cache.n_resid) == (ref.n_sink, ref.n_quant, ref.n_resid)
    want = oa.decode_attention(ref, q, B, Hkv, rope_base=rope_base or None)
    got = out.cpu().numpy().astype(np.float64)
    err = np.abs(got - want)
    tol = _tolerance(v)
    say(f"    splits={kvq.kv_decode_attention_splits(cache)} max_abs={err.max():.3e} tol={tol:.1e} "
        f"max|out|={np.abs(want).max():.2f}")
    assert np.all(np.isfinite(got))
    assert err.max() <= tol
