"""The allocation-free decode entry point (kv_decode_attention_noalloc, split partials in the library's static
per-GPU scratch) against kv_decode_attention with a caller workspace, through the C ABI: the same kernels, so the
outputs must be equal bit for bit, and both within max-abs 2e-3 of the fp64 oracle. Two calls in a row, the second
on a smaller input (fewer sequences, shorter context, fewer splits), so the second call runs over scratch the first
one left behind. Also run: the 4-bit variant, and a call whose partials would not fit the array (rejected on the
host with KVQ_E_SCRATCH, nothing launched)."""
import ctypes
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

from oracle import attention as oa  # noqa: E402
from oracle import cache as oc  # noqa: E402

ATOL = 2e-3


@pytest.fixture(scope="module")
def kvq():
    import decode_attention_quant_amd as m
    return m


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _case(kvq, rng, B, Hq, Hkv, N, bits=2, flags=0):
    k = rng.standard_normal((B, Hkv, N, 128)).astype(np.float32)
    k[..., [5, 33, 90, 127]] *= 20
    k = k.astype(np.float16)
    v = rng.standard_normal((B, Hkv, N, 128)).astype(np.float16)
    q = rng.standard_normal((B, Hq, 128)).astype(np.float16)
    shape = kvq.Shape(B, Hkv, Hq, max_tokens=((N + 31) // 32) * 32 + 32, bits=bits, flags=flags,
                      rope_base=10000.0 if flags & kvq.FLAG_PRE_ROPE else 0.0)
    cache = kvq.KVCache(shape)
    kvq.kv_append_and_flush(cache, _dev(k), _dev(v))
    S = B * Hkv
    ref = oc.SliceCache(S, bits=bits, sink=bool(flags & kvq.FLAG_SINK))
    oc.append_block(ref, k.reshape(S, N, 128), v.reshape(S, N, 128))
    want = oa.decode_attention(ref, q, B, Hkv, rope_base=10000.0 if flags & kvq.FLAG_PRE_ROPE else None)
    return cache, _dev(q), want


def _both(kvq, cache, q):
    """(noalloc output, workspace output), each through the C ABI on the current stream"""
    lib = kvq.library()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    s = cache.shape
    out_n = torch.full((s.batch, s.q_heads, 128), float("nan"), dtype=torch.float32, device="cuda")
    out_w = torch.full_like(out_n, float("nan"))
    rc = lib.kv_decode_attention_noalloc(ctypes.byref(cache._cshape), ctypes.byref(cache.c),
                                         ctypes.c_void_p(q.data_ptr()), 0.0, ctypes.c_void_p(out_n.data_ptr()), st)
    assert rc == 0, kvq.status_string(rc)
    need = lib.kv_decode_attention_workspace_bytes(ctypes.byref(cache._cshape), ctypes.byref(cache.c))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    rc = lib.kv_decode_attention(ctypes.byref(cache._cshape), ctypes.byref(cache.c), ctypes.c_void_p(q.data_ptr()),
                                 0.0, ctypes.c_void_p(out_w.data_ptr()), ctypes.c_void_p(ws.data_ptr()), need, st)
    assert rc == 0, kvq.status_string(rc)
    torch.cuda.synchronize()
    return out_n.cpu().numpy(), out_w.cpu().numpy()


def test_noalloc_equals_workspace_call_twice_then_smaller(kvq):
    rng = np.random.default_rng(77)
    for B, Hq, Hkv, N in ((4, 32, 8, 5000), (2, 8, 2, 700)):
        cache, q, want = _case(kvq, rng, B, Hq, Hkv, N)
        splits = kvq.kv_decode_attention_splits(cache)
        say(f"[noalloc] B={B} Hq={Hq} Hkv={Hkv} N={N} splits={splits} "
            f"partials={kvq.kv_decode_attention_workspace_bytes(cache)} B")
        got_n, got_w = _both(kvq, cache, q)
        assert np.array_equal(got_n.view(np.uint32), got_w.view(np.uint32)), "noalloc differs from the workspace call"
        err = np.abs(got_n.astype(np.float64) - want).max()
        say(f"    bit-equal to the workspace call; max_abs vs oracle {err:.3e}")
        assert err <= ATOL


def test_noalloc_4bit_with_sink_and_rope(kvq):
    rng = np.random.default_rng(78)
    cache, q, want = _case(kvq, rng, 2, 8, 2, 1500, bits=4, flags=kvq.FLAG_SINK | kvq.FLAG_PRE_ROPE)
    got_n, got_w = _both(kvq, cache, q)
    assert np.array_equal(got_n.view(np.uint32), got_w.view(np.uint32))
    assert np.abs(got_n.astype(np.float64) - want).max() <= ATOL


def test_noalloc_rejects_partials_beyond_the_scratch(kvq):
    """2048 sequences, 32 query heads: the partials (34 MB) exceed 16 MiB; rejected before anything is launched (the
    pointers below are never dereferenced)."""
    fake = 0x7f0000000000
    shape = kvq.KvqShape(2048, 8, 32, 128, 2, 32, 128, 0, 1 << 20, 0.0)
    cache = kvq.KvqCache(fake, fake + 4096, fake + 8192, 1 << 20, 5, 0, None)
    lib = kvq.library()
    need = lib.kv_decode_attention_workspace_bytes(ctypes.byref(shape), ctypes.byref(cache))
    assert need > kvq.NOALLOC_SCRATCH_BYTES
    rc = lib.kv_decode_attention_noalloc(ctypes.byref(shape), ctypes.byref(cache), ctypes.c_void_p(fake),
                                         0.0, ctypes.c_void_p(fake + 4096), None)
    assert rc == kvq.E_SCRATCH


def test_noalloc_2bit_dense_and_sparse(kvq):
    """The allocation-free call on a 2-bit dense-and-sparse cache equals the workspace call bit for bit."""
    rng = np.random.default_rng(73)
    B, Hq, Hkv, N = 3, 12, 3, 900
    k = rng.standard_normal((B, Hkv, N, 128)).astype(np.float32)
    k[rng.random(k.shape) < 0.01] *= 30
    v = rng.standard_normal((B, Hkv, N, 128)).astype(np.float16)
    q = rng.standard_normal((B, Hq, 128)).astype(np.float16)
    cache = kvq.KVCache(kvq.Shape(B, Hkv, Hq, max_tokens=1024, flags=kvq.FLAG_SPARSE))
    kvq.kv_append_and_flush(cache, _dev(k.astype(np.float16)), _dev(v))
    want = kvq.kv_decode_attention(cache, _dev(q))
    got = torch.full_like(want, float("nan"))
    kvq.kv_decode_attention_noalloc(cache, _dev(q), got)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
