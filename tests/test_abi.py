"""The C-ABI library loads, exports every entry point ``include/kvq.h`` declares, and rejects bad arguments on the
host with the documented status codes before anything reaches the GPU (no compute call is made here; every
call below fails validation, so no pointer is dereferenced and nothing is launched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")
LIB = os.path.join(ROOT, "decode_attention_quant_amd", "libkvq.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libkvq.so not built (run __graft_entry__.build())")


def declared_functions():
    src = open(HEADER).read()
    return re.findall(r"KVQ_API\s+[\w\s\*]+?\b(\w+)\s*\(", src)


def test_header_declares_the_four_operations_and_helpers():
    names = set(declared_functions())
    assert {"kv_quant_keys_per_channel", "kv_quant_values_per_token", "kv_append_and_flush",
            "kv_decode_attention"} <= names
    assert {"kv_decode_attention_workspace_bytes", "kv_decode_attention_splits", "kvq_status_string"} <= names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_only_declared_symbols_are_exported():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert exported == set(declared_functions())


@pytest.fixture(scope="module")
def kvq():
    import decode_attention_quant_amd as m
    return m


def _shape(kvq, **kw):
    d = dict(batch=2, kv_heads=2, q_heads=4, head_dim=128, bits=2, group=32, residual_cap=128, flags=0,
             max_tokens=1024, rope_base=0.0)
    d.update(kw)
    return kvq.KvqShape(**d)


FAKE = 0x7f0000000000     # 16-byte aligned, never dereferenced: every call below fails validation first


def _cache(kvq, n_quant=0, n_resid=0, tiles=FAKE, k_res=FAKE + 4096, v_res=FAKE + 8192, n_sink=0, sink=None):
    return kvq.KvqCache(tiles, k_res, v_res, n_quant, n_resid, n_sink, sink)


def test_status_strings(kvq):
    for code in range(0, -11, -1):
        assert kvq.status_string(code) and kvq.status_string(code) != "unknown status"
    assert kvq.status_string(-77) == "unknown status"


def test_shape_validation(kvq):
    lib = kvq.library()
    cases = [
        (dict(bits=3), kvq.E_BITS), (dict(bits=8), kvq.E_BITS), (dict(head_dim=64), kvq.E_SHAPE),
        (dict(group=16), kvq.E_SHAPE), (dict(q_heads=3), kvq.E_SHAPE), (dict(residual_cap=100), kvq.E_SHAPE),
        (dict(residual_cap=0), kvq.E_SHAPE), (dict(max_tokens=1000), kvq.E_SHAPE), (dict(batch=0), kvq.E_SHAPE),
        # 2-bit caches take dense-and-sparse groups only; unknown bits and a missing rotary base are rejected
        (dict(flags=kvq.FLAG_SINK), kvq.E_SHAPE), (dict(flags=kvq.FLAG_PRE_ROPE, rope_base=10000.0), kvq.E_SHAPE),
        (dict(flags=kvq.FLAG_SPARSE | kvq.FLAG_SINK), kvq.E_SHAPE), (dict(flags=kvq.FLAG_SPARSE | 8), kvq.E_SHAPE),
        (dict(bits=4, flags=8), kvq.E_SHAPE), (dict(bits=4, flags=kvq.FLAG_SPARSE | 16), kvq.E_SHAPE),
        (dict(bits=4, flags=kvq.FLAG_PRE_ROPE, rope_base=0.0), kvq.E_SHAPE),
        (dict(bits=4, flags=kvq.FLAG_PRE_ROPE, rope_base=1.0), kvq.E_SHAPE),
        (dict(bits=4, flags=kvq.FLAG_PRE_ROPE, rope_base=float("nan")), kvq.E_SHAPE),
    ]
    for kw, code in cases:
        s = _shape(kvq, **kw)
        assert lib.kv_quant_keys_per_channel(ctypes.byref(s), FAKE, 0, 0, 128, 32, 0, FAKE, None) == code, kw
        c = _cache(kvq)
        assert lib.kv_append_and_flush(ctypes.byref(s), ctypes.byref(c), FAKE, FAKE, 0, 0, 128, 1, None) == code
        assert lib.kv_decode_attention(ctypes.byref(s), ctypes.byref(c), FAKE, 0.0, FAKE, FAKE, 1 << 30,
                                       None) == code
    assert lib.kv_quant_keys_per_channel(None, FAKE, 0, 0, 128, 32, 0, FAKE, None) == kvq.E_NULL


def test_quant_argument_validation(kvq):
    lib = kvq.library()
    s = _shape(kvq)
    q = lambda *a: lib.kv_quant_keys_per_channel(ctypes.byref(s), *a, None)
    v = lambda *a: lib.kv_quant_values_per_token(ctypes.byref(s), *a, None)
    for fn in (q, v):
        assert fn(None, 0, 0, 128, 32, 0, FAKE) == kvq.E_NULL
        assert fn(FAKE, 0, 0, 128, 32, 0, None) == kvq.E_NULL
        assert fn(FAKE + 2, 0, 0, 128, 32, 0, FAKE) == kvq.E_ALIGN
        assert fn(FAKE, 0, 0, 100, 32, 0, FAKE) == kvq.E_ALIGN
        assert fn(FAKE, 0, 0, 128, 32, 0, FAKE + 8) == kvq.E_ALIGN
        assert fn(FAKE, 0, 0, 128, 31, 0, FAKE) == kvq.E_SHAPE
        assert fn(FAKE, 0, 0, 128, 0, 0, FAKE) == kvq.E_SHAPE
        assert fn(FAKE, 0, 0, 128, 32, -1, FAKE) == kvq.E_SHAPE
        assert fn(FAKE, 0, 0, 128, 1024, 1, FAKE) == kvq.E_CAPACITY     # tiles 1..32 of 32
        assert fn(FAKE, 0, 0, 128, 64, 31, FAKE) == kvq.E_CAPACITY


def test_append_validation_and_capacity(kvq):
    lib = kvq.library()
    s = _shape(kvq)
    ap = lambda c, *a: lib.kv_append_and_flush(ctypes.byref(s), ctypes.byref(c), *a, None)
    c = _cache(kvq, tiles=0)
    assert ap(c, FAKE, FAKE, 0, 0, 128, 1) == kvq.E_NULL
    c = _cache(kvq)
    assert ap(c, None, FAKE, 0, 0, 128, 1) == kvq.E_NULL
    assert ap(c, FAKE, FAKE, 0, 0, 128, 0) == kvq.E_SHAPE
    assert ap(c, FAKE, FAKE + 4, 0, 0, 128, 1) == kvq.E_ALIGN
    for nq, nr in [(16, 0), (-32, 0), (1056, 0), (0, 129), (0, -1)]:
        c = _cache(kvq, nq, nr)
        assert ap(c, FAKE, FAKE, 0, 0, 128, 1) == kvq.E_STATE, (nq, nr)
    # 1024 quantized tokens of capacity: 1024 + 128 appended tokens flush 1024 -> fits; one more token does not
    c = _cache(kvq, 1024, 128)
    assert ap(c, FAKE, FAKE, 0, 0, 128, 1) == kvq.E_CAPACITY
    c = _cache(kvq, 0, 0)
    assert ap(c, FAKE, FAKE, 0, 0, 128, 1024 + 129) == kvq.E_CAPACITY
    assert (c.n_quant, c.n_resid) == (0, 0)          # nothing modified on error


def test_decode_validation(kvq):
    lib = kvq.library()
    s = _shape(kvq)
    dec = lambda c, q, out, ws, nbytes: lib.kv_decode_attention(ctypes.byref(s), ctypes.byref(c), q, 0.0, out, ws,
                                                                nbytes, None)
    empty = _cache(kvq)
    assert dec(empty, FAKE, FAKE, FAKE, 1 << 30) == kvq.E_EMPTY
    c = _cache(kvq, 512, 5)
    assert dec(c, None, FAKE, FAKE, 1 << 30) == kvq.E_NULL
    assert dec(c, FAKE + 2, FAKE, FAKE, 1 << 30) == kvq.E_ALIGN
    need = lib.kv_decode_attention_workspace_bytes(ctypes.byref(s), ctypes.byref(c))
    S = lib.kv_decode_attention_splits(ctypes.byref(s), ctypes.byref(c))
    assert need == 2 * 4 * S * 130 * 4 and S >= 1
    assert dec(c, FAKE, FAKE, FAKE, need - 1) == kvq.E_WORKSPACE
    assert dec(c, FAKE, FAKE, None, need) == kvq.E_WORKSPACE
    assert lib.kv_decode_attention_splits(ctypes.byref(s), ctypes.byref(empty)) == 0
    assert lib.kv_decode_attention_workspace_bytes(ctypes.byref(s), ctypes.byref(empty)) == 0


@pytest.mark.parametrize("B,Hq,Hkv,n_q,n_r,min_splits", [
    (64, 32, 8, 32640, 128, 6), (1, 32, 32, 1048448, 128, 64), (8, 32, 32, 3968, 128, 8), (1, 1, 1, 896, 128, 1)])
def test_split_plan_covers_every_tile(kvq, B, Hq, Hkv, n_q, n_r, min_splits):
    lib = kvq.library()
    s = _shape(kvq, batch=B, q_heads=Hq, kv_heads=Hkv, max_tokens=n_q + 1024)
    c = _cache(kvq, n_q, n_r)
    S = lib.kv_decode_attention_splits(ctypes.byref(s), ctypes.byref(c))
    n_vt = n_q // 32 + (n_r + 31) // 32
    assert min_splits <= S <= n_vt
    tps = -(-n_vt // S)
    assert (S - 1) * tps < n_vt <= S * tps       # no empty split, every tile covered


def test_sink_cache_validation(kvq):
    """The sink record is required with FLAG_SINK; n_sink is 0/1, only with the flag, and 1 before any other token."""
    lib = kvq.library()
    s = _shape(kvq, bits=4, flags=kvq.FLAG_SINK | kvq.FLAG_PRE_ROPE, rope_base=10000.0)
    ap = lambda c, n=1: lib.kv_append_and_flush(ctypes.byref(s), ctypes.byref(c), FAKE, FAKE, 0, 0, 128, n, None)
    assert ap(_cache(kvq)) == kvq.E_NULL                                    # no sink buffer
    assert ap(_cache(kvq, sink=FAKE + 8)) == kvq.E_ALIGN
    assert ap(_cache(kvq, n_sink=2, sink=FAKE + 16384)) == kvq.E_STATE
    assert ap(_cache(kvq, 32, 1, n_sink=0, sink=FAKE + 16384)) == kvq.E_STATE   # tokens but no sink yet
    plain = _shape(kvq, bits=4)
    c = _cache(kvq, 0, 1, n_sink=1)
    assert lib.kv_append_and_flush(ctypes.byref(plain), ctypes.byref(c), FAKE, FAKE, 0, 0, 128, 1,
                                   None) == kvq.E_STATE                     # n_sink without the flag
    # capacity: the first token of an empty sink cache goes to the sink, the other 1024 + 128 fit exactly
    c = _cache(kvq, sink=FAKE + 16384)
    assert ap(c, 1024 + 130) == kvq.E_CAPACITY
    assert (c.n_quant, c.n_resid, c.n_sink) == (0, 0, 0)


def test_sink_only_cache_has_one_split(kvq):
    lib = kvq.library()
    s = _shape(kvq, bits=4, flags=kvq.FLAG_SINK)
    c = _cache(kvq, n_sink=1, sink=FAKE + 16384)
    assert lib.kv_decode_attention_splits(ctypes.byref(s), ctypes.byref(c)) == 1
    assert lib.kv_decode_attention_workspace_bytes(ctypes.byref(s), ctypes.byref(c)) == 2 * 4 * 130 * 4
    empty = _cache(kvq, sink=FAKE + 16384)
    assert lib.kv_decode_attention_splits(ctypes.byref(s), ctypes.byref(empty)) == 0
    assert lib.kv_decode_attention(ctypes.byref(s), ctypes.byref(empty), FAKE, 0.0, FAKE, FAKE, 1 << 30,
                                   None) == kvq.E_EMPTY


def test_four_bit_splits_cover_every_query_head(kvq):
    """4-bit work units are (batch row, query head): the split count follows B * Hq, not B * Hkv."""
    lib = kvq.library()
    s = _shape(kvq, bits=4, batch=16, kv_heads=32, q_heads=32, max_tokens=16384)
    c = _cache(kvq, 16256, 127)
    S = lib.kv_decode_attention_splits(ctypes.byref(s), ctypes.byref(c))
    n_vt = 16256 // 32 + 4
    tps = -(-n_vt // S)
    assert S >= 1 and -(-n_vt // tps) == S and 16 * 32 * S <= 4096


def _ragged(kvq, tiles=FAKE, k_res=FAKE + 4096, v_res=FAKE + 8192, lens=FAKE + 12288, sync=None):
    return kvq.KvqRagged(tiles, k_res, v_res, None, lens, sync)


def test_ragged_validation(kvq):
    """Ragged calls reject bad arguments before launching: 2-bit without flags only, device lengths required and
    16-byte aligned, b inside the batch, flushed prefill tokens within max_tokens, a large enough workspace."""
    lib = kvq.library()
    s = _shape(kvq)
    r = _ragged(kvq)
    pre = lambda sh, c, b, n: lib.kv_ragged_prefill(ctypes.byref(sh), ctypes.byref(c), b, FAKE, FAKE, 0, 128, n, None)
    assert pre(_shape(kvq, bits=4), r, 0, 1) == kvq.E_BITS
    assert pre(s, _ragged(kvq, lens=0), 0, 1) == kvq.E_NULL
    assert pre(s, _ragged(kvq, lens=FAKE + 12292), 0, 1) == kvq.E_ALIGN
    assert pre(s, r, 2, 1) == kvq.E_SHAPE and pre(s, r, -1, 1) == kvq.E_SHAPE and pre(s, r, 0, -1) == kvq.E_SHAPE
    assert pre(s, r, 0, 1024 + 129) == kvq.E_CAPACITY          # 1152 tokens would be flushed, 1024 fit
    assert lib.kv_ragged_prefill(ctypes.byref(s), ctypes.byref(r), 0, None, FAKE, 0, 128, 5, None) == kvq.E_NULL
    ap = lambda c, kn: lib.kv_ragged_append(ctypes.byref(s), ctypes.byref(c), kn, FAKE, 256, 128, None)
    assert ap(r, None) == kvq.E_NULL and ap(r, FAKE + 2) == kvq.E_ALIGN
    S = lib.kv_ragged_splits(ctypes.byref(s))
    need = lib.kv_ragged_workspace_bytes(ctypes.byref(s))
    assert S >= 1 and need == 2 * 4 * S * 130 * 4
    dec = lambda ws, nbytes: lib.kv_ragged_decode_attention(ctypes.byref(s), ctypes.byref(r), FAKE, 0.0, FAKE, ws,
                                                            nbytes, None)
    assert dec(FAKE, need - 1) == kvq.E_WORKSPACE and dec(None, need) == kvq.E_WORKSPACE
    step = lambda c, nbytes: lib.kv_ragged_decode_step(ctypes.byref(s), ctypes.byref(c), FAKE, FAKE, 256, 128, FAKE,
                                                       0.0, FAKE, FAKE, nbytes, None)
    rs = _ragged(kvq, sync=FAKE + 16384)
    assert step(rs, need - 1) == kvq.E_WORKSPACE
    assert step(r, need) == kvq.E_NULL                       # the single-launch step needs its counters
    assert step(_ragged(kvq, sync=FAKE + 16386), need) == kvq.E_ALIGN
    assert lib.kv_ragged_splits(ctypes.byref(_shape(kvq, bits=4))) == 0
    # counters: one per sequence plus one per (sequence, KV head, chunk of four query heads)
    lib.kv_ragged_sync_words.restype = ctypes.c_size_t
    assert lib.kv_ragged_sync_words(ctypes.byref(_shape(kvq, batch=3, kv_heads=2, q_heads=4))) == 3 * (1 + 2)
    assert lib.kv_ragged_sync_words(ctypes.byref(_shape(kvq, batch=3, kv_heads=2, q_heads=20))) == 3 * (1 + 2 * 3)
    assert lib.kv_ragged_sync_words(ctypes.byref(_shape(kvq, bits=4))) == 0


def test_ragged_splits_follow_capacity(kvq):
    """The ragged split count is the uniform plan of a full cache (max_tokens quantized + R window), whatever the
    lengths: one workspace and one captured step serve every length."""
    lib = kvq.library()
    s = _shape(kvq, batch=3, kv_heads=2, q_heads=8, max_tokens=1024)
    full = _cache(kvq, 1024, 128)
    assert lib.kv_ragged_splits(ctypes.byref(s)) == lib.kv_decode_attention_splits(ctypes.byref(s), ctypes.byref(full))


def test_read_probe_rejects_bad_arguments_before_launching():
    """The benchmark's streaming-read probe (a separate library) validates on the host: nothing is launched here."""
    import os
    import decode_attention_quant_amd as pkg
    path = os.path.join(os.path.dirname(pkg.__file__), "libkvq_probe.so")
    if not os.path.exists(path):
        pytest.skip("probe library not built")
    lib = ctypes.CDLL(path)
    lib.kvq_probe_sink_words.restype = ctypes.c_size_t
    lib.kvq_probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_void_p]
    n = lib.kvq_probe_sink_words()
    assert n > 0
    assert lib.kvq_probe_hbm_read(None, 1 << 20, FAKE, n, None) == -1
    assert lib.kvq_probe_hbm_read(FAKE, 1 << 20, None, n, None) == -1
    assert lib.kvq_probe_hbm_read(FAKE, 1000, FAKE, n, None) == -1          # not a multiple of 16
    assert lib.kvq_probe_hbm_read(FAKE + 8, 1 << 20, FAKE, n, None) == -1   # misaligned
    assert lib.kvq_probe_hbm_read(FAKE, 1 << 20, FAKE, n - 1, None) == -1   # sink too small


def test_noalloc_decode_rejects_partials_beyond_its_scratch(kvq):
    """kv_decode_attention_noalloc checks on the host, before any runtime call, that the split partials fit its
    static scratch: 2048 sequences x 32 query heads (one split each) need 34 MB, more than 16 MiB."""
    lib = kvq.library()
    shape = _shape(kvq, batch=2048, kv_heads=8, q_heads=32, max_tokens=1 << 20)
    cache = _cache(kvq, n_quant=1 << 20, n_resid=5)
    need = lib.kv_decode_attention_workspace_bytes(ctypes.byref(shape), ctypes.byref(cache))
    assert need > kvq.NOALLOC_SCRATCH_BYTES
    rc = lib.kv_decode_attention_noalloc(ctypes.byref(shape), ctypes.byref(cache), ctypes.c_void_p(FAKE), 0.0,
                                         ctypes.c_void_p(FAKE + 16), None)
    assert rc == kvq.E_SCRATCH
    # the usual argument checks come first
    assert lib.kv_decode_attention_noalloc(ctypes.byref(shape), ctypes.byref(cache), None, 0.0,
                                           ctypes.c_void_p(FAKE + 16), None) == kvq.E_NULL
    empty = _cache(kvq)
    assert lib.kv_decode_attention_noalloc(ctypes.byref(shape), ctypes.byref(empty), ctypes.c_void_p(FAKE), 0.0,
                                           ctypes.c_void_p(FAKE + 16), None) == kvq.E_EMPTY


def test_two_bit_sparse_shape_is_accepted_on_the_host(kvq):
    """2-bit dense-and-sparse caches pass the host checks (split plan and workspace computed, no launch), take
    3840-byte records, and are refused by the ragged calls."""
    lib = kvq.library()
    s = _shape(kvq, flags=kvq.FLAG_SPARSE)
    c = _cache(kvq)
    c.n_quant, c.n_resid = 512, 17
    assert lib.kv_decode_attention_splits(ctypes.byref(s), ctypes.byref(c)) > 0
    assert lib.kv_decode_attention_workspace_bytes(ctypes.byref(s), ctypes.byref(c)) > 0
    assert kvq.Shape(2, 2, 8, max_tokens=1024, flags=kvq.FLAG_SPARSE).record_bytes == kvq.RECORD_BYTES_SPARSE == 3840
    assert lib.kv_ragged_splits(ctypes.byref(s)) == 0
