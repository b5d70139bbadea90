"""GPU parity of ragged caches: sequences at their own lengths, the lengths in device memory.

Each sequence is checked against its own oracle cache (the oracle's state machine and attention applied to that
sequence alone): packed tiles, the records of complete window blocks written ahead after them, and window bytes
bit-exact, attention outputs within max-abs 2e-3. The decode step is a
single launch (flush, append, attention, merge and length commit inside one kernel); it must equal
kv_ragged_append + kv_ragged_decode_attention bit for bit, leave its completion counters at zero, and, captured once
in a HIP graph and replayed with new inputs, equal the same step run eagerly on a twin cache, bit for bit.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

from oracle import attention as oa  # noqa: E402
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


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _keys(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    x[..., [5, 33, 90, 127]] *= 20
    return x.astype(np.float16)


def _setup(kvq, rng, lengths, Hkv, Hq, max_tokens, steps=0):
    """Ragged cache prefilled to `lengths`, its per-sequence oracle caches, and the tokens/queries of `steps`
    decode steps."""
    B = len(lengths)
    cache = kvq.RaggedCache(kvq.Shape(B, Hkv, Hq, max_tokens=max_tokens))
    refs = []
    for b, n in enumerate(lengths):
        k = _keys(rng, (Hkv, n, 128))
        v = rng.standard_normal((Hkv, n, 128)).astype(np.float16)
        kvq.kv_ragged_prefill(cache, b, _dev(k), _dev(v))
        ref = oc.SliceCache(Hkv)
        if n:
            oc.append_block(ref, k, v)
        refs.append(ref)
    ks = _keys(rng, (steps, B, Hkv, 128))
    vs = rng.standard_normal((steps, B, Hkv, 128)).astype(np.float16)
    qs = rng.standard_normal((max(steps, 1), B, Hq, 128)).astype(np.float16)
    return cache, refs, ks, vs, qs


def _check_state(cache, refs, what):
    lens = cache.lengths()
    for b, ref in enumerate(refs):
        assert lens[b][:2] == [ref.n_quant, ref.n_resid], f"{what}: seq {b} lens {lens[b]}"
        nt = ref.n_quant // 32
        if nt:
            got = cache.tiles[b, :, :nt].cpu().numpy()
            want = helpers.oracle_records(ref)
            assert np.array_equal(got, want), f"{what}: seq {b}: " + helpers.first_mismatch(got, want)
        nr = ref.n_resid
        # complete window blocks: their records are written ahead, in the tiles after the quantized part
        for k in range(nr // 32):
            slot = nt + k
            if slot >= cache.tiles.shape[2]:
                break
            blk = oc.SliceCache(ref.slices, residual_cap=32)
            oc.append_block(blk, ref.k_res[:, 32 * k:32 * k + 32], ref.v_res[:, 32 * k:32 * k + 32])
            blk.flush()
            got = cache.tiles[b, :, slot:slot + 1].cpu().numpy()
            want = helpers.oracle_records(blk)
            assert np.array_equal(got, want), (f"{what}: seq {b}: window block {k} (tile {slot}) not written ahead: "
                                               + helpers.first_mismatch(got, want))
        kr = cache.k_res[b, :, :nr].cpu().numpy()
        vr = cache.v_res[b, :, :nr].cpu().numpy()
        assert np.array_equal(kr.view(np.uint16), ref.k_res.view(np.uint16)), f"{what}: seq {b} k window"
        assert np.array_equal(vr.view(np.uint16), ref.v_res.view(np.uint16)), f"{what}: seq {b} v window"


def _oracle_out(refs, q, Hkv):
    outs = []
    for b, ref in enumerate(refs):
        if ref.n_tokens == 0:
            outs.append(np.zeros(q.shape[1:]))
        else:
            outs.append(oa.decode_attention(ref, q[b:b + 1], 1, Hkv)[0])
    return np.stack(outs)


@pytest.mark.parametrize("lengths,Hq,Hkv", [([300, 1, 777, 128, 129], 8, 2), ([1000, 33], 4, 4),
                                            ([2, 1500, 640, 5], 16, 2)])
def test_ragged_prefill_and_attention(kvq, lengths, Hq, Hkv):
    say(f"[ragged] lengths={lengths} Hq={Hq} Hkv={Hkv}")
    rng = np.random.default_rng(sum(lengths) + Hq)
    cache, refs, _, _, qs = _setup(kvq, rng, lengths, Hkv, Hq, 1536)
    torch.cuda.synchronize()
    _check_state(cache, refs, "prefill")
    out = kvq.kv_ragged_decode_attention(cache, _dev(qs[0]))
    torch.cuda.synchronize()
    err = np.abs(out.cpu().numpy().astype(np.float64) - _oracle_out(refs, qs[0], Hkv))
    say(f"    splits={kvq.kv_ragged_splits(cache)} max_abs={err.max():.3e}")
    assert err.max() <= ATOL


def test_ragged_decode_steps_cross_flushes_at_different_steps(kvq):
    """130 decode steps: the three sequences flush at steps 85, 120 and 128; after every step each sequence's
    output matches its oracle, and the state is bit-exact after each flush and at the end."""
    rng = np.random.default_rng(99)
    lengths, Hq, Hkv = [300, 1, 777], 8, 2
    steps = 130
    cache, refs, ks, vs, qs = _setup(kvq, rng, lengths, Hkv, Hq, 1024, steps)
    ws = torch.empty(kvq.kv_ragged_workspace_bytes(cache), dtype=torch.uint8, device="cuda")
    worst = 0.0
    for i in range(steps):
        flushed = [ref.n_resid == ref.residual_cap for ref in refs]
        out = kvq.kv_ragged_decode_step(cache, _dev(ks[i]), _dev(vs[i]), _dev(qs[i]), workspace=ws)
        assert not cache.sync.any(), f"step {i}: completion counters not reset"
        for b, ref in enumerate(refs):
            ref.append_token(ks[i, b], vs[i, b])
        got = out.cpu().numpy().astype(np.float64)
        err = np.abs(got - _oracle_out(refs, qs[i], Hkv)).max()
        worst = max(worst, err)
        assert err <= ATOL, f"step {i}: {err}"
        if any(flushed):
            say(f"    step {i}: flush in sequences {[b for b, f in enumerate(flushed) if f]}")
            _check_state(cache, refs, f"step {i}")
    _check_state(cache, refs, "end")
    say(f"    worst max_abs={worst:.3e}")


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (16, 2), (6, 3)])
def test_ragged_append_then_attention_equals_step(kvq, Hq, Hkv):
    """kv_ragged_append followed by kv_ragged_decode_attention gives the same bytes as the single-launch
    kv_ragged_decode_step, across flushes; with 16 query heads on 2 KV heads two query-head chunks of each KV head
    quantize the flushed window in the same launch."""
    rng = np.random.default_rng(7)
    lengths = [127, 128, 255, 3]
    a, _, ks, vs, qs = _setup(kvq, np.random.default_rng(7), lengths, Hkv, Hq, 1024, 4)
    b, _, _, _, _ = _setup(kvq, np.random.default_rng(7), lengths, Hkv, Hq, 1024, 4)
    say(f"[ragged-step==append+attention] Hq={Hq} Hkv={Hkv} splits={kvq.kv_ragged_splits(a)}")
    for i in range(4):
        oa_ = kvq.kv_ragged_decode_step(a, _dev(ks[i]), _dev(vs[i]), _dev(qs[i]))
        kvq.kv_ragged_append(b, _dev(ks[i]), _dev(vs[i]))
        ob = kvq.kv_ragged_decode_attention(b, _dev(qs[i]))
        torch.cuda.synchronize()
        assert torch.equal(oa_, ob)
        assert torch.equal(a.lens, b.lens) and torch.equal(a.tiles, b.tiles) and torch.equal(a.k_res, b.k_res)
        assert torch.equal(a.v_res, b.v_res) and not a.sync.any()
    del rng


def test_ragged_step_graph_replay(kvq):
    """One decode step captured in a HIP graph (fixed input buffers) and replayed 140 times with new inputs copied in
    between replays: every replay equals an eager twin bit for bit (lengths, bytes, outputs) and the oracle."""
    lengths, Hq, Hkv = [300, 1, 777], 8, 2
    steps = 140
    g_cache, refs, ks, vs, qs = _setup(kvq, np.random.default_rng(5), lengths, Hkv, Hq, 1024, steps)
    e_cache, _, _, _, _ = _setup(kvq, np.random.default_rng(5), lengths, Hkv, Hq, 1024, steps)
    kbuf = torch.zeros((len(lengths), Hkv, 128), dtype=torch.float16, device="cuda")
    vbuf, qbuf = torch.zeros_like(kbuf), torch.zeros((len(lengths), Hq, 128), dtype=torch.float16, device="cuda")
    obuf = torch.zeros((len(lengths), Hq, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(kvq.kv_ragged_workspace_bytes(g_cache), dtype=torch.uint8, device="cuda")
    ws_e = torch.empty_like(ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kvq.kv_ragged_decode_step(g_cache, kbuf, vbuf, qbuf, out=obuf, workspace=ws)
    torch.cuda.synchronize()
    assert g_cache.lengths() == e_cache.lengths(), "capture must not run the step"
    worst = 0.0
    for i in range(steps):
        kbuf.copy_(_dev(ks[i]))
        vbuf.copy_(_dev(vs[i]))
        qbuf.copy_(_dev(qs[i]))
        graph.replay()
        oe = kvq.kv_ragged_decode_step(e_cache, _dev(ks[i]), _dev(vs[i]), _dev(qs[i]), workspace=ws_e)
        torch.cuda.synchronize()
        assert torch.equal(obuf, oe), f"replay {i} differs from the eager step"
        assert torch.equal(g_cache.lens, e_cache.lens), f"replay {i}: lengths"
        for b, ref in enumerate(refs):
            ref.append_token(ks[i, b], vs[i, b])
        if i % 10 == 9 or i == steps - 1:
            err = np.abs(obuf.cpu().numpy().astype(np.float64) - _oracle_out(refs, qs[i], Hkv)).max()
            worst = max(worst, err)
            assert err <= ATOL
    assert torch.equal(g_cache.tiles, e_cache.tiles) and torch.equal(g_cache.v_res, e_cache.v_res)
    _check_state(g_cache, refs, "after replays")
    say(f"    {steps} replays, worst max_abs vs oracle={worst:.3e}")


def test_ragged_step_gqa8_crosses_flushes(kvq):
    """Single-launch steps with two query-head chunks per KV head (G = 8) across every sequence's flush: outputs
    within 2e-3 of the oracle after each step and the state bit-exact after each flush."""
    rng = np.random.default_rng(808)
    lengths, Hq, Hkv = [128, 90, 250], 16, 2
    steps = 40
    cache, refs, ks, vs, qs = _setup(kvq, rng, lengths, Hkv, Hq, 512, steps)
    for i in range(steps):
        flushed = [ref.n_resid == ref.residual_cap for ref in refs]
        out = kvq.kv_ragged_decode_step(cache, _dev(ks[i]), _dev(vs[i]), _dev(qs[i]))
        for b, ref in enumerate(refs):
            ref.append_token(ks[i, b], vs[i, b])
        err = np.abs(out.cpu().numpy().astype(np.float64) - _oracle_out(refs, qs[i], Hkv)).max()
        assert err <= ATOL, f"step {i}: {err}"
        if any(flushed):
            _check_state(cache, refs, f"step {i}")
    assert not cache.sync.any()


def test_ragged_full_sequence_is_refused(kvq):
    """A sequence whose flush would pass max_tokens gets status 1 and keeps its lengths (appends refused); the
    others go on; its output stays attention over what it holds."""
    rng = np.random.default_rng(3)
    Hq, Hkv = 4, 2
    # capacity 256 quantized tokens: sequence 0 holds 256 + 128 (full window) and cannot flush again
    cache, refs, ks, vs, qs = _setup(kvq, rng, [384, 10], Hkv, Hq, 256, 3)
    assert cache.lengths()[0][:2] == [256, 128]
    for i in range(3):
        out = kvq.kv_ragged_decode_step(cache, _dev(ks[i]), _dev(vs[i]), _dev(qs[i]))
        refs[1].append_token(ks[i, 1], vs[i, 1])
        lens = cache.lengths()
        assert lens[0] == [256, 128, 0, 1] and lens[1][:2] == [refs[1].n_quant, refs[1].n_resid]
        err = np.abs(out.cpu().numpy().astype(np.float64) - _oracle_out(refs, qs[i], Hkv)).max()
        assert err <= ATOL
    kvq.kv_ragged_prefill(cache, 0, _dev(np.zeros((Hkv, 5, 128), np.float16)),
                          _dev(np.zeros((Hkv, 5, 128), np.float16)))
    assert cache.lengths()[0] == [0, 5, 0, 0]


def test_ragged_empty_sequence_gives_zeros(kvq):
    rng = np.random.default_rng(4)
    cache, refs, _, _, qs = _setup(kvq, rng, [0, 50, 0], 2, 4, 256)
    out = kvq.kv_ragged_decode_attention(cache, _dev(qs[0])).cpu().numpy()
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert np.abs(out[1] - _oracle_out(refs, qs[0], 2)[1]).max() <= ATOL


def test_ragged_step_random_lengths_and_capacity(kvq):
    """200 single-launch steps over seven sequences of seeded random lengths (some empty) in a cache whose capacity
    makes some of them full along the way: each step equals kv_ragged_append + kv_ragged_decode_attention on a twin
    cache bit for bit (outputs, lengths, tiles, window), the counters return to zero, and at the end every sequence
    matches its oracle cache."""
    rng = np.random.default_rng(2027)
    lengths = [int(x) for x in rng.integers(0, 600, 7)]
    lengths[3] = 0
    lengths[0] = 630     # fills the capacity of 640 quantized tokens at its second flush
    Hq, Hkv, steps, cap = 12, 4, 200, 640
    a, refs, ks, vs, qs = _setup(kvq, np.random.default_rng(11), lengths, Hkv, Hq, cap, steps)
    b, _, _, _, _ = _setup(kvq, np.random.default_rng(11), lengths, Hkv, Hq, cap, steps)
    say(f"[ragged-step-fuzz] lengths={lengths} splits={kvq.kv_ragged_splits(a)}")
    full_seen = set()
    for i in range(steps):
        oa_ = kvq.kv_ragged_decode_step(a, _dev(ks[i]), _dev(vs[i]), _dev(qs[i]))
        kvq.kv_ragged_append(b, _dev(ks[i]), _dev(vs[i]))
        ob = kvq.kv_ragged_decode_attention(b, _dev(qs[i]))
        torch.cuda.synchronize()
        assert torch.equal(oa_, ob), f"step {i}: outputs differ"
        assert torch.equal(a.lens, b.lens), f"step {i}: lengths differ"
        assert not a.sync.any(), f"step {i}: counters not reset"
        for s, row in enumerate(a.lengths()):
            if row[3]:
                full_seen.add(s)
            else:
                refs[s].append_token(ks[i, s], vs[i, s])
    assert torch.equal(a.tiles, b.tiles) and torch.equal(a.k_res, b.k_res) and torch.equal(a.v_res, b.v_res)
    say(f"    sequences marked full: {sorted(full_seen)}")
    assert full_seen, "the capacity should fill some sequence"
    for s, row in enumerate(a.lengths()):
        assert row[:2] == [refs[s].n_quant, refs[s].n_resid], f"seq {s}: {row} vs oracle"
    err = np.abs(oa_.cpu().numpy().astype(np.float64) - _oracle_out(refs, qs[steps - 1], Hkv)).max()
    say(f"    last step max_abs vs oracle={err:.3e}")
    assert err <= ATOL
