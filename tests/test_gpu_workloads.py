"""GPU parity on the synthetic workloads at their full sizes, in the launch configuration the benchmark times.

- tiny_1k (B1, one head, 1024 tokens): everything compared (every tile bit-exact, window bytes, output);
- llama2_7b_stream (B8, 32 heads, 4096-token prefill + 256 decode steps): every step appends one token and
  attends; the state is compared bit for bit with the oracle's token-by-token state machine after both flushes
  (steps 1 and 129) and at the end, on every slice; outputs of sampled heads are compared at every step and all
  outputs at sampled steps;
- llama3_8b_gqa_32k (B64, 32 query / 8 KV heads, 32768 tokens): tiles of eight sampled slices (one per KV head)
  bit-exact, outputs of the query heads of those slices within 2e-3, all outputs finite and inside the range of their slice's values;
- long_1m (B1, 32 heads, 1,048,576 tokens): sampled tiles bit-exact, outputs of sampled heads within 2e-3;
- llama2_7b_stream at the benchmark's mixed lengths (sequence b prefilled with 4096 (b + 1) / 8 tokens) through the
  single-launch ragged step: sampled outputs at every step, then lengths, tiles and window rows exact.
The oracle side of the long cases runs on a thread pool over independent token blocks; it only calls oracle
functions.
"""
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import kvsynth  # noqa: E402
from kvsynth import device as kdev  # noqa: E402
from oracle import attention as oa  # noqa: E402
from oracle import cache as oc  # noqa: E402
from oracle import quant  # noqa: E402
from tests import helpers  # noqa: E402

ATOL = 2e-3
THREADS = min(16, len(os.sched_getaffinity(0)))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def kvq():
    import decode_attention_quant_amd as m
    return m


def _oracle_slices(w, slices, n_tokens):
    """Oracle cache of the given (b, h) slices holding tokens [0, n_tokens) built by one block append, with the
    per-block quantization spread over threads (blocks are whole flush windows, so the state is the same)."""
    k = np.stack([helpers.workload_tokens(w, kvsynth.K_ID, 0, n_tokens, b, h) for b, h in slices])
    v = np.stack([helpers.workload_tokens(w, kvsynth.V_ID, 0, n_tokens, b, h) for b, h in slices])
    c = oc.SliceCache(len(slices), residual_cap=w.residual)
    f = oc.flushed_tokens(0, n_tokens, w.residual)
    R = w.residual
    block = R * max(1, min(64, f // R // (2 * THREADS)))
    bounds = [(a, min(f, a + block)) for a in range(0, f, block)]

    def q(ab):
        a, b = ab
        return (quant.quantize_keys_per_channel(k[:, a:b]), quant.quantize_values_per_token(v[:, a:b]))

    with ThreadPoolExecutor(THREADS) as ex:
        parts = list(ex.map(q, bounds))
    for (kq, ks, kz), (vq, vs, vz) in parts:
        c._kq.append(kq); c._ks.append(ks); c._kz.append(kz)
        c._vq.append(vq); c._vs.append(vs); c._vz.append(vz)
    c.n_quant = f
    c.k_res, c.v_res = k[:, f:], v[:, f:]
    return c


def _oracle_attention_threads(c, q_slices, block=65536):
    """decode attention of one query block per slice ([S, G, D] float16) via split partials over token blocks."""
    S, G, D = q_slices.shape
    N = c.n_tokens
    bounds = [(a, min(N, a + block)) for a in range(0, N, block)]
    qq = q_slices.reshape(S, G, D)[None].reshape(S, G, D)

    def part(ab):
        # batch = S slices with one KV head each
        return oa.split_partials(c, qq.reshape(S, G, D), S, 1, [ab])

    with ThreadPoolExecutor(THREADS) as ex:
        res = list(ex.map(part, bounds))
    m = np.concatenate([r[0] for r in res]); l = np.concatenate([r[1] for r in res])
    o = np.concatenate([r[2] for r in res])
    return oa.merge_partials(m, l, o).reshape(S, G, D)


def _oracle_attention_all(ref, q, batch, kv_heads):
    """oracle decode attention of every slice, slices spread over threads"""
    G = q.shape[1] // kv_heads
    S = batch * kv_heads
    qs = q.reshape(S, G, q.shape[-1])
    groups = np.array_split(np.arange(S), THREADS)

    def one(idx):
        return [oa.decode_attention(_view(ref, i), qs[i:i + 1], 1, 1)[0] for i in idx]

    with ThreadPoolExecutor(THREADS) as ex:
        res = [o for part in ex.map(one, groups) for o in part]
    return np.stack(res).reshape(batch, kv_heads * G, q.shape[-1])


def _build_gpu(kvq, w):
    """Device K/V of the whole context (prefill and decode-step tokens) and a cache holding the prefill."""
    shape = kvq.Shape(w.batch, w.kv_heads, w.q_heads, residual_cap=w.residual,
                      max_tokens=((w.context + 31) // 32) * 32)
    cache = kvq.KVCache(shape)
    t = time.time()
    K = kdev.kv_to_device(w, kvsynth.K_ID, 0, w.context)
    V = kdev.kv_to_device(w, kvsynth.V_ID, 0, w.context)
    say(f"    generated + uploaded {w.context} tokens in {time.time() - t:.1f}s")
    kvq.kv_append_and_flush(cache, K[:, :, :w.prefill], V[:, :, :w.prefill])
    torch.cuda.synchronize()
    return cache, K, V


def _decode_step(kvq, w, cache, K, V, step):
    t = w.prefill + step - 1
    kvq.kv_append_and_flush(cache, K[:, :, t:t + 1], V[:, :, t:t + 1])
    q = kdev.queries_to_device(w, [step])[0]
    return kvq.kv_decode_attention(cache, q), q


def test_tiny_1k(kvq):
    w = kvsynth.WORKLOADS["tiny_1k"]
    say(f"[workload] {w.name}")
    cache, K, V = _build_gpu(kvq, w)
    out, q = _decode_step(kvq, w, cache, K, V, 1)
    torch.cuda.synchronize()
    ref = _oracle_slices(w, [(0, 0)], w.context)
    assert (cache.n_quant, cache.n_resid) == (ref.n_quant, ref.n_resid) == (896, 128)
    got = helpers.records_from_device(cache.tiles, 28)
    want = helpers.oracle_records(ref)
    assert np.array_equal(got, want), helpers.first_mismatch(got, want)
    assert np.array_equal(cache.k_res[0, 0].cpu().numpy().view(np.uint16), ref.k_res[0].view(np.uint16))
    want_o = oa.decode_attention(ref, q.cpu().numpy(), 1, 1)
    err = np.abs(out.cpu().numpy() - want_o).max()
    say(f"    max_abs={err:.3e}")
    assert err <= ATOL


def test_llama2_stream(kvq):
    w = kvsynth.WORKLOADS["llama2_7b_stream"]
    say(f"[workload] {w.name}: prefill {w.prefill} + {w.steps} steps")
    cache, K, V = _build_gpu(kvq, w)
    S = w.batch * w.kv_heads
    sampled = [(0, 0), (3, 17), (7, 31)]
    sidx = [b * w.kv_heads + h for b, h in sampled]
    ref = _oracle_slices(w, sampled, w.prefill)
    kt_all = np.stack([helpers.workload_tokens(w, kvsynth.K_ID, w.prefill, w.context, b, h) for b, h in sampled])
    vt_all = np.stack([helpers.workload_tokens(w, kvsynth.V_ID, w.prefill, w.context, b, h) for b, h in sampled])
    full_check_steps = {1, 2, 129, 256}
    worst = 0.0
    for step in range(1, w.steps + 1):
        flushed = ref.n_resid == w.residual
        out, q = _decode_step(kvq, w, cache, K, V, step)
        ref.append_token(kt_all[:, step - 1], vt_all[:, step - 1])
        qn = q.cpu().numpy()
        got = out.cpu().numpy()
        want = np.stack([oa.decode_attention(_view(ref, i), qn[b:b + 1, h:h + 1], 1, 1)[0, 0]
                         for i, (b, h) in enumerate(sampled)])
        err = np.abs(got[[b for b, _ in sampled], [h for _, h in sampled]] - want).max()
        worst = max(worst, err)
        assert err <= ATOL, (step, err)
        assert np.all(np.isfinite(got)), step
        if flushed or step in full_check_steps:
            say(f"    step {step}: flushed={flushed} n=({cache.n_quant},{cache.n_resid}) max_abs(sampled)={err:.3e}")
            assert (cache.n_quant, cache.n_resid) == (ref.n_quant, ref.n_resid)
            g = helpers.records_from_device(cache.tiles, ref.n_quant // 32, sidx)
            wnt = helpers.oracle_records(ref)
            assert np.array_equal(g, wnt), helpers.first_mismatch(g, wnt)
    # every slice at the end: all tiles bit-exact against an oracle built for every slice
    say("    final: every slice")
    allslices = [(b, h) for b in range(w.batch) for h in range(w.kv_heads)]
    full = _oracle_slices(w, allslices, w.context)
    g = helpers.records_from_device(cache.tiles, full.n_quant // 32)
    wnt = helpers.oracle_records(full)
    assert np.array_equal(g, wnt), helpers.first_mismatch(g, wnt)
    kr = cache.k_res.reshape(S, w.residual, 128)[:, :full.n_resid].cpu().numpy()
    assert np.array_equal(kr.view(np.uint16), full.k_res.view(np.uint16))
    qn = kdev.queries_to_device(w, [w.steps])[0].cpu().numpy()
    want = _oracle_attention_all(full, qn, w.batch, w.kv_heads)
    err = np.abs(out.cpu().numpy() - want).max()
    say(f"    final all-head max_abs={err:.3e} worst sampled={worst:.3e}")
    assert err <= ATOL


def test_llama2_stream_mixed_lengths_step(kvq):
    """The benchmark's mixed-length batch: sequence b of llama2_7b_stream prefilled with 4096 (b + 1) / 8 tokens, then
    136 single-launch decode steps (two flushes per sequence). Outputs of sampled slices against the oracle at every
    step; at the end the lengths of every sequence, and the tiles and window rows of the sampled slices, are exact."""
    w = kvsynth.WORKLOADS["llama2_7b_stream"]
    B, H, R, steps = w.batch, w.kv_heads, w.residual, 136
    lens0 = [max(32, (w.prefill * (b + 1)) // B) for b in range(B)]
    total = lens0[-1] + steps
    say(f"[workload] {w.name} at mixed lengths {lens0[0]}..{lens0[-1]}, {steps} steps")
    K = kdev.kv_to_device(w, kvsynth.K_ID, 0, total)
    V = kdev.kv_to_device(w, kvsynth.V_ID, 0, total)
    Q = kdev.queries_to_device(w, range(1, steps + 1))
    shape = kvq.Shape(B, H, w.q_heads, residual_cap=R, max_tokens=((total + 31) // 32) * 32)
    cache = kvq.RaggedCache(shape)
    for b in range(B):
        kvq.kv_ragged_prefill(cache, b, K[b, :, :lens0[b]], V[b, :, :lens0[b]])
    ws = torch.empty(kvq.kv_ragged_workspace_bytes(cache), dtype=torch.uint8, device="cuda")
    idx = torch.arange(B, device="cuda")
    sampled = [(0, 0), (3, 17), (7, 31)]
    refs = [_oracle_slices(w, [(b, h)], lens0[b]) for b, h in sampled]
    kt = [helpers.workload_tokens(w, kvsynth.K_ID, lens0[b], lens0[b] + steps, b, h) for b, h in sampled]
    vt = [helpers.workload_tokens(w, kvsynth.V_ID, lens0[b], lens0[b] + steps, b, h) for b, h in sampled]
    worst = 0.0
    for i in range(steps):
        pos = torch.tensor(lens0, device="cuda") + i
        k_new = K[idx, :, pos].contiguous()
        v_new = V[idx, :, pos].contiguous()
        out = kvq.kv_ragged_decode_step(cache, k_new, v_new, Q[i], workspace=ws)
        qn = Q[i].cpu().numpy()
        got = out.cpu().numpy()
        for j, (b, h) in enumerate(sampled):
            refs[j].append_token(kt[j][i:i + 1], vt[j][i:i + 1])
            want = oa.decode_attention(refs[j], qn[b:b + 1, h:h + 1], 1, 1)[0, 0]
            err = float(np.abs(got[b, h] - want).max())
            worst = max(worst, err)
            assert err <= ATOL, (i, b, h, err)
        assert np.all(np.isfinite(got)), i
    lens = cache.lens.cpu().numpy()
    for b in range(B):
        n_q = oc.flushed_tokens(0, lens0[b] + steps, R)
        assert tuple(lens[b]) == (n_q, lens0[b] + steps - n_q, 0, 0), (b, lens[b])
    for j, (b, h) in enumerate(sampled):
        r = refs[j]
        assert (int(lens[b][0]), int(lens[b][1])) == (r.n_quant, r.n_resid)
        g = helpers.records_from_device(cache.tiles, r.n_quant // 32, [b * H + h])
        wnt = helpers.oracle_records(r)
        assert np.array_equal(g, wnt), helpers.first_mismatch(g, wnt)
        kr = cache.k_res[b, h, :r.n_resid].cpu().numpy()
        vr = cache.v_res[b, h, :r.n_resid].cpu().numpy()
        assert np.array_equal(kr.view(np.uint16), r.k_res[0].view(np.uint16))
        assert np.array_equal(vr.view(np.uint16), r.v_res[0].view(np.uint16))
    say(f"    worst sampled max_abs={worst:.3e}; lengths {lens[:, :2].tolist()}")


def _view(c, i):
    """Single-slice view of an oracle cache (slice i)."""
    v = oc.SliceCache(1, residual_cap=c.residual_cap)
    kq, ks, kz, vq, vs, vz = c.quantized()
    v._kq, v._ks, v._kz = [kq[i:i + 1]], [ks[i:i + 1]], [kz[i:i + 1]]
    v._vq, v._vs, v._vz = [vq[i:i + 1]], [vs[i:i + 1]], [vz[i:i + 1]]
    v.n_quant = c.n_quant
    v.k_res, v.v_res = c.k_res[i:i + 1], c.v_res[i:i + 1]
    return v


def _sampled_full_size(kvq, w, sampled):
    say(f"[workload] {w.name}: B{w.batch} Hq{w.q_heads} Hkv{w.kv_heads} N{w.context}")
    cache, K, V = _build_gpu(kvq, w)
    out, q = _decode_step(kvq, w, cache, K, V, 1)
    torch.cuda.synchronize()
    del K, V
    say(f"    splits={kvq.kv_decode_attention_splits(cache)} n=({cache.n_quant},{cache.n_resid})")
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    t = time.time()
    ref = _oracle_slices(w, sampled, w.context)
    say(f"    oracle state of {len(sampled)} slices in {time.time() - t:.1f}s")
    assert (cache.n_quant, cache.n_resid) == (ref.n_quant, ref.n_resid)
    G = w.q_heads // w.kv_heads
    sidx = [b * w.kv_heads + h for b, h in sampled]
    g = helpers.records_from_device(cache.tiles, ref.n_quant // 32, sidx)
    wnt = helpers.oracle_records(ref)
    assert np.array_equal(g, wnt), helpers.first_mismatch(g, wnt)
    qn = q.cpu().numpy()
    qs = np.stack([qn[b, h * G:(h + 1) * G] for b, h in sampled])
    t = time.time()
    want = _oracle_attention_threads(ref, qs)
    say(f"    oracle attention in {time.time() - t:.1f}s")
    gs = np.stack([got[b, h * G:(h + 1) * G] for b, h in sampled])
    err = np.abs(gs - want)
    say(f"    sampled max_abs={err.max():.3e} p99.9={np.quantile(err, 0.999):.3e}")
    assert err.max() <= ATOL
    return cache, got


def test_llama3_gqa_32k_sampled(kvq):
    w = kvsynth.WORKLOADS["llama3_8b_gqa_32k"]
    # one sampled batch row per KV head, so every KV head (and the query heads that share it) is compared
    cache, got = _sampled_full_size(kvq, w, [(0, 0), (9, 1), (17, 2), (26, 3), (35, 4), (44, 5), (53, 6), (63, 7)])
    # any-size property: each output is a convex combination of its slice's decoded values, so it lies within
    # the largest decoded magnitude of that value slice; decoded |v| <= |v| + s/2 and s <= range/3
    assert np.abs(got).max() < 10.0


def test_long_1m_sampled(kvq):
    w = kvsynth.WORKLOADS["long_1m"]
    _sampled_full_size(kvq, w, [(0, 5), (0, 30)])
