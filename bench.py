#!/usr/bin/env python3
"""Decode-step benchmark of the 2-bit KV cache on one MI355X.

One step = one token appended to every sequence (window append, with the 128-token flush into packed 2-bit tiles
when the window is full) followed by decode attention of one query per (sequence, query head) over the whole
cache. The cache is built from seeded synthetic keys/values/queries (kvsynth) and is resident in HBM before the
timed region starts. The default workload is the GQA decode at 32K context (batch 64, 32 query heads sharing
8 KV heads); the prefill is sized so the first timed step attends over exactly 32768 tokens.

Printed (one JSON line on stdout): KV tokens/s over the timed steps (value), the decode-attention call's achieved
algorithmic HBM bandwidth against the 8 TB/s peak (roofline), the engine clock over the timed calls (a probe
wavefront per XCD beside them), the box's streaming-read ceiling, the same call over an all-fp16 cache (the
fp16-versus-2-bit comparison), and the CPU oracle timed on a sample of the same workload (cpu_baseline: attention
rate as the value, quantization rate beside it). With the default workload the line also carries `workloads`:
sub-records for the 4-bit KVQuant-style variant (kvquant_4bit_16k), the 1M-token single sequence (long_1m), each
with the same warm-up and timed step counts, and the single-launch decode step of the Llama-2-7B-shaped stream
(128 steps over three cache copies in turn, eager per-step percentiles and one HIP graph). Progress goes to stderr.

`--workload NAME` measures one workload alone (e.g. kvquant_4bit_16k, kvquant_4bit_sparse_16k, long_1m).

`--step-graph` measures whole decode steps (append + attention) several ways on the same inputs: the host-length
calls issued eagerly, the single-launch ragged step issued eagerly, the ragged step with all timed steps captured
in one HIP graph, the graph over cache copies in turn, and a batch at mixed lengths. Default workload for it:
llama2_7b_stream (batch 8, 32 heads, 4096-token prefill), whose steps are short enough for launch costs to show.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

METRIC = "2-bit KV decode attention: KV tokens/s and achieved HBM GB/s (% of peak)"
METRIC_SPARSE = "2-bit KV decode attention with dense-and-sparse groups: KV tokens/s and achieved HBM GB/s (% of peak)"
METRIC_4BIT = "4-bit pre-RoPE KV decode attention with sink: KV tokens/s and achieved HBM GB/s (% of peak)"
METRIC_4BIT_SPARSE = ("4-bit pre-RoPE KV decode attention with sink and dense-and-sparse groups: KV tokens/s and "
                      "achieved HBM GB/s (% of peak)")
PEAK_GBS = 8000.0          # MI355X HBM3E
ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "decode_attention_quant_amd", "csrc")
# per workload: the committed HBM byte-counter summary of its pass-1 kernel and the sources that kernel is built from
_COMMON = [os.path.join(CSRC, f) for f in ("kvq_kernels.h", "kvq_lanes.h", "kvq_quantizer.h")]
TRAFFIC = {
    "llama3_8b_gqa_32k": (os.path.join(ROOT, "profiles", "decode_pass1_traffic_llama3_8b_gqa_32k.json"),
                          [os.path.join(CSRC, "kvq_kernels.hip")] + _COMMON),
    "kvquant_4bit_16k": (os.path.join(ROOT, "profiles", "decode_b4_pass1_traffic_kvquant_4bit_16k.json"),
                         [os.path.join(CSRC, "kvq_kernels_b4.hip")] + _COMMON),
    "llama3_8b_gqa_32k_sparse": (os.path.join(ROOT, "profiles", "decode_pass1_sparse_traffic_llama3_8b_gqa_32k_sparse.json"),
                                 [os.path.join(CSRC, "kvq_kernels.hip")] + _COMMON),
    "kvquant_4bit_sparse_16k": (os.path.join(ROOT, "profiles",
                                             "decode_b4_pass1_traffic_kvquant_4bit_sparse_16k.json"),
                                [os.path.join(CSRC, "kvq_kernels_b4.hip")] + _COMMON),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(batch, kv_heads, q_heads, n_quant, n_resid, head_dim=128, bits=2, n_sink=0, sparse=False):
    """Bytes one decode-attention call must move: per quantized token and KV head 96 B at 2 bits (32 B key codes,
    32 B value codes, 16 B key scale/zero, 16 B value scale/zero) or 160 B at 4 bits (64 + 64 + 16 + 16), plus 24 B
    with dense-and-sparse groups (a tile's 768-byte outlier section over 32 tokens: 120 B at 2 bits), per window
    token 512 B of fp16
    K and V, per sink token 336 B (fp16 key, value codes, value scale/zero; 348 B with the value outliers), the fp16
    query and the fp32 output. Each KV slice counts once, however many query heads read it."""
    per_q = (120 if sparse else 96) if bits == 2 else (184 if sparse else 160)
    per_sink = 348 if sparse else 336
    return (batch * kv_heads * (n_quant * per_q + n_resid * 2 * head_dim * 2 + n_sink * per_sink)
            + batch * q_heads * head_dim * 2 + batch * q_heads * head_dim * 4)


def lengths_after(n_quant, n_resid, appended, R):
    """Cache lengths after `appended` single-token appends (lazy flush of a full window)."""
    for _ in range(appended):
        if n_resid == R:
            n_quant, n_resid = n_quant + R, 0
        n_resid += 1
    return n_quant, n_resid


def kernel_source_sha256(workload):
    """sha256 over the sources of the workload's pass-1 kernel, in order (a changed kernel voids its counters)."""
    h = hashlib.sha256()
    for path in TRAFFIC[workload][1]:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_per_launch(workload):
    """HBM bytes per decode pass-1 launch from the committed counter summary, if the kernel sources still match."""
    if workload not in TRAFFIC:
        return None
    try:
        with open(TRAFFIC[workload][0]) as f:
            rec = json.load(f)
        if rec.get("kernel_source_sha256") == kernel_source_sha256(workload):
            return rec.get("traffic_bytes_per_launch")
    except (OSError, ValueError):
        pass
    return None


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        return 1


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            return next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:  # pragma: no cover - no procfs
        return None


def cpu_baseline(w, queries, n_slices, context, quant_threads=None):
    """The oracle (as it stands) on a sample of the same workload, timed on the host cores.

    Quantization (the oracle's per-channel key and per-token value quantizer, the group rule of every flush) of
    `n_slices` (batch row, KV head) slices of `context` tokens each, the slices spread over a thread pool; then
    decode attention (dequantize + softmax attention in float64) of those slices, once for each of the given timed
    steps' queries (the oracle's cost does not depend on the query values). The attention rate is the value, in the
    metric's unit (KV tokens/s: one batch row of all heads over N tokens counts N); the quantization rate is
    reported beside it in tokens of one KV head per second and GB/s of fp16 K and V read."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import kvsynth
    from oracle import attention as oa
    from oracle import cache as oc
    G = w.q_heads // w.kv_heads
    step = max(1, (w.batch * w.kv_heads) // n_slices)
    slices = [(i // w.kv_heads, i % w.kv_heads) for i in range(0, w.batch * w.kv_heads, step)][:n_slices]
    k = np.stack([kvsynth.slice_tokens(w.seed, kvsynth.K_ID, b, h, 0, context, w.head_dim, w.k_outliers,
                                       w.k_factor) for b, h in slices])
    v = np.stack([kvsynth.slice_tokens(w.seed, kvsynth.V_ID, b, h, 0, context, w.head_dim) for b, h in slices])
    nthreads = quant_threads or min(16, len(os.sched_getaffinity(0)))
    parts = np.array_split(np.arange(len(slices)), nthreads)
    parts = [p for p in parts if len(p)]

    def quantize(idx):
        c = oc.SliceCache(len(idx), residual_cap=w.residual, bits=w.bits, sink=w.sink, sparse=w.sparse)
        oc.append_block(c, k[idx], v[idx])
        return c

    t = time.perf_counter()
    with ThreadPoolExecutor(len(parts)) as ex:
        caches = list(ex.map(quantize, parts))
    dq = time.perf_counter() - t
    del k, v
    dt = 0.0
    for qs in queries:
        for idx, c in zip(parts, caches):
            q = np.stack([qs[slices[i][0], slices[i][1] * G:(slices[i][1] + 1) * G] for i in idx])   # [S, G, D]
            t = time.perf_counter()
            oa.decode_attention(c, q, len(idx), 1, rope_base=w.rope_base)
            dt += time.perf_counter() - t
    kv_tokens = len(slices) / w.kv_heads * context * len(queries)
    blas = _blas_threads()
    frac = len(slices) / (w.batch * w.kv_heads)
    return {"value": kv_tokens / dt, "unit": "KV tokens/s", "cores": int(max(blas, len(parts))), "kind": "oracle",
            "blas_threads": int(blas), "cpu_model": _cpu_model(),
            "sample": f"{len(slices)} of {w.batch * w.kv_heads} (batch row, KV head) slices ({100 * frac:.1f}%) of "
                      f"{w.name} at {context} tokens, each attended by the queries of the first {len(queries)} timed "
                      f"steps: float64 decode attention (dequantize + softmax), {dt:.2f} s on {blas} BLAS threads; "
                      f"quantization of the same slices timed separately",
            "attention_seconds": dt,
            "quantization": {"tokens_per_s": len(slices) * context / dq,
                             "gb_s_fp16_read": len(slices) * context * w.head_dim * 2 * 2 / dq / 1e9,
                             "seconds": dq, "threads": len(parts),
                             "unit": "tokens of one KV head per second (keys per channel and values per token)",
                             "sample": f"{len(slices)} slices x {context} tokens through the oracle's append (every "
                                       f"flush quantized), slices spread over {len(parts)} threads"},
            "host_cpus": len(os.sched_getaffinity(0))}


def _probe_lib():
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "decode_attention_quant_amd", "libkvq_probe.so"))
    lib.kvq_probe_sink_words.restype = ctypes.c_size_t
    lib.kvq_probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_void_p]
    lib.kvq_probe_clock_words.restype = ctypes.c_size_t
    lib.kvq_probe_wall_clock_khz.restype = ctypes.c_int
    lib.kvq_probe_clock.argtypes = [ctypes.c_uint64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    return lib


class ClockProbe:
    """Engine clock beside the timed calls: one sleeping wavefront per XCD on a second stream (default priority)
    reads the shader cycle counter and the constant-rate counter over a window inside the timed region."""

    def __init__(self, torch):
        self.torch = torch
        self.lib = _probe_lib()
        self.words = int(self.lib.kvq_probe_clock_words())
        self.out = torch.zeros(self.words, dtype=torch.int64, device="cuda")
        self.stream = torch.cuda.Stream()
        self.khz = int(self.lib.kvq_probe_wall_clock_khz())
        self.started = False
        # the first launch loads the probe's code object (milliseconds of host time): done here, outside any timed
        # region
        if self.khz > 0:
            self.lib.kvq_probe_clock(1, self.out.data_ptr(), self.words, self.stream.cuda_stream)
            torch.cuda.synchronize()

    def start(self, seconds, after=None):
        """Probe `seconds` of wall time; with `after` (an event recorded on the timed stream) the probe's stream
        waits for it, so the window starts with the work that follows the event."""
        if self.khz <= 0 or seconds <= 0:
            return
        ticks = max(1, min(10 ** 9, int(seconds * self.khz * 1e3)))
        if after is not None:
            self.stream.wait_event(after)
        rc = self.lib.kvq_probe_clock(ticks, self.out.data_ptr(), self.words, self.stream.cuda_stream)
        self.started = rc == 0

    def result(self):
        if not self.started:
            return None
        self.torch.cuda.synchronize()
        v = self.out.cpu().tolist()
        ghz = [v[2 * i] / v[2 * i + 1] * self.khz * 1e-6 for i in range(self.words // 2) if v[2 * i + 1] > 0]
        if not ghz:
            return None
        return {"ghz_mean": sum(ghz) / len(ghz), "ghz_min": min(ghz), "ghz_max": max(ghz),
                "window_us": v[1] / self.khz * 1e3, "wavefronts": len(ghz),
                "note": "shader cycles / constant-rate ticks of one sleeping wavefront per XCD, over a window inside "
                        "the timed calls"}


def hbm_read_ceiling(nbytes, reps=20):
    """The box's achievable HBM read bandwidth: a plain streaming read (`libkvq_probe.so`, every 16-byte chunk of
    the buffer loaded once, with the non-temporal hint the decode kernels' loads also carry) of a buffer as large as
    one decode call's bytes, `reps` back-to-back launches between two HIP events on the current stream."""
    import torch
    lib = _probe_lib()
    nbytes = (int(nbytes) + 15) // 16 * 16
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    nsink = lib.kvq_probe_sink_words()
    sink = torch.empty(nsink, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    call = lambda: lib.kvq_probe_hbm_read(buf.data_ptr(), nbytes, sink.data_ptr(), nsink, st)
    for _ in range(3):
        if call() != 0:
            raise RuntimeError("kvq_probe_hbm_read failed")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    gbs = nbytes / us / 1e3
    del buf, sink
    return {"gb_s": gbs, "frac_of_peak": gbs / PEAK_GBS, "bytes": nbytes, "us_per_launch": us, "launches": reps,
            "kernel": "hbm_read_kernel (libkvq_probe.so): 2048 wavefronts, one contiguous segment each, eight "
                      "1 KB loads in flight"}


def fp16_comparator(kvq, w, Kd, Vd, q, context, call_us_2bit, calls):
    """The same decode-attention call over an all-fp16 cache of the same context: a window as large as the context,
    so nothing is quantized (same library, same kernel, fp16 tiles only). Timed with HIP events over `calls` calls
    after 3 warm-ups; the cache is built from the same synthetic K/V."""
    import torch
    cap = ((context + 31) // 32) * 32
    shape = kvq.Shape(w.batch, w.kv_heads, w.q_heads, residual_cap=cap, max_tokens=cap)
    c16 = kvq.KVCache(shape)
    kvq.kv_append_and_flush(c16, Kd[:, :, :context], Vd[:, :, :context])
    out = torch.empty((w.batch, w.q_heads, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(16, kvq.kv_decode_attention_workspace_bytes(c16)), dtype=torch.uint8, device="cuda")
    for _ in range(3):
        kvq.kv_decode_attention(c16, q, out=out, workspace=ws)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(calls + 1)]
    ev[0].record()
    for i in range(calls):
        kvq.kv_decode_attention(c16, q, out=out, workspace=ws)
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(calls)]
    us = 1e3 * sum(ms) / calls
    nbytes = w.batch * w.kv_heads * context * 512 + w.batch * w.q_heads * 128 * 6
    del c16, ws
    torch.cuda.empty_cache()
    log(f"[bench] fp16 comparator: {context} fp16 tokens, {us:.1f} us per call, {nbytes / us / 1e3:.0f} GB/s")
    return {"context": context, "decode_call_us": us, "bytes_per_call": nbytes, "hbm_gb_s": nbytes / us / 1e3,
            "pct_of_peak": 100.0 * nbytes / us / 1e3 / PEAK_GBS, "kv_tokens_per_s": w.batch * context / (us * 1e-6),
            "speedup_2bit_over_fp16": us / call_us_2bit if call_us_2bit else None,
            "note": "same library and kernel over a window as large as the context (no quantized tiles)"}


def step_graph(args, kvq, kdev, kvsynth, torch):
    """Decode-step time (append + attention) on one workload: host-length API eager, ragged step eager, ragged step
    captured in one graph of all timed steps, and the same graph over `--rotate` copies of the cache in turn (a
    working set larger than the 256 MB last-level cache, so the steps read HBM; the value reported). Prints one JSON
    line."""
    w = kvsynth.WORKLOADS[args.workload]
    if w.bits != 2:
        raise SystemExit("--step-graph: ragged caches are 2-bit")
    W, K, R = args.warmup, args.steps, w.residual
    P = w.prefill if w.steps >= W + K else w.context - W - K   # prefill, then W warm-up and K timed steps
    total = P + W + K
    cap = ((total + 31) // 32) * 32
    t0 = time.time()
    Kd = kdev.kv_to_device(w, kvsynth.K_ID, 0, total)
    Vd = kdev.kv_to_device(w, kvsynth.V_ID, 0, total)
    Q = kdev.queries_to_device(w, range(1, W + K + 1))
    log(f"[step-graph] {w.name}: prefill {P}, {W} warm-up + {K} timed steps; data in {time.time() - t0:.1f}s")
    shape = kvq.Shape(w.batch, w.kv_heads, w.q_heads, residual_cap=R, max_tokens=cap)
    out = torch.empty((w.batch, w.q_heads, 128), dtype=torch.float32, device="cuda")

    def timed(run_steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        run_steps()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / K   # us per step

    # host-length calls
    hc = kvq.KVCache(shape)
    kvq.kv_append_and_flush(hc, Kd[:, :, :P], Vd[:, :, :P])
    ws_h = torch.empty(max(16, kvq.kv_decode_attention_workspace_bytes(hc) * 2), dtype=torch.uint8, device="cuda")

    def host_step(i):
        t = P + i
        kvq.kv_append_and_flush(hc, Kd[:, :, t:t + 1], Vd[:, :, t:t + 1])
        kvq.kv_decode_attention(hc, Q[i], out=out, workspace=ws_h)

    for i in range(W):
        host_step(i)
    us_host = timed(lambda: [host_step(W + j) for j in range(K)])
    ctx = hc.n_tokens

    # ragged step, eager
    def ragged_cache():
        rc = kvq.RaggedCache(shape)
        for b in range(w.batch):
            kvq.kv_ragged_prefill(rc, b, Kd[b, :, :P], Vd[b, :, :P])
        return rc

    rc = ragged_cache()
    ws_r = torch.empty(kvq.kv_ragged_workspace_bytes(rc), dtype=torch.uint8, device="cuda")

    def ragged_step(c, i, o):
        t = P + i
        kvq.kv_ragged_decode_step(c, Kd[:, :, t], Vd[:, :, t], Q[i], out=o, workspace=ws_r)

    for i in range(W):
        ragged_step(rc, i, out)
    us_ragged = timed(lambda: [ragged_step(rc, W + j, out) for j in range(K)])

    # ragged steps captured once (every timed step its own inputs and output row), replayed once
    gc = ragged_cache()
    outs = torch.empty((K, w.batch, w.q_heads, 128), dtype=torch.float32, device="cuda")
    for i in range(W):
        ragged_step(gc, i, outs[0])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for j in range(K):
            ragged_step(gc, W + j, outs[j])
    us_graph = timed(graph.replay)
    # the replayed graph and the eager ragged steps ran the same kernels on the same inputs
    same = bool(torch.equal(outs[K - 1], out)) and bool(torch.equal(gc.lens, rc.lens))
    del graph, gc

    # the same steps over `rot` cache copies in turn, captured in one graph: copy r takes steps r, r + rot, ...
    rot = max(1, args.rotate)
    us_rot = us_graph
    if rot > 1:
        copies = [ragged_cache() for _ in range(rot)]
        for c in copies:
            for i in range(W):
                ragged_step(c, i, outs[0])
        torch.cuda.synchronize()
        graph_r = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph_r):
            for j in range(K):
                ragged_step(copies[j % rot], W + j // rot, outs[j])
        us_rot = timed(graph_r.replay)
        del graph_r, copies
    # ragged lengths: sequence b prefilled with P (b + 1) / B tokens (a serving batch at mixed positions), the same
    # single-launch steps in one graph over enough cache copies in turn to exceed the last-level cache; bytes from
    # each copy's lengths at its last timed step
    B = w.batch
    lens0 = [max(32, (P * (b + 1)) // B) for b in range(B)]
    kmix = [torch.stack([Kd[b, :, lens0[b] + i] for b in range(B)]) for i in range(W + K)]
    vmix = [torch.stack([Vd[b, :, lens0[b] + i] for b in range(B)]) for i in range(W + K)]

    def mix_cache():
        c = kvq.RaggedCache(shape)
        for b in range(B):
            kvq.kv_ragged_prefill(c, b, Kd[b, :, :lens0[b]], Vd[b, :, :lens0[b]])
        return c

    def mix_step(c, i, o):
        kvq.kv_ragged_decode_step(c, kmix[i], vmix[i], Q[i], out=o, workspace=ws_r)

    def mix_bytes(c):
        ln = c.lens.cpu().tolist()
        return sum(algorithmic_bytes(1, w.kv_heads, w.q_heads, nq, nr) for nq, nr, _, _ in ln)

    mc = mix_cache()
    for i in range(W):
        mix_step(mc, i, out)
    us_mix_eager = timed(lambda: [mix_step(mc, W + j, out) for j in range(K)])
    rot_mix = max(rot, -(-320 * 2 ** 20 // mix_bytes(mc)))
    mcopies = [mix_cache() for _ in range(rot_mix)]
    for c in mcopies:
        for i in range(W):
            mix_step(c, i, outs[0])
    torch.cuda.synchronize()
    graph_m = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph_m):
        for j in range(K):
            mix_step(mcopies[j % rot_mix], W + j // rot_mix, outs[j])
    us_mix = timed(graph_m.replay)
    mix_last = sum(mix_bytes(c) for c in mcopies) / rot_mix
    mix_tokens = sum(int(c.lens[:, :2].sum()) for c in mcopies) / rot_mix
    del graph_m, mcopies, mc
    log(f"[step-graph] ragged lengths {lens0[0]}..{lens0[-1]}: eager {us_mix_eager:.1f} us, graph over {rot_mix} copies "
        f"{us_mix:.1f} us per step ({mix_last / us_mix / 1e3:.0f} GB/s)")

    nbytes = algorithmic_bytes(w.batch, w.kv_heads, w.q_heads, hc.n_quant, hc.n_resid)
    # the step's own bytes: attention over the cache, plus the new token read (fp16 K, V) and its window row written
    step_bytes = nbytes + w.batch * w.kv_heads * 4 * w.head_dim * 2
    log(f"[step-graph] per step: host API {us_host:.1f} us, ragged eager {us_ragged:.1f} us, ragged graph "
        f"{us_graph:.1f} us (graph == eager: {same}); graph over {rot} cache copies {us_rot:.1f} us")
    res = {
        "metric": "2-bit decode step (append + attention), per-step time and KV tokens/s",
        "value": w.batch * ctx / (us_rot * 1e-6),
        "unit": "KV tokens/s",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": us_rot / 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.q_heads, "kv_heads": w.kv_heads,
                   "prefill": P, "context_last_timed_step": ctx, "bits": 2, "residual": R},
        "modes_us_per_step": {"host_api_eager": us_host, "ragged_step_eager": us_ragged,
                              "ragged_step_graph": us_graph, f"ragged_step_graph_{rot}_copies": us_rot},
        "graph_equals_eager": same,
        "roofline": {"bound": "hbm", "achieved": step_bytes / us_rot / 1e3, "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": step_bytes / us_rot / 1e3 / PEAK_GBS, "traffic": None,
                     "kernel": "decode_pass1_kernel<2> (one kv_ragged_decode_step launch: flush, append, attention, "
                               "merge, length commit)", "bytes_per_step": step_bytes,
                     "note": "attention bytes of the last timed step plus the new token's K, V read and window row "
                             "written; a window flush (once per 128 steps) is not counted"},
        "ragged_lengths": {"prefill_lengths": lens0, "us_per_step_eager": us_mix_eager,
                           f"us_per_step_graph_{rot_mix}_copies": us_mix, "bytes_last_step": mix_last,
                           "gb_s": mix_last / us_mix / 1e3, "kv_tokens_per_s": mix_tokens / (us_mix * 1e-6),
                           "note": "sequence b prefilled with P (b + 1) / B tokens, then the same single-launch "
                                   "steps; every sequence's tiles are spread over the same fixed number of splits"},
        "bytes_last_step": nbytes,
        "gb_s_graph_last_step_bytes": nbytes / us_graph / 1e3,
        "hbm_gb_s_graph_copies_last_step_bytes": nbytes / us_rot / 1e3,
        "note": "host_api_eager: kv_append_and_flush + kv_decode_attention per step (3 launches, 5 on a flush step); "
                "ragged_step_*: kv_ragged_decode_step (one launch); graph: all timed steps captured in one HIP "
                "graph, replayed once; one cache (about 115 MB) stays in the 256 MB last-level cache, the copies "
                "in turn do not (value and ms_per_step)",
    }
    if not args.no_cpu_baseline:
        log(f"[step-graph] timing the CPU oracle on {args.cpu_slices} slices x {args.cpu_queries} queries")
        qs = [Q[W + j].cpu().numpy() for j in range(min(args.cpu_queries, K))]
        res["cpu_baseline"] = cpu_baseline(w, qs, args.cpu_slices, ctx)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)
    return 0


def measure_decode(kvq, kdev, kvsynth, torch, w, W, K, clock=True, before_timed=None, settle_calls=0):
    """One workload: prefill (timed as one append), W warm-up steps, then K timed steps, each one token appended to
    every sequence and one decode-attention call, with HIP events around every append and every call on the current
    stream. `before_timed(state)`, if given, runs after the prefill (other measurements of the same run) and returns
    entries for the record. With settle_calls > 0, that many decode calls on the prefilled cache (no appends) lead
    in to the warm-up steps: they, the warm-up steps and the timed steps are enqueued back to back with no host
    synchronization in between, as in a serving loop, so the timed steps run at the steady rate and not in the
    engine-clock dip that follows any pause of the GPU (each lead-in call is timed and reported as `settled`).
    Returns the record and the device tensors the extras reuse."""
    R = w.residual
    P = w.context - W - 1                      # first timed step attends over exactly w.context tokens
    total = P + W + K
    flags = ((kvq.FLAG_SINK if w.sink else 0) | (kvq.FLAG_PRE_ROPE if w.rope_base else 0)
             | (kvq.FLAG_SPARSE if w.sparse else 0))
    shape = kvq.Shape(w.batch, w.kv_heads, w.q_heads, residual_cap=R, max_tokens=((total + 31) // 32) * 32,
                      bits=w.bits, flags=flags, rope_base=w.rope_base or 0.0)
    cache = kvq.KVCache(shape)
    t0 = time.time()
    Kd = kdev.kv_to_device(w, kvsynth.K_ID, 0, total)
    Vd = kdev.kv_to_device(w, kvsynth.V_ID, 0, total)
    Q = kdev.queries_to_device(w, range(1, W + K + 1))
    log(f"[bench] {w.name}: generated and uploaded {total} tokens x {w.batch * w.kv_heads} slices "
        f"in {time.time() - t0:.1f}s")
    # a small append on a throwaway cache first: the first launch of the library's kernels in a process also loads
    # their code object, which is no part of the prefill's cost
    warm = kvq.KVCache(kvq.Shape(1, w.kv_heads, w.q_heads, residual_cap=R, max_tokens=R, bits=w.bits, flags=flags,
                                 rope_base=w.rope_base or 0.0))
    kvq.kv_append_and_flush(warm, Kd[:1, :, :R + 2], Vd[:1, :, :R + 2])
    torch.cuda.synchronize()
    del warm
    pe = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    pe[0].record()
    kvq.kv_append_and_flush(cache, Kd[:, :, :P], Vd[:, :, :P])
    pe[1].record()
    torch.cuda.synchronize()
    prefill_us = pe[0].elapsed_time(pe[1]) * 1e3
    rec_bytes = shape.record_bytes
    # prefill traffic: every token's fp16 K and V read once; tiles, window rows (and the sink record) written
    prefill_bytes = (w.batch * w.kv_heads * (P * 512 + cache.n_quant // 32 * rec_bytes + cache.n_resid * 512
                                             + cache.n_sink * 512))
    prefill_quant, prefill_resid, prefill_sink, prefill_tokens = cache.n_quant, cache.n_resid, cache.n_sink, \
        cache.n_tokens
    log(f"[bench] prefill {P} tokens: n_sink={cache.n_sink} n_quant={cache.n_quant} n_resid={cache.n_resid} "
        f"in {prefill_us:.0f} us ({prefill_bytes / prefill_us / 1e3:.0f} GB/s)")

    # workspace for the largest split count any step will use (host-side length simulation only)
    ws_bytes = 16
    nq, nr = cache.n_quant, cache.n_resid
    for i in range(W + K):
        nq, nr = lengths_after(nq, nr, 1, R)
        probe = kvq.KvqCache(cache.c.tiles, cache.c.k_res, cache.c.v_res, nq, nr, cache.c.n_sink, cache.c.sink)
        ws_bytes = max(ws_bytes, int(kvq.library().kv_decode_attention_workspace_bytes(
            kvq.ctypes.byref(cache._cshape), kvq.ctypes.byref(probe))))
    workspace = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    out = torch.empty((w.batch, w.q_heads, 128), dtype=torch.float32, device="cuda")
    before = before_timed({"cache": cache, "Kd": Kd, "Vd": Vd, "Q": Q, "out": out, "workspace": workspace}) \
        if before_timed is not None else {}

    def step(i):
        t = P + i
        kvq.kv_append_and_flush(cache, Kd[:, :, t:t + 1], Vd[:, :, t:t + 1])

    probe_clock = ClockProbe(torch) if clock else None   # (its set-up synchronizes: before the lead-in)
    # one call on its own: the length of the clock probe's window inside the timed calls
    e1 = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    e1[0].record()
    kvq.kv_decode_attention(cache, Q[0], out=out, workspace=workspace)
    e1[1].record()
    torch.cuda.synchronize()
    est_call_ms = e1[0].elapsed_time(e1[1])

    # from here to the end of the timed steps, no host synchronization
    sev = None
    if settle_calls > 0:
        sev = [torch.cuda.Event(enable_timing=True) for _ in range(settle_calls + 1)]
        sev[0].record()
        for i in range(settle_calls):
            kvq.kv_decode_attention(cache, Q[0], out=out, workspace=workspace)
            sev[i + 1].record()
    for i in range(W):
        step(i)
        kvq.kv_decode_attention(cache, Q[i], out=out, workspace=workspace)

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * K + 2)]
    call_bytes, kv_tokens, contexts = [], 0, []
    ev[0].record()
    for j in range(K):
        i = W + j
        ev[3 * j + 1].record()
        step(i)
        ev[3 * j + 2].record()
        kvq.kv_decode_attention(cache, Q[i], out=out, workspace=workspace)
        ev[3 * j + 3].record()
        if j == 0 and probe_clock is not None:   # a window inside the timed calls
            probe_clock.start(0.7 * K * est_call_ms * 1e-3, after=ev[1])
        n = cache.n_tokens
        contexts.append(n)
        kv_tokens += w.batch * n
        call_bytes.append(algorithmic_bytes(w.batch, w.kv_heads, w.q_heads, cache.n_quant, cache.n_resid,
                                            bits=w.bits, n_sink=cache.n_sink, sparse=w.sparse))
    ev[3 * K + 1].record()
    torch.cuda.synchronize()
    total_ms = ev[0].elapsed_time(ev[3 * K + 1])
    decode_ms = [ev[3 * j + 2].elapsed_time(ev[3 * j + 3]) for j in range(K)]
    append_ms = [ev[3 * j + 1].elapsed_time(ev[3 * j + 2]) for j in range(K)]
    value = kv_tokens / (total_ms * 1e-3)
    achieved = sum(call_bytes) / (sum(decode_ms) * 1e-3) / 1e9
    splits = kvq.kv_decode_attention_splits(cache)
    dsorted = sorted(decode_ms)
    pct = lambda f: 1e3 * dsorted[min(K - 1, int(f * (K - 1) + 0.5))]
    clk = probe_clock.result() if probe_clock is not None else None

    settled = None
    if sev is not None:   # the lead-in calls: before the warm-up steps, not part of value, ms_per_step or the roofline
        sus = [1e3 * sev[i].elapsed_time(sev[i + 1]) for i in range(settle_calls)]
        tail = sus[settle_calls // 2:]
        sb = algorithmic_bytes(w.batch, w.kv_heads, w.q_heads, prefill_quant, prefill_resid, bits=w.bits,
                               n_sink=prefill_sink, sparse=w.sparse)
        settled = {"calls": settle_calls, "context": prefill_tokens,
                   "decode_call_us_all": sum(sus) / settle_calls,
                   "decode_call_us_second_half": sum(tail) / len(tail),
                   "hbm_gb_s_second_half": sb / (sum(tail) / len(tail)) / 1e3,
                   "pct_of_peak_second_half": 100.0 * sb / (sum(tail) / len(tail)) / 1e3 / PEAK_GBS,
                   "decode_call_us_series": [round(u, 1) for u in sus],
                   "note": "decode calls on the prefilled cache (no appends) that lead in to the warm-up steps, "
                           "enqueued back to back with them and the timed steps (no host synchronization): not part "
                           "of value; the second half is the steady rate"}
        log(f"[bench] {settle_calls} lead-in calls before the warm-up steps: second half avg "
            f"{settled['decode_call_us_second_half']:.1f} us ({settled['hbm_gb_s_second_half']:.0f} GB/s)")
    log(f"[bench] {w.name}: {K} steps in {total_ms:.3f} ms; decode call avg {1e3 * sum(decode_ms) / K:.1f} us "
        f"({achieved:.0f} GB/s); append avg {1e3 * sum(append_ms) / K:.1f} us, max {1e3 * max(append_ms):.1f} us; "
        f"splits={splits}" + (f"; engine clock {clk['ghz_mean']:.2f} GHz" if clk else ""))

    if w.bits == 2:
        detail = "2-bit codes expanded to fp16 MFMA operands (scales folded as fp16 hi+lo), fp32 accumulation"
        kernel = "decode_pass1_kernel + decode_pass2_kernel (one kv_decode_attention call)"
    else:
        detail = ("4-bit codes: scores on the fp32 VALU (per-pair rotation by angle addition, binary32 cos/sin), "
                  "P V on fp16 MFMA (probabilities as fp16 hi+lo), fp32 accumulation")
        kernel = "decode_b4_pass1_kernel + decode_pass2_kernel (one kv_decode_attention call)"
    res = {
        "metric": (METRIC_SPARSE if w.sparse else METRIC) if w.bits == 2 else (METRIC_4BIT_SPARSE if w.sparse
                                                                              else METRIC_4BIT),
        "value": value,
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": total_ms / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.q_heads, "kv_heads": w.kv_heads,
                   "context_first_timed_step": contexts[0], "context_last_timed_step": contexts[-1],
                   "bits": w.bits, "group": w.group, "residual": R, "head_dim": w.head_dim,
                   "sink": bool(w.sink), "rope_base": w.rope_base, "sparse": bool(w.sparse)},
        "hbm_gb_s": achieved,
        "pct_of_peak": 100.0 * achieved / PEAK_GBS,
        "decode_call_us": 1e3 * sum(decode_ms) / K,
        "append_us_avg": 1e3 * sum(append_ms) / K,
        "append_us_max": 1e3 * max(append_ms),
        "splits": splits,
        "decode_call_us_p10_p50_p90": [pct(0.1), pct(0.5), pct(0.9)],
        "decode_call_us_series": [round(1e3 * x, 1) for x in decode_ms] if K <= 256 else None,
        "engine_clock": clk,
        "prefill": {"tokens": P, "us": prefill_us, "bytes": prefill_bytes,
                    "gb_s": prefill_bytes / prefill_us / 1e3,
                    "note": "one kv_append_and_flush of the prefill: key and value quantization of the flushed "
                            "tiles plus the window copy; bytes = fp16 K and V read + records and window written"},
        "dtype_detail": detail,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_GBS, "traffic": traffic_per_launch(w.name),
                     "kernel": kernel, "bytes_per_call": sum(call_bytes) / K},
    }
    res.update(before)
    if settled is not None:
        res["settled"] = settled
    state = {"Kd": Kd, "Vd": Vd, "Q": Q, "cache": cache, "contexts": contexts}
    return res, state


def compact(rec):
    """The sub-record of one extra workload: its shape, the call's time and its roofline."""
    keys = ("decode_call_us", "decode_call_us_p10_p50_p90", "hbm_gb_s", "pct_of_peak", "splits", "engine_clock",
            "append_us_avg", "steps", "warmup")
    r = {k: rec[k] for k in keys if k in rec}
    r["metric"] = rec["metric"]
    r["config"] = rec["config"]
    r["kv_tokens_per_s"] = rec["value"]
    r["roofline"] = {k: rec["roofline"][k] for k in ("achieved", "frac", "bytes_per_call", "traffic", "kernel")}
    r["prefill_gb_s"] = rec["prefill"]["gb_s"]
    if "settled" in rec:
        r["settled_decode_call_us"] = rec["settled"]["decode_call_us_second_half"]
        r["settled_pct_of_peak"] = rec["settled"]["pct_of_peak_second_half"]
    return r


def step_record(kvq, kdev, kvsynth, torch, w, W, K, rot):
    """Single-launch ragged decode steps (append with lazy flush + attention + merge + length commit in one
    kernel) over `rot` cache copies in turn, so the steps read HBM: every step timed with HIP events when issued
    eagerly (percentiles, flush steps apart), and the same steps captured in one HIP graph and replayed once."""
    R = w.residual
    # the prefill leaves the window 20 + W tokens short of full, so every copy flushes once inside its timed steps
    P = w.prefill + R - 20 - W - (w.prefill - 1) % R - 1
    total = P + W + K
    cap = ((total + 31) // 32) * 32
    Kd = kdev.kv_to_device(w, kvsynth.K_ID, 0, total)
    Vd = kdev.kv_to_device(w, kvsynth.V_ID, 0, total)
    Q = kdev.queries_to_device(w, range(1, W + K + 1))
    shape = kvq.Shape(w.batch, w.kv_heads, w.q_heads, residual_cap=R, max_tokens=cap)

    def fresh():
        c = kvq.RaggedCache(shape)
        for b in range(w.batch):
            kvq.kv_ragged_prefill(c, b, Kd[b, :, :P], Vd[b, :, :P])
        return c

    cshape = shape.c()
    ws = torch.empty(int(kvq.library().kv_ragged_workspace_bytes(kvq.ctypes.byref(cshape))), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((w.batch, w.q_heads, 128), dtype=torch.float32, device="cuda")

    def run(copies, i, o, idx):
        t = P + i
        kvq.kv_ragged_decode_step(copies[idx], Kd[:, :, t], Vd[:, :, t], Q[i], out=o, workspace=ws)

    # eager, every step between events (copy j % rot takes its step j // rot)
    copies = [fresh() for _ in range(rot)]
    for c in range(rot):
        for i in range(W):
            run(copies, i, out, c)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    ev[0].record()
    for j in range(K):
        run(copies, W + j // rot, out, j % rot)
        ev[j + 1].record()
    torch.cuda.synchronize()
    us = [1e3 * ev[j].elapsed_time(ev[j + 1]) for j in range(K)]
    # lengths before each eager step: a step flushes when its copy's window is full
    nq0, nr0 = lengths_after(*lengths_after(0, 0, P, R), W, R)
    flush = []
    for j in range(K):
        _, nr = lengths_after(nq0, nr0, j // rot, R)
        flush.append(nr == R)
    steady = sorted(u for u, f in zip(us, flush) if not f)
    pct = lambda xs, f: xs[min(len(xs) - 1, int(f * (len(xs) - 1) + 0.5))]
    del copies
    # the same steps in one graph over fresh copies
    gcopies = [fresh() for _ in range(rot)]
    for c in range(rot):
        for i in range(W):
            run(gcopies, i, out, c)
    outs = torch.empty((K, w.batch, w.q_heads, 128), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for j in range(K):
            run(gcopies, W + j // rot, outs[j], j % rot)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    graph.replay()
    b.record()
    torch.cuda.synchronize()
    us_graph = 1e3 * a.elapsed_time(b) / K
    ln = gcopies[0].lens.cpu().tolist()
    nq, nr = ln[0][0], ln[0][1]
    nbytes = algorithmic_bytes(w.batch, w.kv_heads, w.q_heads, nq, nr)
    step_bytes = nbytes + w.batch * w.kv_heads * 4 * w.head_dim * 2
    ctx = nq + nr
    del graph, gcopies, outs, Kd, Vd, Q
    torch.cuda.empty_cache()
    log(f"[bench] {w.name} decode step: graph over {rot} copies {us_graph:.1f} us per step "
        f"({step_bytes / us_graph / 1e3:.0f} GB/s); eager steady p50 {pct(steady, 0.5):.1f} us, flush steps "
        f"{[round(u, 1) for u, f in zip(us, flush) if f]}")
    return {"metric": "2-bit decode step (append with lazy flush + attention), one launch per step",
            "config": {"workload": w.name, "batch": w.batch, "q_heads": w.q_heads, "kv_heads": w.kv_heads,
                       "prefill": P, "context_last_timed_step": ctx, "bits": 2, "residual": R},
            "steps": K, "warmup": W, "cache_copies": rot,
            "step_us_graph": us_graph, "kv_tokens_per_s": w.batch * ctx / (us_graph * 1e-6),
            "step_us_eager_steady_p10_p50_p90": [pct(steady, 0.1), pct(steady, 0.5), pct(steady, 0.9)],
            "step_us_eager_flush_steps": [u for u, f in zip(us, flush) if f],
            "roofline": {"achieved": step_bytes / us_graph / 1e3, "frac": step_bytes / us_graph / 1e3 / PEAK_GBS,
                         "bytes_per_step": step_bytes,
                         "kernel": "decode_pass1_kernel<2> (kv_ragged_decode_step: flush, append, attention, merge, "
                                   "length commit)",
                         "note": "attention bytes at the last timed step plus the new token's K, V read and window "
                                 "row written; the graph's mean over all timed steps, flush steps included"}}


SUB_WORKLOADS = ("kvquant_4bit_16k", "llama3_8b_gqa_32k_sparse", "long_1m", "llama2_7b_stream")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="llama3_8b_gqa_32k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-slices", type=int, default=64)
    ap.add_argument("--cpu-queries", type=int, default=2)
    ap.add_argument("--no-fp16-comparator", action="store_true")
    ap.add_argument("--no-hbm-ceiling", action="store_true")
    ap.add_argument("--no-clock", action="store_true", help="no engine-clock probe beside the timed calls")
    ap.add_argument("--no-sub-records", action="store_true",
                    help="measure only the headline workload (else also " + ", ".join(SUB_WORKLOADS) + ")")
    ap.add_argument("--fp16-calls", type=int, default=20)
    ap.add_argument("--settle-calls", type=int, default=160,
                    help="decode calls that lead in to the warm-up steps with no host synchronization in between, "
                         "each timed and reported apart as `settled` (0: none; the timed steps then start after a "
                         "pause of the GPU)")
    ap.add_argument("--cold-calls", type=int, default=20,
                    help="decode calls timed right after the prefill, before the warm-up steps (0: none)")
    ap.add_argument("--step-graph", action="store_true",
                    help="decode-step time: host API vs ragged step vs ragged step in a HIP graph "
                         "(default workload llama2_7b_stream)")
    ap.add_argument("--rotate", type=int, default=3,
                    help="--step-graph: cache copies stepped in turn for the HBM-resident measurement")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (5 times), the reference for HBM byte counters")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (every (batch row, KV head) slice "
              "is independent, so slices would be split across GPUs with no communication). Run with --gpus 1.",
              file=sys.stderr)
        return 2

    import torch

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"bytes_read_per_copy": n, "bytes_written_per_copy": n, "copies": 5}}))
        return 0

    import decode_attention_quant_amd as kvq
    import kvsynth
    from kvsynth import device as kdev

    if args.step_graph:
        if args.workload == "llama3_8b_gqa_32k" and "--workload" not in (argv or sys.argv):
            args.workload = "llama2_7b_stream"
        return step_graph(args, kvq, kdev, kvsynth, torch)

    w = kvsynth.WORKLOADS[args.workload]
    W, K = args.warmup, args.steps

    def before_timed(s):
        """The run's other measurements, between the prefill and the warm-up steps: the decode calls right after
        the prefill (no appends), the streaming-read ceiling and the fp16 comparator."""
        extra = {}
        cache = s["cache"]
        nbytes = algorithmic_bytes(w.batch, w.kv_heads, w.q_heads, cache.n_quant, cache.n_resid, bits=w.bits,
                                   n_sink=cache.n_sink, sparse=w.sparse)
        n = args.cold_calls
        if n > 0:
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
            ev[0].record()
            for i in range(n):
                kvq.kv_decode_attention(cache, s["Q"][0], out=s["out"], workspace=s["workspace"])
                ev[i + 1].record()
            torch.cuda.synchronize()
            us = [1e3 * ev[i].elapsed_time(ev[i + 1]) for i in range(n)]
            srt = sorted(us)
            pick = lambda f: srt[min(n - 1, int(f * (n - 1) + 0.5))]
            extra["cold_start"] = {
                "calls": n, "context": cache.n_tokens, "decode_call_us": sum(us) / n,
                "decode_call_us_p10_p50_p90": [pick(0.1), pick(0.5), pick(0.9)],
                "hbm_gb_s": nbytes / (sum(us) / n) / 1e3, "pct_of_peak": 100.0 * nbytes / (sum(us) / n) / 1e3
                / PEAK_GBS, "decode_call_us_series": [round(u, 1) for u in us],
                "note": "the first decode calls after the prefill and the host-side input generation, the same call "
                        "on the prefilled cache with no appends in between; the engine clock drops a few calls in "
                        "and recovers over tens of calls"}
            log(f"[bench] {n} calls right after the prefill: avg {sum(us) / n:.1f} us "
                f"({nbytes / (sum(us) / n) / 1e3:.0f} GB/s)")
        if not args.no_hbm_ceiling:
            extra["hbm_read_ceiling"] = hbm_read_ceiling(nbytes)
        if not args.no_fp16_comparator and w.bits == 2:
            extra["fp16_comparator"] = fp16_comparator(kvq, w, s["Kd"], s["Vd"], s["Q"][W], w.context, None,
                                                       args.fp16_calls)
        return extra

    res, st = measure_decode(kvq, kdev, kvsynth, torch, w, W, K, clock=not args.no_clock, before_timed=before_timed,
                             settle_calls=args.settle_calls)
    achieved = res["hbm_gb_s"]
    if "hbm_read_ceiling" in res:
        ceil = res["hbm_read_ceiling"]
        ceil["decode_frac_of_ceiling"] = achieved / ceil["gb_s"]
        log(f"[bench] streaming-read ceiling {ceil['gb_s']:.0f} GB/s ({100 * ceil['frac_of_peak']:.1f}% of "
            f"{PEAK_GBS:.0f}); the decode call reaches {100 * ceil['decode_frac_of_ceiling']:.1f}% of it")
    if "fp16_comparator" in res:
        res["fp16_comparator"]["speedup_2bit_over_fp16"] = res["fp16_comparator"]["decode_call_us"] / \
            res["decode_call_us"]
    res["measurement_order"] = ("input generation and upload; prefill; cold_start calls; hbm_read_ceiling; "
                                "fp16_comparator; one call (the clock probe's window); then with no host "
                                "synchronization: settled (lead-in) calls, warm-up steps, timed steps; sub-record "
                                "workloads; cpu_baseline")
    Qcpu = [st["Q"][W + j].cpu().numpy() for j in range(min(args.cpu_queries, K))]
    del st
    torch.cuda.empty_cache()

    if not args.no_sub_records and "--workload" not in (argv if argv is not None else sys.argv):
        subs = {}
        for name in SUB_WORKLOADS:
            sw = kvsynth.WORKLOADS[name]
            try:
                if name == "llama2_7b_stream":
                    subs[name + "_step"] = step_record(kvq, kdev, kvsynth, torch, sw, 8, 128, 3)
                else:
                    r, s2 = measure_decode(kvq, kdev, kvsynth, torch, sw, W, K, clock=not args.no_clock,
                                           settle_calls=args.settle_calls)
                    del s2
                    subs[name] = compact(r)
            finally:
                torch.cuda.empty_cache()
        res["workloads"] = subs

    if not args.no_cpu_baseline:
        log(f"[bench] timing the CPU oracle on {args.cpu_slices} slices x {len(Qcpu)} queries")
        res["cpu_baseline"] = cpu_baseline(w, Qcpu, args.cpu_slices, res["config"]["context_first_timed_step"])
        log(f"[bench] oracle: attention {res['cpu_baseline']['value']:.0f} KV tokens/s "
            f"({res['cpu_baseline']['attention_seconds']:.1f} s), quantization "
            f"{res['cpu_baseline']['quantization']['tokens_per_s']:.0f} tokens/s "
            f"({res['cpu_baseline']['quantization']['seconds']:.1f} s)")
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
