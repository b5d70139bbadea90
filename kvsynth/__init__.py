"""Seeded, chunk-addressable synthetic inputs for the 2-bit KV-cache decode path.

This module only draws numbers. It holds none of the method's arithmetic (no quantizer, no packing, no
attention), so both the CPU oracle and the GPU path may consume what it produces.

Distribution (KIVI page, paragraph on what the cache contains; synthetic.wiki "Keys are harder than values"):
keys carry a few fixed channels of very large magnitude, values show no such pattern. Synthetic stand-in:
every element ~ N(0, 1) drawn in float32; for keys, a fixed set of outlier channels per KV head (the same for
every batch row and token) is multiplied by a factor before rounding to float16. The pages measure on model
activations and public benchmarks that are not available here; these tensors stand in for them.

Addressing: the tokens of one (batch row b, head h) slice are cut into chunks of ``CHUNK`` tokens; chunk c is
drawn from its own PCG64 stream seeded with ``SeedSequence([seed, tensor_id, b, h, c])``. Any token range of any
slice can therefore be regenerated on its own, which lets the oracle check sampled slices of a workload that
does not fit in host memory as a whole.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

CHUNK = 65536

# tensor ids of the streams
K_ID = 0
V_ID = 1
Q_ID = 2
OUTLIER_ID = 99


def outlier_channels(seed: int, h: int, n_out: int, head_dim: int = 128) -> np.ndarray:
    """Sorted indices of the ``n_out`` outlier channels of KV head ``h`` (drawn without replacement)."""
    if n_out <= 0:
        return np.zeros(0, dtype=np.int64)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, OUTLIER_ID, h])))
    return np.sort(g.choice(head_dim, n_out, replace=False))


def _chunk(seed: int, tensor_id: int, b: int, h: int, c: int, n: int, head_dim: int) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id, b, h, c])))
    return g.standard_normal((n, head_dim), dtype=np.float32)


def slice_tokens(seed: int, tensor_id: int, b: int, h: int, t0: int, t1: int, head_dim: int = 128,
                 n_out: int = 0, factor: float = 1.0) -> np.ndarray:
    """Tokens ``[t0, t1)`` of slice (b, h) as float16 ``[t1 - t0, head_dim]``.

    Chunk c always holds ``CHUNK`` tokens of its stream, so the values of a token do not depend on the range asked
    for. Outlier channels (``n_out`` of them, scaled by ``factor``) are scaled in float32 before the float16
    rounding.
    """
    if t1 <= t0:
        return np.zeros((0, head_dim), dtype=np.float16)
    out = np.empty((t1 - t0, head_dim), dtype=np.float32)
    c0, c1 = t0 // CHUNK, (t1 - 1) // CHUNK
    for c in range(c0, c1 + 1):
        lo, hi = max(t0, c * CHUNK), min(t1, (c + 1) * CHUNK)
        full = _chunk(seed, tensor_id, b, h, c, min(CHUNK, hi - c * CHUNK), head_dim)
        out[lo - t0:hi - t0] = full[lo - c * CHUNK:hi - c * CHUNK]
    if n_out > 0 and factor != 1.0:
        ch = outlier_channels(seed, h, n_out, head_dim)
        out[:, ch] *= np.float32(factor)
    return out.astype(np.float16)


def kv_tensor(seed: int, tensor_id: int, batch: int, heads: int, t0: int, t1: int, head_dim: int = 128,
              n_out: int = 0, factor: float = 1.0, threads: int | None = None,
              out: np.ndarray | None = None) -> np.ndarray:
    """Tokens ``[t0, t1)`` of every slice as float16 ``[batch, heads, t1 - t0, head_dim]``."""
    if out is None:
        out = np.empty((batch, heads, t1 - t0, head_dim), dtype=np.float16)
    jobs = [(b, h) for b in range(batch) for h in range(heads)]

    def one(bh):
        b, h = bh
        out[b, h] = slice_tokens(seed, tensor_id, b, h, t0, t1, head_dim, n_out, factor)

    nthreads = threads or min(16, len(os.sched_getaffinity(0)))
    if nthreads <= 1 or len(jobs) == 1:
        for j in jobs:
            one(j)
    else:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(one, jobs))
    return out


def query(seed: int, step: int, batch: int, q_heads: int, head_dim: int = 128) -> np.ndarray:
    """Decode query of step ``step`` as float16 ``[batch, q_heads, head_dim]``, ~ N(0, 1)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, Q_ID, step])))
    return g.standard_normal((batch, q_heads, head_dim), dtype=np.float32).astype(np.float16)


@dataclass(frozen=True)
class Workload:
    """Shape and distribution of one synthetic workload."""
    name: str
    batch: int
    q_heads: int
    kv_heads: int
    context: int            # tokens in the cache at the measured decode call (prefill + steps)
    prefill: int            # tokens written by the prefill append
    steps: int              # decode steps after the prefill (each appends one token, then attends)
    seed: int
    k_outliers: int
    k_factor: float
    bits: int = 2
    head_dim: int = 128
    group: int = 32
    residual: int = 128
    sink: bool = False              # token 0's keys kept in fp16 (KVQuant variant)
    rope_base: float | None = None  # keys cached before the rotary embedding, rotated at decode time
    sparse: bool = False            # dense-and-sparse groups: each group's largest element kept apart in fp16
    notes: str = ""
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    # batch 1, one head, 1024 tokens: 896 quantized + 128 fp16 after the lazy flush rule.
    "tiny_1k": Workload("tiny_1k", 1, 1, 1, 1024, 1023, 1, 1001, 4, 20.0,
                        notes="B1 H1 D128 N1024, K outliers 4 ch x20, one decode query"),
    # Llama-2-7B-shaped layer: batch 8, 32 heads, 4096-token prefill then 256 decode steps.
    "llama2_7b_stream": Workload("llama2_7b_stream", 8, 32, 32, 4096 + 256, 4096, 256, 1002, 4, 15.0,
                                 notes="B8 H32 D128, prefill 4096 + 256 decode steps, K outliers 4 ch x15"),
    # Llama-3-8B-shaped GQA decode at 32K context.
    "llama3_8b_gqa_32k": Workload("llama3_8b_gqa_32k", 64, 32, 8, 32768, 32767, 1, 1003, 6, 20.0,
                                  notes="B64 Hq32 Hkv8 D128 N32768, K outliers 6 ch x20"),
    # The GQA 32K cache with 2-bit dense-and-sparse groups (one fp16 outlier per group of 32).
    "llama3_8b_gqa_32k_sparse": Workload("llama3_8b_gqa_32k_sparse", 64, 32, 8, 32768, 32767, 1, 1003, 6, 20.0,
                                         sparse=True,
                                         notes="llama3_8b_gqa_32k with dense-and-sparse groups: per key channel and "
                                               "value token group of 32, the largest element kept in fp16"),
    # One sequence of 1,048,576 tokens, 32 heads.
    "long_1m": Workload("long_1m", 1, 32, 32, 1048576, 1048575, 1, 1004, 4, 20.0,
                        notes="B1 H32 D128 N1048576, K outliers 4 ch x20"),
    # KVQuant-style variant: 4-bit codes, keys cached before RoPE (base 10000), token 0's keys in fp16.
    "kvquant_4bit_16k": Workload("kvquant_4bit_16k", 16, 32, 32, 16384, 16383, 1, 1005, 4, 20.0, bits=4,
                                 sink=True, rope_base=10000.0,
                                 notes="B16 H32 D128 N16384, 4-bit, pre-RoPE keys (base 10000), fp16 sink token 0, "
                                       "K outliers 4 ch x20 (values plain N(0,1))"),
    # The same cache and data with dense-and-sparse groups (one fp16 outlier per group of 32).
    "kvquant_4bit_sparse_16k": Workload("kvquant_4bit_sparse_16k", 16, 32, 32, 16384, 16383, 1, 1005, 4, 20.0,
                                        bits=4, sink=True, rope_base=10000.0, sparse=True,
                                        notes="kvquant_4bit_16k with dense-and-sparse groups: per key channel and "
                                              "value token group of 32, the largest element kept in fp16"),
}
