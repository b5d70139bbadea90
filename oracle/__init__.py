"""CPU oracle for KIVI-style 2-bit (and KVQuant-style 4-bit) KV-cache quantization and decode attention.

TEST INFRASTRUCTURE ONLY. Only the tests, the package smoke check and the benchmark's CPU-baseline leg may import
this package. The product path (the HIP library and its Python binding) never imports, calls or links it, and the
two share no code: only the seeded input generators in ``kvsynth`` serve both.

The oracle is plain numpy, in float64 except where a step is defined in binary32 or binary16 arithmetic, in which
case that arithmetic is emulated exactly (each binary32 operation is done in float64 and rounded once to float32;
binary64 carries more than 2*24+2 bits, so the double rounding is innocuous for +, -, * and /).

Sources, as cited in each function:
- KIVI page (fdeinterviews.com, "KIVI: A Tuning-Free Asymmetric 2bit Quantization for KV Cache"): keys are grouped
  per channel, 32 tokens of one channel per group; values per token; the newest tokens (up to R = 128) stay in
  full precision and are quantized in blocks when the window fills.
- synthetic.wiki "KV cache quantization", section "Keys are harder than values": per-channel keys, per-token
  values, and the grouped part plus residual part of the key cache that are combined when computing attention
  scores.

Modules:
- ``quant``: the asymmetric min/max group quantizer and its decoder.
- ``layout``: the packed 3072-byte tile record the library stores, packed and unpacked independently here.
- ``cache``: the grouped + residual cache state machine (append one token at a time, flush a full window).
- ``attention``: attention over the decoded cache, chunked, plus the algebraic refold and split-K merge; with the
  KVQuant variant's sink token and rotary embedding of pre-RoPE keys.
- ``layout4``: the 5120-byte 4-bit tile record and the per-slice sink record of the KVQuant variant.
- ``rope``: the rotary embedding (adjacent channel pairs, theta_i = base ** (-2 i / D), absolute positions).

synthetic.wiki "KV cache quantization: putting the bits in the cached vectors, not the weights" on KVQuant:
section "Keys are harder than values" (keys quantized before RoPE, the rotation applied after dequantization) and
section "What they report" (the first token's keys kept in full precision; per-vector dense-and-sparse groups);
4-bit codes are the KVQuant-style workload's width.
"""
