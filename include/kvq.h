/*
 * kvq.h — C ABI of a quantized KV-cache library for AMD MI355X (gfx950): KIVI-style asymmetric quantization of keys
 * per channel and values per token (2-bit, or 4-bit in the KVQuant-style variant), a full-precision window of the
 * newest tokens, and decode attention computed straight from the packed codes plus that window. The 4-bit variant
 * can also keep keys cached before the rotary embedding (rotated at decode time), hold token 0 apart as an
 * attention sink with a full-precision key, and keep each group's largest element apart in fp16 (dense-and-sparse
 * groups).
 *
 * Sources (the pages this library follows):
 *  - KIVI page, fdeinterviews.com "KIVI: A Tuning-Free Asymmetric 2bit Quantization for KV Cache": keys grouped per
 *    channel (a group is 32 tokens of one channel), values per token, the newest tokens (up to R = 128) kept in full
 *    precision and quantized in blocks when the window fills; 2 bits per element.
 *  - synthetic.wiki "KV cache quantization", section "Keys are harder than values": per-channel keys, per-token
 *    values, and a key cache split into a grouped part and a residual part that are combined when computing
 *    attention scores.
 *  - synthetic.wiki "KV cache quantization: putting the bits in the cached vectors, not the weights", on KVQuant:
 *    section "Keys are harder than values" (per-channel keys quantized before the rotary embedding, RoPE applied
 *    after dequantization; per-token values) and section "What they report" (the first token's keys kept in full
 *    precision as an attention sink; per-vector dense-and-sparse quantization, outliers held apart so they do not
 *    stretch the quantization range). The 4-bit width is the KVQuant-style workload's.
 *
 * Conventions for every call:
 *  - All pointers named as device pointers refer to memory on the current HIP device; host pointers are named so.
 *    The caller owns every buffer. The library never allocates or frees memory and holds no global state; calls are
 *    re-entrant. The one exception is kv_decode_attention_noalloc, which keeps its scratch in a static array per
 *    GPU (see there). Work is enqueued on the caller's HIP stream (`stream` is a hipStream_t; NULL = the null stream);
 *    no call synchronizes. Calls that touch one cache must be issued on one stream, in order.
 *  - Return value: 0 on success (work enqueued; device faults, if any, surface at the caller's next
 *    synchronization). A negative KVQ_E_* code means the arguments were rejected on the host and NOTHING was
 *    launched or modified (host-side cache fields included), except KVQ_E_LAUNCH, which reports a launch failure
 *    returned by the HIP runtime after host validation succeeded.
 *  - Inputs must be finite; non-finite keys or values give unspecified codes.
 *  - Element type "fp16" is IEEE binary16; "fp32" is IEEE binary32.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define KVQ_API __attribute__((visibility("default")))
#else
#define KVQ_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define KVQ_OK 0
#define KVQ_E_NULL (-1)      /* a required pointer is NULL */
#define KVQ_E_SHAPE (-2)     /* head_dim != 128, group != 32, q_heads % kv_heads != 0, R not a positive multiple
                                of 32, non-positive sizes, a token count/offset that is not a multiple of 32,
                                unknown flags, flags with bits != 4, or KVQ_FLAG_PRE_ROPE with rope_base <= 1 (or
                                not finite) */
#define KVQ_E_BITS (-3)      /* bits not 2 or 4 */
#define KVQ_E_ALIGN (-4)     /* a device pointer is not 16-byte aligned, or a token/head/batch stride is not a
                                multiple of 8 elements (rows must be 16-byte aligned; the channel stride is 1) */
#define KVQ_E_CAPACITY (-5)  /* the quantized part would exceed max_tokens, or a tile range exceeds it */
#define KVQ_E_WORKSPACE (-6) /* workspace NULL or smaller than kv_decode_attention_workspace_bytes() */
#define KVQ_E_EMPTY (-7)     /* attention over a cache that holds no token */
#define KVQ_E_LAUNCH (-8)    /* the HIP runtime reported an error when launching */
#define KVQ_E_STATE (-9)     /* cache host fields inconsistent: n_quant not a multiple of 32 or outside
                                [0, max_tokens], n_resid outside [0, R], n_sink not 0/1, n_sink = 1 without
                                KVQ_FLAG_SINK, or (with KVQ_FLAG_SINK) n_sink = 0 while the cache holds tokens */
#define KVQ_E_SCRATCH (-10)  /* kv_decode_attention_noalloc: the call's split partials need more than
                                KVQ_NOALLOC_SCRATCH_BYTES */

/* Fixed sizes of the layouts. */
#define KVQ_HEAD_DIM 128
#define KVQ_GROUP 32
#define KVQ_TILE_TOKENS 32
#define KVQ_RECORD_BYTES 3072       /* one 32-token tile, 2-bit codes */
#define KVQ_RECORD_BYTES_SPARSE 3840  /* one 32-token tile, 2-bit codes with dense-and-sparse groups */
#define KVQ_RECORD_BYTES_4BIT 5120  /* one 32-token tile, 4-bit codes */
#define KVQ_RECORD_BYTES_4BIT_SPARSE 5888  /* one 32-token tile, 4-bit codes with dense-and-sparse groups */
#define KVQ_SINK_BYTES 512          /* the sink record of one (batch row, KV head) slice */
#define KVQ_NOALLOC_SCRATCH_BYTES (16 << 20)  /* static scratch per GPU of kv_decode_attention_noalloc */

/* kvq_shape.flags (4-bit: any OR of the three; 2-bit: 0 or KVQ_FLAG_SPARSE alone). */
#define KVQ_FLAG_SINK 1      /* token 0 is held apart: fp16 key, per-token 4-bit value (synthetic.wiki "KV cache
                                quantization", section "What they report": KVQuant's attention sink) */
#define KVQ_FLAG_PRE_ROPE 2  /* keys are given and cached before the rotary embedding; attention rotates every key
                                (sink, quantized and window alike) by its absolute position (synthetic.wiki "KV
                                cache quantization", section "Keys are harder than values": pre-RoPE keys) */
#define KVQ_FLAG_SPARSE 4    /* dense-and-sparse groups (synthetic.wiki "KV cache quantization", section "What they
                                report": per-vector dense-and-sparse quantization): in every key group (32 tokens
                                of a channel) and value group (32 channels of a token), the sink's value groups
                                included, the element of largest magnitude (the lowest index on ties) is stored
                                apart as its fp16 value and index; the other 31 are quantized by the rule of
                                kv_quant_keys_per_channel over their own minimum and maximum, and the outlier's
                                code is 0. Records are 5888 bytes (4-bit) or 3840 bytes (2-bit). */

/*
 * Shape of one cache (one attention layer).
 *   batch, kv_heads, q_heads: B, Hkv, Hq (Hq a multiple of Hkv; query head hq uses KV head hq / (Hq / Hkv), i.e.
 *   consecutive query heads share a KV head — the usual grouped-query layout);
 *   head_dim: must be 128; bits: 2 or 4; group: must be 32 (tokens per key group, channels per value group);
 *   residual_cap: R, the number of newest tokens kept in fp16 (a positive multiple of 32; 128 on the pages);
 *   flags: 0, or (bits = 4) an OR of KVQ_FLAG_SINK, KVQ_FLAG_PRE_ROPE and KVQ_FLAG_SPARSE, or (bits = 2)
 *     KVQ_FLAG_SPARSE alone; ragged caches take 2-bit codes with flags 0 only;
 *   max_tokens: capacity of the quantized part in tokens (a positive multiple of 32);
 *   rope_base: with KVQ_FLAG_PRE_ROPE, the rotary base (10000 in the usual models; must be > 1); ignored otherwise.
 *     Rotary form: channel pairs (2i, 2i+1), i = 0..63, turned by the angle m * theta_i with
 *     theta_i = rope_base^(-2i/128) at absolute position m (the sink is position 0, token k of the quantized part is
 *     position n_sink + k, window row r is position n_sink + n_quant + r): (x0, x1) -> (x0 cos - x1 sin,
 *     x0 sin + x1 cos). The query passed to kv_decode_attention is already rotated for its own position.
 */
typedef struct kvq_shape {
    int32_t batch;
    int32_t kv_heads;
    int32_t q_heads;
    int32_t head_dim;
    int32_t bits;
    int32_t group;
    int32_t residual_cap;
    int32_t flags;
    int64_t max_tokens;
    double rope_base;
} kvq_shape;

/*
 * One cache: caller-owned device buffers plus three host integers.
 *   tiles: device, uint8 [B][Hkv][max_tokens / 32][record]: the quantized part. Tile j of slice (b, h) holds
 *     quantized tokens 32 j .. 32 j + 31 as one record. 2-bit: a 3072-byte record
 *       bytes    0..1023  key codes,   256 little-endian uint32 words (16 two-bit codes each)
 *       bytes 1024..2047  value codes, 256 uint32 words
 *       bytes 2048..2303  key scale s_K[c] (fp16, c = 0..127; one per channel of the tile)
 *       bytes 2304..2559  key zero  z_K[c] (fp16)
 *       bytes 2560..2815  value scale s_V[g][t] (fp16 at index 32 g + t; g = channel group 0..3, t = token 0..31)
 *       bytes 2816..3071  value zero  z_V[g][t] (fp16)
 *     Key code of token t, channel c: word 4 (t%16 + 16 ((c%32)/8)) + 2 (t/16) + (c/32)/2,
 *       bit 4 (c%8) + 2 ((c/32)%2).
 *     Value code of channel c, token t: with (kc, e) = (t/4, t%4) for t < 16 and ((t-16)/4, 4 + (t-16)%4) otherwise,
 *       word 4 (c%16 + 16 kc) + (c/16)/2, bit 4 e + 2 ((c/16)%2).
 *     Decoding: x = code * s + z.
 *     2-bit with KVQ_FLAG_SPARSE: a 3840-byte record, the 3072 bytes above followed by the outlier section laid out
 *     as in the 4-bit one (bytes 3072..3327 o_K[c], 3328..3455 its token, 3456..3711 o_V[g][t] at 32 g + t,
 *     3712..3839 its channel within group g); the outlier's code is 0 and it decodes as o.
 *     4-bit: a 5120-byte record (a library layout; the pages fix only the code width)
 *       bytes    0..2047  key codes,   512 little-endian uint32 words (8 four-bit codes each)
 *       bytes 2048..4095  value codes, 512 words
 *       bytes 4096..4351  key scale s_K[c];  4352..4607 key zero z_K[c]
 *       bytes 4608..4863  value scale s_V[g][t] (index 32 g + t);  4864..5119 value zero z_V[g][t]
 *     Key code of token t, channel c: word 8 (c/8 + 16 (t/8)) + t%8, bit 4 (c%8).
 *     Value code of channel c, token t: word 4 c + t/8, bit 4 (t%8).
 *     4-bit with KVQ_FLAG_SPARSE: a 5888-byte record, the 5120 bytes above followed by
 *       bytes 5120..5375  key outlier o_K[c] (fp16, one per channel);  5376..5503 its token t (uint8, 0..31)
 *       bytes 5504..5759  value outlier o_V[g][t] (fp16, index 32 g + t);  5760..5887 its channel within group g
 *                         (uint8 at 5760 + 32 g + t, 0..31)
 *     the outlier's code is 0 and it decodes as o instead of code * s + z.
 *   k_res, v_res: device, fp16 [B][Hkv][R][128]: the residual window; rows 0 .. n_resid-1 hold the newest tokens
 *     exactly as appended.
 *   n_quant (host): tokens in the quantized part (a multiple of 32). n_resid (host): tokens in the window (0..R).
 *   n_sink (host): 1 once the sink holds token 0 (KVQ_FLAG_SINK), else 0. The cache then holds
 *     n_sink + n_quant + n_resid tokens, in that order.
 *   sink: device, uint8 [B][Hkv][512], required with KVQ_FLAG_SINK (else ignored): bytes 0..255 the fp16 key of
 *     token 0; bytes 256..319 its value codes (channel c at byte 256 + c/2, bit 4 (c%2)); bytes 320..327 value scales
 *     s_V[g] and 328..335 value zeros z_V[g] (fp16, g = 0..3); bytes 336..511 zero. With KVQ_FLAG_SPARSE: bytes
 *     336..343 the value outliers o_V[g] (fp16) and 344..347 their channels within the group (uint8); 348..511
 *     zero.
 * A new cache starts with n_quant = n_resid = n_sink = 0.
 */
typedef struct kvq_cache {
    void *tiles;
    void *k_res;
    void *v_res;
    int64_t n_quant;
    int32_t n_resid;
    int32_t n_sink;
    void *sink;
} kvq_cache;

/*
 * Per-channel key quantization (KIVI page, paragraph on the cache contents: each key group is 32 tokens of one
 * channel; asymmetric min/max form).
 *   k: device fp16, element (b, h, t, c) at k[b*stride_b + h*stride_h + t*stride_t + c], t in [0, n_tokens).
 *   n_tokens: a positive multiple of 32. tile0: first destination tile index (tokens 32*tile0 ...).
 *   tiles: device, the tile array of a cache of this shape; for tiles tile0 .. tile0 + n_tokens/32 - 1 of every
 *     slice, the key codes and key scale/zero fields are written; the value fields are left untouched.
 * Per group (32 tokens of one channel), with x the fp16 inputs and L = 2^bits - 1 (3 or 15):
 *   r = RN32(max - min); s = RN16(RN32(r / L)); if (L + 1/2) * s < r then s = next binary16 above s;
 *   z = min (a zero minimum stored as +0); code = 0 if s == 0, else
 *   clamp(round_half_even(RN32(RN32(x - z) / s)), 0, L); RN32/RN16 = round to nearest even into binary32/binary16,
 *   division correctly rounded. With KVQ_FLAG_SPARSE, min and max run over the group without its outlier, whose
 *   value and index fill the record's outlier fields (also written).
 * Errors: KVQ_E_NULL, KVQ_E_SHAPE, KVQ_E_BITS, KVQ_E_ALIGN, KVQ_E_CAPACITY (tile range beyond max_tokens/32),
 *   KVQ_E_LAUNCH.
 */
KVQ_API int kv_quant_keys_per_channel(const kvq_shape *shape, const void *k, int64_t stride_b, int64_t stride_h,
                              int64_t stride_t, int64_t n_tokens, int64_t tile0, void *tiles, void *stream);

/*
 * Per-token value quantization (KIVI page and synthetic.wiki "Keys are harder than values": values grouped per
 * token; 32 channels per group, four groups per token). Same quantizer and arguments as
 * kv_quant_keys_per_channel; writes the value codes and value scale/zero fields of the tiles only.
 */
KVQ_API int kv_quant_values_per_token(const kvq_shape *shape, const void *v, int64_t stride_b, int64_t stride_h,
                              int64_t stride_t, int64_t n_tokens, int64_t tile0, void *tiles, void *stream);

/*
 * Append n_tokens new tokens to every slice and manage the residual window (KIVI page, paragraph on the
 * recent-token window). The result equals n_tokens single appends, each of which first flushes a full window
 * (quantizing its R tokens into R/32 tiles, keys per channel and values per token) and then stores the token:
 *   F = R * floor((n_resid + n_tokens - 1) / R) tokens are flushed: the first F of (window, new tokens);
 *   the remaining tokens become the window.
 *   With KVQ_FLAG_SINK and n_sink = 0, the first new token is written to the sink record instead (n_sink becomes 1)
 *   and the rule above applies to the other n_tokens - 1 tokens.
 *   k_new, v_new: device fp16 with the same stride convention as kv_quant_keys_per_channel; n_tokens >= 1.
 *   cache: host struct; on success cache->n_quant and cache->n_resid are updated at enqueue time.
 * Errors: KVQ_E_NULL, KVQ_E_SHAPE, KVQ_E_BITS, KVQ_E_ALIGN, KVQ_E_STATE, KVQ_E_CAPACITY (n_quant + F > max_tokens),
 *   KVQ_E_LAUNCH.
 */
KVQ_API int kv_append_and_flush(const kvq_shape *shape, kvq_cache *cache, const void *k_new, const void *v_new,
                        int64_t stride_b, int64_t stride_h, int64_t stride_t, int64_t n_tokens, void *stream);

/*
 * Number of token splits kv_decode_attention uses for the cache's current length (split-K along tokens; each
 * split covers a contiguous range of 32-token tiles, the residual window being the last tiles; the sink token goes
 * with the first split), and the workspace
 * it needs: batch * q_heads * splits * (128 + 2) * 4 bytes. Return 0 when the arguments are invalid.
 */
KVQ_API int32_t kv_decode_attention_splits(const kvq_shape *shape, const kvq_cache *cache);
KVQ_API size_t kv_decode_attention_workspace_bytes(const kvq_shape *shape, const kvq_cache *cache);

/*
 * Decode attention of one query per (batch row, query head) over the whole cache: grouped part and residual
 * window (synthetic.wiki "Keys are harder than values", last bullet). For query head hq of batch row b, with
 * KV head h = hq / (Hq / Hkv) and decoded keys/values K, V (codes * scale + zero; window tokens as stored):
 *   out[b][hq][c] = sum_t softmax_t(sm_scale * q . K[t]) V[t][c],
 * over the sink token (if any), the quantized part and the window. With KVQ_FLAG_PRE_ROPE, K[t] is the decoded key
 * rotated by its absolute position (see kvq_shape).
 *   q: device fp16 [B][Hq][128], contiguous. sm_scale: softmax scale; a value <= 0 selects 1/sqrt(128).
 *   out: device fp32 [B][Hq][128], contiguous.
 *   workspace: device, >= kv_decode_attention_workspace_bytes(shape, cache) bytes, 16-byte aligned (split
 *     partials: maximum, exponent sum and unnormalized output per split, merged by a second kernel).
 * Errors: KVQ_E_NULL, KVQ_E_SHAPE, KVQ_E_BITS, KVQ_E_ALIGN, KVQ_E_STATE, KVQ_E_EMPTY, KVQ_E_WORKSPACE,
 *   KVQ_E_LAUNCH.
 */
KVQ_API int kv_decode_attention(const kvq_shape *shape, const kvq_cache *cache, const void *q, float sm_scale, float *out,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * kv_decode_attention without a workspace argument and without any allocation, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * definition, arguments, kernels and results as kv_decode_attention (bit for bit), except that the split partials
 * live in a static device array of KVQ_NOALLOC_SCRATCH_BYTES (16 MiB) that the library holds on every GPU it runs
 * on until the process ends. The call allocates and frees nothing; on the first call on a device it looks up that
 * device's copy of the array (hipGetSymbolAddress, with that device current) and keeps the address.
 *   Every call on one GPU shares that GPU's array: calls that overlap on one GPU (on different streams, or from
 *   several host threads without ordering) race and give undefined outputs. Issue them on one stream, in order.
 *   Nothing in the array needs to start at zero: every partial a call reads was written earlier in the same call.
 *   Limit: batch * q_heads * splits * 520 bytes <= KVQ_NOALLOC_SCRATCH_BYTES, with splits as returned by
 *   kv_decode_attention_splits (e.g. 64 sequences x 32 query heads x 8 splits = 8.5 MB at 32K tokens).
 * Errors: as kv_decode_attention (without KVQ_E_WORKSPACE); KVQ_E_SCRATCH when the limit is exceeded (checked on
 *   the host before any runtime call); KVQ_E_LAUNCH also when the array's address cannot be obtained.
 */
KVQ_API int kv_decode_attention_noalloc(const kvq_shape *shape, const kvq_cache *cache, const void *q, float sm_scale,
                                        float *out, void *stream);

/*
 * Ragged caches: every sequence (batch row) at its own length, the lengths held in device memory, so a whole
 * decode step is enqueued with fixed arguments and can be captured once in a HIP graph and replayed (no host state
 * changes between steps). Serving batches hold sequences at different positions; the pages' per-sequence cache
 * (KIVI page, paragraph on the recent-token window) is applied to each sequence on its own. 2-bit caches only
 * (bits = 2, flags = 0; otherwise KVQ_E_BITS).
 *   tiles, k_res, v_res: as in kvq_cache; sink: unused (may be NULL).
 *   lens: device int32 [B][4], 16-byte aligned: {n_quant, n_resid, n_sink (0), status} of sequence b. A new cache
 *     has all zeros. status 1 marks a sequence whose flush did not fit max_tokens: its appends are refused from then
 *     on and its lengths stay, until it is prefilled again.
 *   sync: device uint32 [kv_ragged_sync_words(shape)], 4-byte aligned, all zero when the cache is created; used by
 *     kv_ragged_decode_step only (completion counters inside its single launch), which leaves it zero again.
 *     Required by kv_ragged_decode_step (KVQ_E_NULL), ignored by the other calls.
 * Window blocks are quantized ahead: whenever sequence b's window holds a complete 32-row block k, tile
 * n_quant / 32 + k (if below max_tokens / 32) already holds that block's record, written by the call that completed
 * the block (kv_ragged_prefill, kv_ragged_append or kv_ragged_decode_step). These are the bytes a flush writes, so a
 * flush in kv_ragged_decode_step only moves the lengths. The cache state (tiles, window rows, lens) must therefore be
 * changed through these calls only.
 * Calls on one ragged cache must be issued on one stream, in order.
 */
typedef struct kvq_ragged {
    void *tiles;
    void *k_res;
    void *v_res;
    void *sink;
    int32_t *lens;
    uint32_t *sync;
} kvq_ragged;

/* Words of kvq_ragged.sync: B * (1 + Hkv * ceil((Hq / Hkv) / 4)). 0 on invalid arguments. */
KVQ_API size_t kv_ragged_sync_words(const kvq_shape *shape);

/*
 * Replaces sequence b's contents with n_tokens tokens (n_tokens >= 0; 0 empties it): k, v fp16 [Hkv][n_tokens][128]
 * with element strides stride_h, stride_t (16-byte aligned rows). Same state as n_tokens single appends to an empty
 * sequence (KIVI page, paragraph on the recent-token window); writes lens[b] = {flushed, n_tokens - flushed, 0, 0}
 * and the records of the window's complete blocks (written ahead, as above). Other sequences are untouched.
 * Errors: KVQ_E_NULL, KVQ_E_SHAPE (b outside [0, B), n_tokens < 0), KVQ_E_BITS, KVQ_E_ALIGN, KVQ_E_CAPACITY
 *   (flushed tokens > max_tokens), KVQ_E_LAUNCH.
 */
KVQ_API int kv_ragged_prefill(const kvq_shape *shape, const kvq_ragged *cache, int32_t b, const void *k,
                              const void *v, int64_t stride_h, int64_t stride_t, int64_t n_tokens, void *stream);

/*
 * Appends one token to every sequence: k_new, v_new fp16 [B][Hkv][128] with element strides stride_b, stride_h.
 * Per sequence on the device: a full window is first quantized into R/32 tiles (lazy flush), then the token is
 * stored; equals kv_append_and_flush with one token applied to each sequence at its own length. A token that
 * completes a window block also gets that block's record written ahead.
 * Errors: KVQ_E_NULL, KVQ_E_SHAPE, KVQ_E_BITS, KVQ_E_ALIGN, KVQ_E_LAUNCH.
 */
KVQ_API int kv_ragged_append(const kvq_shape *shape, const kvq_ragged *cache, const void *k_new, const void *v_new,
                             int64_t stride_b, int64_t stride_h, void *stream);

/* Splits and workspace of the ragged decode calls: fixed by the capacity (max_tokens + R per sequence), so one
 * workspace serves every step; workspace = B * q_heads * splits * (128 + 2) * 4 bytes. 0 on invalid arguments. */
KVQ_API int32_t kv_ragged_splits(const kvq_shape *shape);
KVQ_API size_t kv_ragged_workspace_bytes(const kvq_shape *shape);

/*
 * Decode attention of one query per (sequence, query head) over that sequence's tokens (same definition and
 * arguments as kv_decode_attention). A sequence that holds no token gets zeros.
 * Errors: KVQ_E_NULL, KVQ_E_SHAPE, KVQ_E_BITS, KVQ_E_ALIGN, KVQ_E_WORKSPACE, KVQ_E_LAUNCH.
 */
KVQ_API int kv_ragged_decode_attention(const kvq_shape *shape, const kvq_ragged *cache, const void *q,
                                       float sm_scale, float *out, void *workspace, size_t workspace_bytes,
                                       void *stream);

/*
 * One decode step: the result of kv_ragged_append(k_new, v_new) then kv_ragged_decode_attention(q), bit for bit, in a
 * single launch (KIVI page, paragraphs on the recent-token window and on decoding from the grouped and residual
 * parts). Every workgroup derives its sequence's step from the lengths before it; a flushed window's tiles were
 * written ahead, so the flush only moves the lengths; a token that completes a window block has that block's record
 * written ahead by a workgroup running beside the attention; the new token is attended from k_new/v_new; the last
 * split of each (sequence, KV head, chunk of four query heads) merges the splits, and the last of a sequence writes
 * the new window rows and lengths (counted in cache->sync, left zero). k_new, v_new must not alias the cache.
 * Errors: as kv_ragged_append and kv_ragged_decode_attention; KVQ_E_NULL without cache->sync.
 */
KVQ_API int kv_ragged_decode_step(const kvq_shape *shape, const kvq_ragged *cache, const void *k_new,
                                  const void *v_new, int64_t stride_b, int64_t stride_h, const void *q,
                                  float sm_scale, float *out, void *workspace, size_t workspace_bytes, void *stream);

/* Human-readable name of a status code (static string, never NULL). */
KVQ_API const char *kvq_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
