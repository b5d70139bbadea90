// HIP kernels for gfx950 (CDNA4): KIVI-style 2-bit KV-cache quantization, residual-window append, and split-K
// decode attention computed from the packed codes. Host entry points live in kvq_api.hip.
//
// Sources: KIVI page (fdeinterviews.com, "KIVI: A Tuning-Free Asymmetric 2bit Quantization for KV Cache"),
// paragraphs on the cache contents (per-channel key groups of 32 tokens, per-token values) and on the recent-token
// window (R = 128 newest tokens in full precision, quantized in blocks); synthetic.wiki "KV cache quantization",
// section "Keys are harder than values" (grouped + residual key parts combined when computing scores).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_kernels.h"
#include "kvq_quantizer.h"
#include "kvq_lanes.h"

namespace kvq {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Every byte of the cache is read once per decode call: the loads of tile records and fp16 window rows carry the
// non-temporal hint. On MI355X a plain streaming read of a 1.6 GB buffer runs at 6.0-6.2 TB/s and the same read
// with non-temporal loads at 6.9-7.1 TB/s. 16 bytes at p + 16 * i.
__device__ __forceinline__ uint4 load_stream(const void *p, int i) {
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p) + i));
}

constexpr int D = 128;
constexpr int REC = 3072;
// dense-and-sparse records: the 3072 bytes above, then the outlier section (key outliers per channel, value outliers
// per token and group; see kvq.h)
constexpr int REC_SPARSE = 3840;
constexpr int K_OUT = 3072, K_IDX = 3328, V_OUT = 3456, V_IDX = 3712;
template <bool SPARSE>
constexpr int rec_bytes() { return SPARSE ? REC_SPARSE : REC; }

// Keys of one tile (tokens t_first .. t_first + 31 of slice (b, h)) into the record at `rec`: one workgroup of 64
// lanes; lane l owns channels 2l and 2l+1 over the tile's 32 tokens. `words` is 1 KB of LDS.
// SPARSE (dense-and-sparse groups; synthetic.wiki "KV cache quantization", section "What they report"): each
// channel's token of largest magnitude (the first on ties) is kept apart as its fp16 value and token index; min and
// max run over the other 31 tokens and the outlier's code is 0.
template <bool SPARSE = false>
__device__ __forceinline__ void quant_keys_tile(const TokSrc &src, int64_t t_first, int b, int h, uint8_t *rec,
                                                uint32_t *words) {
    const int l = threadIdx.x;

    uint32_t xw[32];   // token i: channels 2l (low half) and 2l + 1 (high half), binary16
    load_pairs32_packed(src, t_first, b, h, 2 * l, xw);
    h2v mn, mx;
    int i0 = -1, i1 = -1;   // SPARSE: the outlier tokens of channels 2l, 2l+1
    if constexpr (SPARSE) {
        uint32_t k0 = 0u, k1 = 0u;   // |x| bits (binary16 order) above 31 - token: the largest is the first maximum
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            k0 = max(k0, ((xw[i] & 0x7FFFu) << 5) | (31u - i));
            k1 = max(k1, (((xw[i] >> 16) & 0x7FFFu) << 5) | (31u - i));
        }
        i0 = 31 - (int)(k0 & 31u);
        i1 = 31 - (int)(k1 & 31u);
        // min/max over the other 31: the outlier's half takes the value of a neighbouring token of its channel
        const int r0 = i0 == 0 ? 1 : 0, r1 = i1 == 0 ? 1 : 0;
        uint32_t lo = 0u, hi = 0u;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            lo = i == r0 ? xw[i] : lo;
            hi = i == r1 ? xw[i] : hi;
        }
        mn = __builtin_bit_cast(h2v, (lo & 0xFFFFu) | (hi & 0xFFFF0000u));
        mx = mn;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const uint32_t w = (i == i0 ? (xw[i] & 0xFFFF0000u) | (lo & 0xFFFFu) : xw[i]);
            const uint32_t v = (i == i1 ? (w & 0xFFFFu) | (hi & 0xFFFF0000u) : w);
            mn = __builtin_elementwise_min(mn, __builtin_bit_cast(h2v, v));
            mx = __builtin_elementwise_max(mx, __builtin_bit_cast(h2v, v));
        }
    } else {
        minmax_pairs32(xw, mn, mx);
    }
    _Float16 s0, z0, s1, z1;
    group_params((float)mn[0], (float)mx[0], 3.0f, s0, z0);
    group_params((float)mn[1], (float)mx[1], 3.0f, s1, z1);
    const float fs0 = (float)s0, fz0 = (float)z0, fs1 = (float)s1, fz1 = (float)z1;
    // a constant group (s = 0) gets rs = 0, hence t' = 0 and code 0
    const float rs0 = fs0 > 0.0f ? __builtin_amdgcn_rcpf(fs0) : 0.0f;
    const float rs1 = fs1 > 0.0f ? __builtin_amdgcn_rcpf(fs1) : 0.0f;

    // channel c = 2l: ks = c / 32, kc = (c % 32) / 8, e = c % 8 (even, so c + 1 sits in the next nibble). The 16
    // codes of a word come from the 8 lanes 32 (ks / 2) + 16 (ks % 2) + 4 kc + 0..3: OR over the lane quad, then with
    // the other row of the row pair; lane 32 (ks / 2) + 4 kc writes the word.
    const int c = 2 * l, ks = c >> 5, kc = (c & 31) >> 3, e = c & 7;
    const int shift = 4 * e + 2 * (ks & 1);
    const bool writer = (l & 3) == 0 && (ks & 1) == 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const int m = i >> 4, n = i & 15;
        const int w = 4 * (n + 16 * kc) + 2 * m + (ks >> 1);
        uint32_t q0 = code_from_diff(diff_half<false>(xw[i], fz0), fs0, rs0, 3u);
        uint32_t q1 = code_from_diff(diff_half<true>(xw[i], fz1), fs1, rs1, 3u);
        if constexpr (SPARSE) {
            q0 = i == i0 ? 0u : q0;
            q1 = i == i1 ? 0u : q1;
        }
        const uint32_t bits = quad_or((q0 << shift) | (q1 << (shift + 4)));
        uint32_t lo, hi;
        swap16(bits, lo, hi);
        if (writer) words[w] = lo | hi;
    }
    __syncthreads();
    reinterpret_cast<uint4 *>(rec)[l] = reinterpret_cast<const uint4 *>(words)[l];
    h2 sp = {s0, s1}, zp = {z0, z1};
    reinterpret_cast<h2 *>(rec + 2048)[l] = sp;
    reinterpret_cast<h2 *>(rec + 2304)[l] = zp;
    if constexpr (SPARSE) {
        uint32_t ow = 0u;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            ow = i == i0 ? (ow & 0xFFFF0000u) | (xw[i] & 0xFFFFu) : ow;
            ow = i == i1 ? (ow & 0xFFFFu) | (xw[i] & 0xFFFF0000u) : ow;
        }
        reinterpret_cast<uint32_t *>(rec + K_OUT)[l] = ow;
        reinterpret_cast<uint16_t *>(rec + K_IDX)[l] = (uint16_t)(i0 | (i1 << 8));
    }
}

// Values of one tile into the record at `rec`. Parameters: lane l reduces the groups (token l / 4 and 16 + l / 4,
// channel group l % 4) from their own 64-byte rows (packed binary16 min/max, no cross-lane step) and stores scale,
// zero and reciprocal scale; codes: lane l owns channels 2l and 2l+1 of every token (the row g = l / 16 of lanes
// owns channel group g) and builds its code words over the tokens. LDS: `words` 1 KB, `sv`/`zv` 256 B each,
// `gp` 2 KB ({s, z, 1/s, 0} as binary32 per (token, group)).
// SPARSE: the group's outlier (largest magnitude, lowest channel on ties) is the maximum of an order key (|x| bits,
// then the lower channel, then the sign bit, which recovers the value); min/max over the other 31 elements run with
// the outlier's half replaced by the other half of its 32-bit word (an element of the same group, so the extremes
// are unchanged), and the outlier's code is 0. `ov` (256 B) and `oi` (128 B) of LDS hold the outliers [g][t].
template <bool SPARSE = false>
__device__ __forceinline__ void quant_values_tile(const TokSrc &src, int64_t t_first, int b, int h, uint8_t *rec,
                                                  uint32_t *words, _Float16 *sv, _Float16 *zv, float *gp,
                                                  _Float16 *ov = nullptr, uint8_t *oi = nullptr) {
    const int l = threadIdx.x;
    const int c = 2 * l, j = c >> 4, cc = c & 15, g = l >> 4;
    uint32_t xw[32];
    load_pairs32_packed(src, t_first, b, h, c, xw);
    const int gq = l & 3;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int tk = (l >> 2) + 16 * k;
        const uint4 *row = reinterpret_cast<const uint4 *>(tok_row(src, b, h, t_first + tk) + 32 * gq);
        uint4 r4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) r4[q] = row[q];
        if constexpr (SPARSE) {
            uint32_t kmax = 0u;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const uint32_t we = r4[e >> 2][e & 3];
                const uint32_t klo = ((we & 0x7FFFu) << 6) | ((31u - 2u * e) << 1) | ((we >> 15) & 1u);
                const uint32_t khi = (((we >> 16) & 0x7FFFu) << 6) | ((30u - 2u * e) << 1) | (we >> 31);
                kmax = max(kmax, max(klo, khi));
            }
            const uint32_t w = 31u - ((kmax >> 1) & 31u);
            const uint32_t sel = (w & 1u) ? 0x01000100u : 0x03020302u;   // both halves = the partner half
            ov[32 * gq + tk] = __builtin_bit_cast(_Float16, (uint16_t)(((kmax >> 6) & 0x7FFFu) | ((kmax & 1u) << 15)));
            oi[32 * gq + tk] = (uint8_t)w;
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if ((uint32_t)e == (w >> 1)) r4[e >> 2][e & 3] = __builtin_amdgcn_perm(r4[e >> 2][e & 3], r4[e >> 2][e & 3], sel);
        }
        h2v mn = __builtin_bit_cast(h2v, r4[0].x), mx = mn;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int e = (q == 0 ? 1 : 0); e < 4; ++e) {
                const h2v v = __builtin_bit_cast(h2v, r4[q][e]);
                mn = __builtin_elementwise_min(mn, v);
                mx = __builtin_elementwise_max(mx, v);
            }
        }
        _Float16 sh, zh;
        group_params((float)__builtin_fminf16(mn[0], mn[1]), (float)__builtin_fmaxf16(mx[0], mx[1]), 3.0f, sh, zh);
        sv[32 * gq + tk] = sh;
        zv[32 * gq + tk] = zh;
        const float fs = (float)sh;
        reinterpret_cast<f4 *>(gp)[4 * tk + gq] = f4{fs, (float)zh, fs > 0.0f ? __builtin_amdgcn_rcpf(fs) : 0.0f, 0.0f};
    }
    __syncthreads();
    // lane l's channels fill words 4 (cc + 16 kc) + j / 2 (channel 2l) and the next-but-three (channel 2l + 1) for
    // kc = 0..3, built in registers over the tokens; lane l ^ 8 fills the other half of each word
    uint32_t wv[4][2] = {{0u, 0u}, {0u, 0u}, {0u, 0u}, {0u, 0u}};
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const f4 prm = reinterpret_cast<const f4 *>(gp)[4 * i + g];
        int kc, e;
        if (i < 16) { kc = i >> 2; e = i & 3; } else { kc = (i - 16) >> 2; e = 4 + ((i - 16) & 3); }
        const int shift = 4 * e + 2 * (j & 1);
        uint32_t q0 = code_from_diff(diff_half<false>(xw[i], prm[1]), prm[0], prm[2], 3u);
        uint32_t q1 = code_from_diff(diff_half<true>(xw[i], prm[1]), prm[0], prm[2], 3u);
        if constexpr (SPARSE) {
            const uint32_t oc = oi[32 * g + i], c0 = 2 * (l & 15);
            q0 = oc == c0 ? 0u : q0;
            q1 = oc == c0 + 1 ? 0u : q1;
        }
        wv[kc][0] |= q0 << shift;
        wv[kc][1] |= q1 << shift;
    }
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const uint32_t word = dpp_xor_or<DPP_ROW_ROR8>(wv[kc][q]);
            if ((j & 1) == 0) words[4 * (cc + q + 16 * kc) + (j >> 1)] = word;
        }
    }
    __syncthreads();
    reinterpret_cast<uint4 *>(rec + 1024)[l] = reinterpret_cast<const uint4 *>(words)[l];
    reinterpret_cast<uint32_t *>(rec + 2560)[l] = reinterpret_cast<const uint32_t *>(sv)[l];
    reinterpret_cast<uint32_t *>(rec + 2816)[l] = reinterpret_cast<const uint32_t *>(zv)[l];
    if constexpr (SPARSE) {
        reinterpret_cast<uint32_t *>(rec + V_OUT)[l] = reinterpret_cast<const uint32_t *>(ov)[l];
        reinterpret_cast<uint16_t *>(rec + V_IDX)[l] = reinterpret_cast<const uint16_t *>(oi)[l];
    }
}

template <bool SPARSE>
__global__ __launch_bounds__(64) void quant_keys_kernel(TokSrc src, int64_t t_begin, int kv_heads, uint8_t *tiles,
                                                        int64_t max_tiles, int64_t tile0) {
    __shared__ uint32_t words[256];
    const int64_t tile = blockIdx.x;
    const int h = blockIdx.y, b = blockIdx.z;
    uint8_t *rec = tiles + ((int64_t)(b * kv_heads + h) * max_tiles + tile0 + tile) * rec_bytes<SPARSE>();
    quant_keys_tile<SPARSE>(src, t_begin + tile * 32, b, h, rec, words);
}

// five wavefronts per SIMD (85 registers): a memory-bound kernel whose loads want more wavefronts in flight (the
// outlier search of dense-and-sparse groups needs more registers: four)
template <bool SPARSE>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(SPARSE ? 4 : 5))) void quant_values_kernel(TokSrc src, int64_t t_begin, int kv_heads,
                                                          uint8_t *tiles, int64_t max_tiles, int64_t tile0) {
    __shared__ uint32_t words[256];
    __shared__ _Float16 sv[128], zv[128];
    __shared__ __align__(16) float gp[512];
    __shared__ __align__(16) _Float16 ov[SPARSE ? 128 : 1];
    __shared__ __align__(16) uint8_t oi[SPARSE ? 128 : 1];
    const int64_t tile = blockIdx.x;
    const int h = blockIdx.y, b = blockIdx.z;
    uint8_t *rec = tiles + ((int64_t)(b * kv_heads + h) * max_tiles + tile0 + tile) * rec_bytes<SPARSE>();
    quant_values_tile<SPARSE>(src, t_begin + tile * 32, b, h, rec, words, sv, zv, gp, ov, oi);
}

// ------------------------------------------------------------------------------------------------ window append
// Copies n tokens (source tokens t_begin ..) of every slice's keys and values into window rows dst0 .. ; 16 lanes
// move one 256-byte key row and the matching value row, a workgroup of 64 lanes moves 4 rows of each.
__global__ __launch_bounds__(64) void copy_rows_kernel(TokSrc ksrc, TokSrc vsrc, int64_t t_begin, int64_t n,
                                                       int kv_heads, _Float16 *kres, _Float16 *vres, int res_cap,
                                                       int dst0) {
    const int l = threadIdx.x;
    const int64_t r = blockIdx.x * 4 + (l >> 4);
    const int h = blockIdx.y, b = blockIdx.z;
    if (r >= n) return;
    const uint4 kw = reinterpret_cast<const uint4 *>(tok_row(ksrc, b, h, t_begin + r))[l & 15];
    const uint4 vw = reinterpret_cast<const uint4 *>(tok_row(vsrc, b, h, t_begin + r))[l & 15];
    const int64_t dst = ((int64_t)(b * kv_heads + h) * res_cap + dst0 + r) * D;
    reinterpret_cast<uint4 *>(kres + dst)[l & 15] = kw;
    reinterpret_cast<uint4 *>(vres + dst)[l & 15] = vw;
}

// ------------------------------------------------------------------------------------------------ ragged caches
// Per-sequence state in device memory, lens[b] = {n_quant, n_resid, n_sink, status}. status 1 (sticky until the
// sequence is prefilled again) marks a sequence whose flush did not fit the tile capacity: its appends are refused
// and its lengths stay. Effective state after appending one token: a full window is flushed (R tokens more in the
// quantized part), then the token opens or extends the window.
__device__ __forceinline__ void ragged_after_append(const int32_t *ln, int res_cap, int &nq, int &nr) {
    nq = ln[0];
    nr = ln[1];
    if (ln[3] != 0) return;
    if (nr == res_cap) {
        nq += nr;
        nr = 1;
    } else {
        nr += 1;
    }
}

// Window blocks of a ragged cache are quantized ahead: whenever a window holds a complete 32-row block k, tile
// n_quant / 32 + k (when it is within the capacity) already holds that block's record, written by the call that
// completed the block (prefill, append or decode step). A flush then only moves the lengths in the single-launch
// decode step; the records are the same bytes a quantization at flush time writes.
__device__ __forceinline__ TokSrc window_then_new(const _Float16 *res, int kv_heads, int res_cap, int row,
                                                   const _Float16 *nw, int64_t new_sb, int64_t new_sh) {
    TokSrc s;   // rows below `row` from the window, row `row` from the new token
    s.a = res; s.a_sb = (int64_t)kv_heads * res_cap * D; s.a_sh = (int64_t)res_cap * D; s.a_st = D; s.n_a = row;
    s.b = nw; s.b_sb = new_sb; s.b_sh = new_sh; s.b_st = 0;
    return s;
}

// Quantizes the window block that ends with the token appended at window row `row` (row % 32 == 31) into tile
// `slot` of slice (b, h). LDS: 4 KB.
__device__ __forceinline__ void quant_window_block(const _Float16 *k_res, const _Float16 *v_res, const _Float16 *k_new,
                                                   const _Float16 *v_new, int64_t new_sb, int64_t new_sh,
                                                   int kv_heads, int res_cap, int row, int b, int h, uint8_t *tiles,
                                                   int64_t max_tiles, int64_t slot, unsigned char *lds) {
    const TokSrc wk = window_then_new(k_res, kv_heads, res_cap, row, k_new, new_sb, new_sh);
    const TokSrc wv = window_then_new(v_res, kv_heads, res_cap, row, v_new, new_sb, new_sh);
    uint32_t *words = reinterpret_cast<uint32_t *>(lds);
    _Float16 *sv = reinterpret_cast<_Float16 *>(lds + 1024), *zv = sv + 128;
    float *gp = reinterpret_cast<float *>(lds + 2048);
    uint8_t *rec = tiles + (((int64_t)b * kv_heads + h) * max_tiles + slot) * REC;
    quant_keys_tile(wk, row - 31, b, h, rec, words);
    __syncthreads();
    quant_values_tile(wv, row - 31, b, h, rec, words, sv, zv, gp);
    __syncthreads();
}

// One decode-step append for every sequence: workgroup (i, h, b) quantizes window tile i of slice (b, h) into tile
// n_quant / 32 + i when the window is full (lazy flush), and workgroup (0, h, b) then copies the new token into
// window row n_resid (row 0 after a flush, once its own tile's reads are done; the other tiles never read row 0).
// When the token completes a window block, the last workgroup writes that block's record ahead.
__global__ __launch_bounds__(64) void ragged_flush_append_kernel(TokSrc knew, TokSrc vnew, int kv_heads,
                                                                 uint8_t *tiles, int64_t max_tiles, _Float16 *k_res,
                                                                 _Float16 *v_res, int res_cap, int32_t *lens) {
    __shared__ __align__(16) unsigned char lds[4096];   // words 1 KB, sv and zv 256 B each, gp 2 KB (from 2048)
    uint32_t *words = reinterpret_cast<uint32_t *>(lds);
    _Float16 *sv = reinterpret_cast<_Float16 *>(lds + 1024), *zv = sv + 128;
    float *gp = reinterpret_cast<float *>(lds + 2048);
    const int l = threadIdx.x;
    const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    int32_t *ln = lens + 4 * b;
    const int nq = ln[0], nr = ln[1];
    const bool flush = nr == res_cap;
    if (ln[3] != 0) return;   // full sequence: appends refused
    if (flush && (int64_t)nq + res_cap > max_tiles * 32) {   // no room for the flushed tiles: refuse the token
        if (i == 0 && h == 0 && l == 0) ln[3] = 1;           // (workgroups reading 1 here also return)
        return;
    }
    if (flush) {
        TokSrc wk;
        wk.a = k_res; wk.a_sb = (int64_t)kv_heads * res_cap * D; wk.a_sh = (int64_t)res_cap * D; wk.a_st = D;
        wk.n_a = INT64_MAX;
        wk.b = wk.a; wk.b_sb = wk.a_sb; wk.b_sh = wk.a_sh; wk.b_st = wk.a_st;
        TokSrc wv = wk;
        wv.a = v_res; wv.b = v_res;
        uint8_t *rec = tiles + ((int64_t)(b * kv_heads + h) * max_tiles + nq / 32 + i) * REC;
        quant_keys_tile(wk, 32 * i, b, h, rec, words);
        quant_values_tile(wv, 32 * i, b, h, rec, words, sv, zv, gp);
        __syncthreads();
    }
    const int row = flush ? 0 : nr;
    if (i == 0) {
        const int64_t dst = ((int64_t)(b * kv_heads + h) * res_cap + row) * D;
        reinterpret_cast<uint32_t *>(k_res + dst)[l] = reinterpret_cast<const uint32_t *>(tok_row(knew, b, h, 0))[l];
        reinterpret_cast<uint32_t *>(v_res + dst)[l] = reinterpret_cast<const uint32_t *>(tok_row(vnew, b, h, 0))[l];
    }
    // (a flush leaves row 0, so a completed block is never one of a flush; rows below `row` are not written here)
    if (i == (int)gridDim.x - 1 && (row & 31) == 31) {
        const int64_t slot = nq / 32 + row / 32;
        if (slot < max_tiles)
            quant_window_block(k_res, v_res, knew.a, vnew.a, knew.a_sb, knew.a_sh, kv_heads, res_cap, row, b, h, tiles,
                               max_tiles, slot, lds);
    }
}

// Makes the append of the last ragged_flush_append_kernel visible in the lengths.
__global__ __launch_bounds__(256) void ragged_commit_kernel(int32_t *lens, int batch, int res_cap) {
    for (int b = blockIdx.x * blockDim.x + threadIdx.x; b < batch; b += gridDim.x * blockDim.x) {
        int32_t *ln = lens + 4 * b;
        int nq, nr;
        ragged_after_append(ln, res_cap, nq, nr);
        ln[0] = nq;
        ln[1] = nr;
    }
}

// Sets the lengths of sequence b (after a prefill of that sequence alone).
__global__ void ragged_set_kernel(int32_t *lens, int b, int nq, int nr, int ns) {
    int32_t *ln = lens + 4 * b;
    ln[0] = nq;
    ln[1] = nr;
    ln[2] = ns;
    ln[3] = 0;
}

// ------------------------------------------------------------------------------------------------ decode pass 1
// Expand eight packed 2-bit codes into eight fp16 values. `nib` holds one code in the low two bits of each nibble
// (upper two bits zero); the gfx950 fp4 (e2m1) converter reads nibble 00cc as c/2, the scale 2 makes it c.
__device__ __forceinline__ h8 expand8(uint32_t nib) {
    h2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib, 2.0f, 0);
    h2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib, 2.0f, 1);
    h2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib, 2.0f, 2);
    h2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib, 2.0f, 3);
    h8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
    return r;
}

__device__ __forceinline__ uint32_t nibbles(uint32_t w, int parity) {
    return (parity ? (w >> 2) : w) & 0x33333333u;
}

// 2^k for -126 <= k <= 127
__device__ __forceinline__ float pow2(int k) { return __builtin_bit_cast(float, (uint32_t)(127 + k) << 23); }

__device__ __forceinline__ f4 mfma(h8 a, h8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }

// x = (pa * s.lo, pb * s.hi) for an fp32 pair (pa, pb) and a packed fp16 pair s: hi = RN16(x), lo = RN16(x - hi),
// packed. x is formed in binary32 (one mixed-precision fma each, one rounding), its high parts by one packed
// conversion, the exact remainders x - hi by mixed fmas that read hi's halves, the low parts by a second packed
// conversion: six instructions at the full vector rate (fp16-destination mixed fmas, which would write the halves
// directly, issue at about half that rate). hi + lo is x to within 2^-22 |x|.
__device__ __forceinline__ void split_pair(float pa, float pb, uint32_t s, uint32_t &hi, uint32_t &lo) {
    float x0, x1;
    asm("v_fma_mix_f32 %2, %4, %6, 0 op_sel_hi:[0,1,0]\n\t"
        "v_fma_mix_f32 %3, %5, %6, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]\n\t"
        "v_cvt_pk_f16_f32 %0, %2, %3\n\t"
        "v_fma_mix_f32 %2, -%0, 1.0, %2 op_sel_hi:[1,0,0]\n\t"
        "v_fma_mix_f32 %3, -%0, 1.0, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
        "v_cvt_pk_f16_f32 %1, %2, %3"
        : "=&v"(hi), "=&v"(lo), "=&v"(x0), "=&v"(x1)
        : "v"(pa), "v"(pb), "v"(s));
}

// gfx950 LDS transpose read of 16-bit elements: within each 16-lane row, lane i receives element i % 4 of the 8-byte
// chunks read by lanes i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4 (in that order)
typedef short s4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ h4 read_tr16(const _Float16 *lds) {
    return __builtin_bit_cast(h4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4 *)lds));
}

constexpr int PASS2_MAX_SPLITS = 1024;

// Device-coherent access to split partials that another workgroup of the same launch reads (device-scope relaxed
// atomics: the store writes through to the device's point of coherence, the load reads from it).
__device__ __forceinline__ void coherent_store(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_load(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The merge of one (batch row, query head) row bh by one wavefront; `wts` is LDS for `splits` floats. With
// zero_empty, a row with no token (every split empty) gets zeros. COHERENT: the partials were written in this launch
// (read through coherent loads). Splits past the first eight are loaded BATCH at a time, one memory round trip per
// batch (the last batch rereads the last split). `wts` holds max(8, BATCH) zero weights after the last split, so
// every weight read is unconditional and the reads of a batch are contiguous.
template <bool COHERENT = false, int BATCH = 8>
__device__ __forceinline__ void merge_splits(const float *part_o, const float *part_ml, float *out, int splits,
                                             int64_t bh, float *wts, bool zero_empty) {
    auto ld = [](const float *p) { return COHERENT ? coherent_load(p) : *p; };
    const int l = threadIdx.x;
    const float *pm = part_ml + bh * splits * 2;
    const float2 *po = reinterpret_cast<const float2 *>(part_o + bh * splits * D) + l;
    auto ld2 = [&](int k) -> float2 {
        if constexpr (COHERENT) {
            const float *f = reinterpret_cast<const float *>(po + k * (D / 2));
            return float2{coherent_load(f), coherent_load(f + 1)};
        } else {
            return po[k * (D / 2)];
        }
    };
    // the first eight splits' partial outputs are loaded together with the (m, l) pairs (one memory round trip
    // for up to eight splits)
    float2 first[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) first[k] = k < splits ? ld2(k) : float2{0.0f, 0.0f};
    const float NEG_INF = -__builtin_inff();
    float M = NEG_INF;
    for (int sp = l; sp < splits; sp += 64) M = fmaxf(M, ld(pm + 2 * sp));
    M = rows_max(row16_max(M));
    float L = 0.0f;
    for (int sp = l; sp < splits; sp += 64) {
        const float ms = ld(pm + 2 * sp);
        const float w = (ms == NEG_INF) ? 0.0f : __builtin_amdgcn_exp2f(ms - M);
        wts[sp] = w;
        L += w * ld(pm + 2 * sp + 1);
    }
    constexpr int PAD = BATCH > 8 ? BATCH : 8;
    if (l < PAD) wts[splits + l] = 0.0f;
    L = rows_sum(row16_sum(L));
    __syncthreads();
    if (zero_empty && !(L > 0.0f)) {
        reinterpret_cast<float2 *>(out + bh * D)[l] = float2{0.0f, 0.0f};
        return;
    }
    float o0 = 0.0f, o1 = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {   // weights past the last split are 0 (and so are those partials)
        const float w = wts[k];
        o0 = fmaf(w, first[k].x, o0);
        o1 = fmaf(w, first[k].y, o1);
    }
    for (int sp = 8; sp < splits; sp += BATCH) {   // the last batch: loads clamped to the last split, weights 0
        float2 v[BATCH];
#pragma unroll
        for (int k = 0; k < BATCH; ++k) v[k] = ld2(min(sp + k, splits - 1));
#pragma unroll
        for (int k = 0; k < BATCH; ++k) {
            const float w = wts[sp + k];
            o0 = fmaf(w, v[k].x, o0);
            o1 = fmaf(w, v[k].y, o1);
        }
    }
    reinterpret_cast<float2 *>(out + bh * D)[l] = float2{o0 / L, o1 / L};
}

// One wavefront per (split, batch row, KV head, chunk of up to 4 query heads of that KV head); lane l = n + 16 kc.
//
// Scores. The query with the tile's key scales folded in, q~[h][c] = q'[h][c] s_K[c], is split into an fp16 high
// part and an fp16 low part (q' = q 2^-E_h with |q'| < 1, so both stay in range for any fp16 scale). One
// 16x16x32 fp16 MFMA per (16-token block, 32-channel block) takes A = q~ with row m = 4 h + r carrying the high
// part of head h for even r and the low part for odd r, and B = the key codes (exact small integers, expanded
// from the packed 2-bit words with the gfx950 fp4 converter), column = token. Output lane (t, kc) then holds head
// kc's high-part and low-part sums for token t in its first two accumulator registers: one add gives the score,
// and each lane owns the scores of exactly one (head, token) pair per block, two per tile. The accumulator starts
// at beta[h] - mr[h] in the high-part row, where beta[h] = sum_c q'[h][c] z_K[c] is the tile's zero-point term
// (computed once per tile on the VALU: packed fp16 dot products, fp32 sums, kept in a register of every lane of
// row h) and mr[h] the running maximum, so the sum is already relative to the maximum.
//
// Softmax. Lagged maximum: p = 2^(C_h (score - mr)) is taken directly unless some score exceeds mr (or on the
// first tile); only then the tile maximum is reduced over the row, mr raised and the accumulators rescaled.
//
// PV. The probabilities go through 512 B of LDS to lane (n, kc), which forms p~ = p s_V[g][t] of head n / 4 and
// value group g = n % 4 for its eight tokens as fp16 high and low parts (mixed-precision fmas, one rounding each).
// A second LDS pass (2 KB) regroups them into two A operands, one per value-group pair (groups 0, 1 and 2, 3):
// row 4 h + 2 m + r carries part r of head h for group m of the pair. Channel block j (16 channels, group j / 2)
// takes one MFMA with the operand of its pair, 8 per tile; its output lane (channel, kc) holds head kc's four rows,
// and the two rows of group j / 2 (high and low part) are added once, before the partials are stored. The value
// zero-point term sum_t p z_V[g][t] is accumulated on the VALU.
//
// Per-wavefront LDS: the tile's scales/zeros and the folded query, both written for tile v + 1 at the end of iteration
// v after every read of tile v has been issued (a wavefront's LDS operations complete in order); the probability
// exchange and the P V operands; the fp16 window value tile (8 KB, reusing the first region). Rows that lanes read
// together are padded so that they fall in different LDS banks (64 banks of 4 bytes): unpadded, the eight 256-byte rows
// of the folded query all start in bank 0 and every A-operand read of the score contraction is an 8-way conflict.
constexpr int LDS_SZ = 0;            // s_K[128], z_K[128] (fp16), then s_V[4][32], z_V[4][32] with each group's 64 bytes
                                     // followed by 16 bytes of padding (1152 bytes)
constexpr int QT_ROW = 136;          // fp16 per (part, head) row of the folded query: 128 channels + 8 padding
constexpr int LDS_QT = 1152;         // fp16 [2 (high, low)][4 heads][QT_ROW]
constexpr int P_ROW = 18;            // float2 per head of the probability exchange: 16 + 2 padding
constexpr int LDS_P = 8192;          // float2 [4 heads][P_ROW]: p of tokens i and 16 + i
constexpr int LDS_BYTES = LDS_P + 4 * P_ROW * 8;    // [0, 8192) also holds the fp16 window value tile [32][128]
// Dense-and-sparse records (the sparse kernel only): the tile's outlier section (768 B) and the integer correction
// sums (H, L) of the key outliers per (head, token) inside the window-tile region, which the quantized loop leaves
// free; the value-outlier sums per (head, channel) after the probability exchange.
constexpr int LDS_OUT = 3456;        // the record's bytes 3072..3839
// Every row of 32 sums (int64) is padded to 33, so the banks of one target differ between heads and groups and a
// wave's atomics spread over the banks.
constexpr int KROW = 33, KSUMS = 4 * KROW;             // [4 heads][33]
constexpr int VROW = 33, VSUMS = 16 * VROW;            // [4 heads][4 groups][33]
constexpr int LDS_KACC = 4224;       // int64 [4 heads][KROW]: key-outlier sums per (head, token)
constexpr int LDS_VACC = LDS_BYTES;  // int64 [4 heads][4 groups][VROW]: value-outlier sums per (head, channel)
constexpr int LDS_BYTES_SPARSE = LDS_VACC + VSUMS * 8;
// The P V A operands of the quantized loop (two value-group pairs x 64 lanes x 16 bytes; the second starts 16
// bytes past the first's end, so the 16 lanes of a write pass hit distinct banks), inside the region the
// quantized loop leaves free (after the outlier section and the key-outlier sums of the sparse kernel)
constexpr int LDS_PV = 5376;
constexpr int PV_PAIR = 65;   // 16-byte units from one pair's operand to the next
static_assert(LDS_PV >= LDS_KACC + KSUMS * 8 && LDS_PV + 16 * (PV_PAIR + 64) <= LDS_P,
              "P V operands inside the free region");
// 256 zero bytes after each kernel's LDS, read by the score operand's unused rows; placed in banks the folded-query
// rows of the same reads do not use
template <bool SPARSE>
constexpr int lds_zero() { return SPARSE ? LDS_BYTES_SPARSE + 64 : LDS_BYTES; }
template <bool SPARSE>
constexpr int lds_total() { return lds_zero<SPARSE>() + 256; }
static_assert(LDS_OUT >= LDS_QT + 8 * QT_ROW * 2 && LDS_KACC + KSUMS * 8 <= 8192, "sparse regions inside the free window region");
static_assert(LDS_KACC % 8 == 0 && LDS_VACC % 8 == 0, "64-bit sums");
// Exact sums of corrections through integer LDS atomics (float LDS atomics cost some thirty times an integer one on
// this chip). Every correction is below 2^17 in magnitude (a query scaled below 1 or a probability at most 1, times
// the difference of two binary16 values), so x = H 2^-6 + L 2^-29 + e with integers |H|, |L| < 2^23 and |e| < 2^-29,
// and X = H 2^23 + L is x 2^29 truncated to an integer, |X| < 2^46: up to 128 terms per target stay far inside int64,
// added by one 64-bit atomic per term.
__device__ __forceinline__ int64_t fix_split(float x) {
#pragma clang fp contract(off)
    const int32_t H = (int32_t)(x * 64.0f);
    const float r = __builtin_fmaf(-(float)H, 0x1p-6f, x);   // exact: the low bits of x
    const int32_t L = (int32_t)(r * 0x1p29f);
    return (int64_t)H * 8388608 + L;
}
__device__ __forceinline__ float fix_join(int64_t X) {
    const int32_t hi = (int32_t)(X >> 32);
    const uint32_t lo = (uint32_t)X;
    return __builtin_fmaf((float)hi, 0x1p3f, (float)lo * 0x1p-29f);   // 2^32 2^-29 = 2^3
}
__device__ __forceinline__ void lds_add64(int64_t *p, int64_t x) {
    __hip_atomic_fetch_add(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// byte offset of metadata byte x (0..1023 of a record's scale/zero section) in the staged copy
__device__ __forceinline__ int sz_off(int x) { return x < 512 ? x : x + 16 * ((x - 512) >> 6); }

// MODE: 0 uniform lengths; 1 per-sequence lengths (ragged); 2 the single-launch ragged decode step (below).
//
// Decode step (MODE 2). Every workgroup derives the step of its sequence from the lengths before it (append the
// token; a full window is flushed first; a sequence whose flush would pass the capacity refuses the token and is
// marked full) and attends over the state after it. The tiles of a flushed window were quantized ahead (see the
// ragged append), so a flush only moves the lengths. The last grid row holds one block workgroup per (sequence, KV
// head, chunk): when the appended token completes a window block, the chunk-0 workgroup writes that block's record
// ahead (from the window rows below the token and the token itself, from the input), beside the attention. It is
// dispatched after the splits (first, it cost the steps ~1 us: the splits' own dispatch order matters more), and its
// ~10 us of work ends well within a step. The other rows are the splits. The new token is attended straight from the
// input (its window row is written only at the end). After its partials are stored, a split counts itself in
// sync[(b, KV head, chunk)]; the last of the splits merges them (the pass-2 code) and counts the chunk in sync[b], as
// does every block workgroup once its loads are complete; the last of the sequence's 2 * KV heads * chunks counts
// writes the new window rows (several chunks per KV head) and the lengths, by when every workgroup of the sequence has
// read them. Counters are reset by the workgroup that completes them. No workgroup waits for another. Ordering: the
// tickets are relaxed agent-scope atomics, so they carry no happens-before edge of the HIP memory model. The merge is
// correct because of three hardware facts this kernel relies on instead: every value another workgroup reads (the split
// partials) is written with agent-scope atomic stores, which write through to the device's coherence point, and read
// with agent-scope atomic loads, which read from it (never from a non-coherent per-XCD L2 line); a workgroup waits for
// all its memory operations (s_waitcnt vmcnt(0): stores acknowledged, loads returned) before taking its ticket; the
// ticket is itself performed at the coherence point. A plain store that another workgroup of the launch read would need
// a release/acquire pair instead (at agent scope an L2 write-back and invalidate per workgroup, which costs the step
// several times its length).
//
// G1 (one query head per KV head): head row 0 of the score operand holds the head; with dense records rows 1..3 are
// zero (with dense-and-sparse records they repeat it), and the softmax state of row 0 drives every accumulator row. PV
// puts the high and low parts of p~ in different A-operand rows (row 4 part + group) straight from the probability
// exchange, with no regrouping pass: 8 MFMAs per tile (rows 8..15 zero with dense records). The parts are added across
// lanes (n, 0) and (n, 1) once, before the partials are stored.
//
// SPARSE (dense-and-sparse records, uniform lengths): a key outlier decodes as its zero point inside the dense
// contraction (its code is 0), so its token's score misses q'_c (o - z_c); lane (n, kc) adds these for its eight
// channels of head kc into the (head, token) sums while staging the tile, and the score lanes take them with the
// zero-point term. A value outlier likewise adds p_t (o - z) to its channel: each lane adds those of its (head,
// group, eight tokens) into the (head, channel) sums before PV and the output lanes read them back after it. Both
// sums are exact integer sums (fix_split), so the result does not depend on the order of the adds.
template <int MODE, bool G1, bool SPARSE>
__device__ __forceinline__ void decode_pass1_body(const DecodeArgs &a, unsigned char *smem) {
    constexpr int RECB = rec_bytes<SPARSE>();
    // G1, dense records: only head part 0 of the score operand and P V parts 0, 1 are read back, so the repeated
    // rows are zero (lower matrix-unit power); the softmax of head part 0 drives every row
    constexpr bool G1Z = G1 && !SPARSE;
    uint32_t *sz_lds = reinterpret_cast<uint32_t *>(smem + LDS_SZ);
    const _Float16 *szh = reinterpret_cast<const _Float16 *>(smem + LDS_SZ);
    _Float16 *qt_lds = reinterpret_cast<_Float16 *>(smem + LDS_QT);
    float *p_lds = reinterpret_cast<float *>(smem + LDS_P);
    _Float16 *vres_lds = reinterpret_cast<_Float16 *>(smem);

    // The workgroup's indices, lengths and tile range are uniform; they are kept in scalar registers (integer
    // division runs on the vector unit, and its results would otherwise stay in vector registers: the loop counter
    // and every record address would then cost vector instructions per tile, and in MODE 2 they spill around the
    // in-kernel flush)
    auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
    const int l = threadIdx.x;
    const int n = l & 15, kc = l >> 4, hl = n >> 2, g = n & 3;
    const int unit = blockIdx.x;
    // splits (MODE 2: the last grid row holds the block workgroups); the split holding the fp16 window tiles is
    // dispatched first
    const int nsplit = MODE == 2 ? (int)gridDim.y - 1 : (int)gridDim.y;
    const int split = nsplit - 1 - (int)blockIdx.y;
    const int chunk = uni(unit % a.chunks);
    const int hkv = uni((unit / a.chunks) % a.kv_heads);
    const int b = uni(unit / (a.chunks * a.kv_heads));
    const int G = a.q_heads / a.kv_heads;
    const int gc = min(4, G - 4 * chunk);
    const int h0 = hkv * G + 4 * chunk;

    int n_qtiles = a.n_qtiles, n_resid = a.n_resid, tiles_per_split = a.tiles_per_split;
    int new_row = -1;    // MODE 2: window row of the token this step appends (or -1)
    bool refuse = false; // MODE 2: the flush does not fit: the token is refused and the sequence marked full
    if constexpr (MODE != 0) {   // this sequence's lengths; the splits share its tiles evenly
        const int32_t *ln = a.lens + 4 * b;
        int nq = ln[0], nr = ln[1];
        if constexpr (MODE == 1) {
            if (a.appended) ragged_after_append(ln, a.res_cap, nq, nr);
        } else if (ln[3] == 0) {
            if (nr == a.res_cap) {
                if ((int64_t)nq + a.res_cap <= a.max_tiles * 32) {
                    nq += nr;
                    nr = 1;
                    new_row = 0;
                } else {
                    refuse = true;
                }
            } else {
                new_row = nr;
                nr += 1;
            }
        }
        n_qtiles = uni(nq / 32);
        n_resid = uni(nr);
        tiles_per_split = uni((n_qtiles + (n_resid + 31) / 32 + nsplit - 1) / nsplit);
        new_row = uni(new_row);
    }

    // MODE 2: the appended token's window rows of KV head h
    auto write_rows = [&](int h) {
        const int64_t dst = (((int64_t)b * a.kv_heads + h) * a.res_cap + new_row) * D;
        const int64_t src = b * a.new_sb + h * a.new_sh;
        const uint32_t kw = reinterpret_cast<const uint32_t *>(a.k_new + src)[l];
        const uint32_t vw = reinterpret_cast<const uint32_t *>(a.v_new + src)[l];
        reinterpret_cast<uint32_t *>(a.k_res_w + dst)[l] = kw;
        reinterpret_cast<uint32_t *>(a.v_res_w + dst)[l] = vw;
    };
    // MODE 2: counts this workgroup in sync[b]; the sequence's last count writes the window rows (when a KV head has
    // several chunks) and the lengths. Every counted workgroup has finished reading the lengths and the window rows:
    // its loads were complete before its tickets. Nothing in this launch reads the rows or lengths written here.
    auto sequence_ticket = [&]() {
        uint32_t *cb = a.sync + b;
        uint32_t prev = 0u;
        if (l == 0) prev = __hip_atomic_fetch_add(cb, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        prev = __shfl(prev, 0);
        if (prev + 1u != (uint32_t)(2 * a.kv_heads * a.chunks)) return;
        if (l == 0) *cb = 0u;
        if (new_row >= 0) {
            if (a.chunks > 1) {
                int h = 0;
                for (; h + 4 <= a.kv_heads; h += 4) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) write_rows(h + k);
                }
                for (; h < a.kv_heads; ++h) write_rows(h);
            }
            if (l == 0) {
                a.lens_w[4 * b] = n_qtiles * 32;
                a.lens_w[4 * b + 1] = n_resid;
            }
        } else if (refuse && l == 0) {
            a.lens_w[4 * b + 3] = 1;
        }
    };
    if constexpr (MODE == 2) {
        if ((int)blockIdx.y == nsplit) {   // block workgroup (no flush here: a flush leaves the token in row 0)
            if (chunk == 0 && new_row >= 0 && (new_row & 31) == 31) {
                const int64_t slot = n_qtiles + new_row / 32;
                if (slot < a.max_tiles)
                    quant_window_block(a.k_res, a.v_res, a.k_new, a.v_new, a.new_sb, a.new_sh, a.kv_heads, a.res_cap,
                                       new_row, b, hkv, a.tiles_w, a.max_tiles, slot, smem);
            }
            wait_vmcnt<0>();
            sequence_ticket();
            return;
        }
    }
    const int n_vt = n_qtiles + (n_resid + 31) / 32;
    const int v0 = uni(split * tiles_per_split);
    const int v1 = uni(min(v0 + tiles_per_split, n_vt));
    const int qend = uni(min(v1, n_qtiles));
    const uint8_t *base = a.tiles + ((int64_t)b * a.kv_heads + hkv) * a.max_tiles * (int64_t)RECB;

    // ---- query: lane (n, kc) holds head kc of the chunk (if valid), channels 8n .. 8n+7, scaled by 2^-E with
    // 2^E > max |q| of that head (qmax is a float16 value widened, hence a normal binary32 number: its exponent
    // field gives E). C turns a raw score of head kc (in q' units) into the log2 domain.
    h8 qf = {};
    float C;
    {
        const bool hv = G1 || kc < gc;
        const h8 raw = *reinterpret_cast<const h8 *>(a.q + ((int64_t)b * a.q_heads + h0 + (G1 || !hv ? 0 : kc)) * D + 8 * n);
        float qmax = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) qmax = fmaxf(qmax, fabsf((float)raw[e]));
        qmax = row16_max(qmax);
        int E = 0;
        if (qmax > 0.0f) E = (int)((__builtin_bit_cast(uint32_t, qmax) >> 23) & 0xffu) - 127 + 1;
        const float qsc = pow2(-E);
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[e] = hv ? (_Float16)((float)raw[e] * qsc) : (_Float16)0.0f;
        C = a.sm_log2 * pow2(E);
    }

    // softmax state of head kc (lanes of row kc agree): running maximum mr of the raw scores, valid once `seen`
    float mr = 0.0f, lsum = 0.0f;
    bool seen = false;
    // PV state: o[j] rows (head kc, group r) (G1: part kc, group r), column n = channel n + 16 j; gam: lane (n, kc)
    // for (head hl, group g)
    float gam = 0.0f;
    f4 o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = f4{0.0f, 0.0f, 0.0f, 0.0f};


    // s0, s1: raw score minus mr of head kc for tokens n and 16 + n of the tile (-inf for absent tokens).
    // Raises mr to the tile maximum where it is exceeded (every head on the first tile) and rescales.
    auto rescale = [&](float &s0, float &s1) {
        float d = row16_max(fmaxf(s0, s1));
        if (seen) d = fmaxf(d, 0.0f);
        const float alpha = seen ? __builtin_amdgcn_exp2f(-d * C) : 1.0f;
        mr += d;
        s0 -= d;
        s1 -= d;
        lsum *= alpha;
        const float ao = G1Z ? __shfl(alpha, 0) : alpha;
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) o[j][r] *= ao;
        gam *= G1Z ? ao : __shfl(alpha, 16 * hl);
        seen = true;
    };
    // p of tokens n and 16 + n to LDS; returns, for the PV A layout of lane (n, kc), p of tokens 4kc + i (p[i]) and
    // 16 + 4kc + i (p[4 + i]) of head hl (G1 with dense records: of head row 0 for parts hl = 0, 1 and zeros for the
    // repeated parts 2, 3)
    auto exchange = [&](float p0, float p1, float p[8]) {
        reinterpret_cast<float2 *>(p_lds)[P_ROW * kc + n] = float2{p0, p1};
        wave_lds_order();
        const f4 *pr = G1Z ? (hl < 2 ? reinterpret_cast<const f4 *>(p_lds) + 2 * kc
                                     : reinterpret_cast<const f4 *>(smem + lds_zero<SPARSE>()))
                           : reinterpret_cast<const f4 *>(p_lds) + (P_ROW * hl + 4 * kc) / 2;
        const f4 pa = pr[0];
        const f4 pb = pr[1];
        p[0] = pa[0]; p[4] = pa[1]; p[1] = pa[2]; p[5] = pa[3];
        p[2] = pb[0]; p[6] = pb[1]; p[3] = pb[2]; p[7] = pb[3];
    };

    int64_t *kacc = reinterpret_cast<int64_t *>(smem + LDS_KACC);
    int64_t *vacc = reinterpret_cast<int64_t *>(smem + LDS_VACC);
    if constexpr (SPARSE) {
        for (int i = l; i < KSUMS; i += 64) kacc[i] = 0;
        for (int i = l; i < VSUMS; i += 64) vacc[i] = 0;
        wave_lds_order();
    }

    // stage a tile's scales/zeros and its folded query (high, low) into LDS (SPARSE: and its outlier section, with
    // the key-outlier corrections of the lane's eight channels added into the (head, token) sums); returns the
    // tile's beta of head kc minus the running maximum, the same in every lane of row kc (each of the row's 16
    // partial sums starts at -mr / 16; mr only changes after the next tile's scores)
    auto stage = [&](const uint4 &sw, const uint4 &ow) -> float {
        *reinterpret_cast<uint4 *>(smem + LDS_SZ + sz_off(16 * l)) = sw;
        if constexpr (SPARSE) {
            if (l < 48) reinterpret_cast<uint4 *>(smem + LDS_OUT)[l] = ow;
        }
        wave_lds_order();
        const h8 sk = *reinterpret_cast<const h8 *>(szh + 8 * n);
        const h8 zk = *reinterpret_cast<const h8 *>(szh + 128 + 8 * n);
        if constexpr (SPARSE) {
            const h8 ok = *reinterpret_cast<const h8 *>(smem + LDS_OUT + 16 * n);
            const uint2 uk = *reinterpret_cast<const uint2 *>(smem + LDS_OUT + 256 + 8 * n);
            const int krow = KROW * kc;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float qe = (float)qf[e];
                const float corr = __builtin_fmaf(qe, (float)ok[e], -(qe * (float)zk[e]));   // q' o and q' z exact
                const uint32_t u = ((e < 4 ? uk.x : uk.y) >> (8 * (e & 3))) & 31u;
                lds_add64(kacc + krow + u, fix_split(corr));
            }
        }
        const h8 hi = qf * sk;
        const h8 lo = __builtin_elementwise_fma(qf, sk, -hi);
        *reinterpret_cast<h8 *>(qt_lds + QT_ROW * kc + 8 * n) = hi;
        *reinterpret_cast<h8 *>(qt_lds + QT_ROW * (4 + kc) + 8 * n) = lo;
        float bp = -0.0625f * mr;
#pragma unroll
        for (int e = 0; e < 8; e += 2)
            bp = __builtin_amdgcn_fdot2(h2{zk[e], zk[e + 1]}, h2{qf[e], qf[e + 1]}, bp, false);
        wave_lds_order();
        return row16_sum(bp);
    };

    // ------------------------------------------------------------------ quantized tiles
    // Each code word is reloaded for the next tile right after its last use in this one (scales: at the top of the
    // iteration, key codes after the score contraction, value codes after PV), so no register holds two tiles. On
    // the last tile the index is clamped: the reload hits the just-read record in cache.
    // A operand row n = 4 h + r: head h, high part (r = 0), low part (r = 1); rows r = 2, 3 (outputs never used), and
    // with G1 and dense records head rows 1..3, read a zero row: zero operands draw less power than repeated ones, and
    // the clock this kernel runs at is power-limited
    const _Float16 *qta = ((n & 2) || (G1Z && hl > 0)) ? reinterpret_cast<const _Float16 *>(smem + lds_zero<SPARSE>()) + 8 * kc
                                  : qt_lds + QT_ROW * (4 * (n & 1) + hl) + 8 * kc;
    reinterpret_cast<uint32_t *>(smem + lds_zero<SPARSE>())[l] = 0u;
    uint4 kw, vw, sw, ow = {};
    // start of the score accumulators: row 0 (high part) beta - mr of the current tile, rows 1..3 zero
    f4 ci = {0.0f, 0.0f, 0.0f, 0.0f};
    const int ol = l < 48 ? l : l - 48;   // SPARSE: lanes 0..47 load the outlier section (the rest reload a part)
    if (v0 < qend) {
        const uint8_t *rec = base + (int64_t)v0 * RECB;
        kw = load_stream(rec, l);
        vw = load_stream(rec + 1024, l);
        sw = load_stream(rec + 2048, l);
        if constexpr (SPARSE) ow = load_stream(rec + REC, ol);
        ci[0] = stage(sw, ow);
    }
    for (int v = v0; v < qend; ++v) {
        // the next record's address is uniform: kept in scalar registers (opaque to the compiler, which would
        // otherwise hoist a per-lane 64-bit base out of the loop and rebuild every address with vector arithmetic),
        // each load a scalar base plus the lane's offset
        const uint8_t *next = base + (int64_t)min(v + 1, qend - 1) * RECB;
        uint64_t next_s = reinterpret_cast<uint64_t>(next);
        asm volatile("" : "+s"(next_s));
        typedef __attribute__((address_space(1))) const u32x4 g_u32x4;
        g_u32x4 *next_g = reinterpret_cast<g_u32x4 *>(next_s);
        auto load_rec = [&](int off) { return __builtin_bit_cast(uint4, __builtin_nontemporal_load(next_g + off / 16 + l)); };
        sw = load_rec(2048);
        if constexpr (SPARSE) ow = load_stream(next + REC, ol);

        f4 acc0 = ci, acc1 = ci;   // tokens n (acc0) and 16 + n (acc1); rows (head kc, part r)
        if constexpr (SPARSE) {   // the key-outlier sums of tokens n and 16 + n of head kc, then cleared
            int64_t *kr = kacc + KROW * kc + n;
            acc0[0] += fix_join(kr[0]);
            acc1[0] += fix_join(kr[16]);
            wave_lds_order();
            kr[0] = 0;
            kr[16] = 0;
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const h8 bq = *reinterpret_cast<const h8 *>(qta + 32 * ks);
            acc0 = mfma(bq, expand8(nibbles(kw[ks >> 1], ks & 1)), acc0);
            acc1 = mfma(bq, expand8(nibbles(kw[2 + (ks >> 1)], ks & 1)), acc1);
        }
        kw = load_rec(0);
        float s0 = acc0[0] + acc0[1], s1 = acc1[0] + acc1[1];
        if (!seen || __any(fmaxf(s0, s1) > 0.0f)) rescale(s0, s1);
        const float p0 = __builtin_amdgcn_exp2f(s0 * C), p1 = __builtin_amdgcn_exp2f(s1 * C);
        lsum += p0 + p1;
        float p[8];
        exchange(p0, p1, p);

        // p~ = p * s_V of group g, fp16 high part and the fp16 rounding of the remainder; value zero points
        const unsigned char *szb = smem + LDS_SZ;
        const h4 sv0 = *reinterpret_cast<const h4 *>(szb + sz_off(512 + 64 * g + 8 * kc));
        const h4 sv1 = *reinterpret_cast<const h4 *>(szb + sz_off(512 + 64 * g + 32 + 8 * kc));
        const h4 zv0 = *reinterpret_cast<const h4 *>(szb + sz_off(768 + 64 * g + 8 * kc));
        const h4 zv1 = *reinterpret_cast<const h4 *>(szb + sz_off(768 + 64 * g + 32 + 8 * kc));
        const uint2 sa = __builtin_bit_cast(uint2, sv0), sb = __builtin_bit_cast(uint2, sv1);
        uint4 uh, ul;
        split_pair(p[0], p[1], sa.x, uh.x, ul.x);
        split_pair(p[2], p[3], sa.y, uh.y, ul.y);
        split_pair(p[4], p[5], sb.x, uh.z, ul.z);
        split_pair(p[6], p[7], sb.y, uh.w, ul.w);
        const h8 phi = __builtin_bit_cast(h8, uh), plo = __builtin_bit_cast(h8, ul);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            gam = __builtin_fmaf(p[i], (float)zv0[i], gam);
            gam = __builtin_fmaf(p[4 + i], (float)zv1[i], gam);
        }
        if constexpr (SPARSE) {   // value outliers of (head hl, group g) at tokens 4kc + i and 16 + 4kc + i
            const unsigned char *os = smem + LDS_OUT;
            const h4 ov0 = *reinterpret_cast<const h4 *>(os + 384 + 64 * g + 8 * kc);
            const h4 ov1 = *reinterpret_cast<const h4 *>(os + 384 + 64 * g + 32 + 8 * kc);
            const uint32_t oi0 = *reinterpret_cast<const uint32_t *>(os + 640 + 32 * g + 4 * kc);
            const uint32_t oi1 = *reinterpret_cast<const uint32_t *>(os + 640 + 32 * g + 16 + 4 * kc);
            const int vrow = VROW * (4 * hl + g);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float d = (i < 4 ? (float)ov0[i] - (float)zv0[i] : (float)ov1[i - 4] - (float)zv1[i - 4]);
                const uint32_t c = ((i < 4 ? oi0 : oi1) >> (8 * (i & 3))) & 31u;
                lds_add64(vacc + vrow + c, fix_split(p[i] * d));
            }
        }
        if constexpr (G1) {
            const h8 pp = (hl & 1) ? plo : phi;
#pragma unroll
            for (int j = 0; j < 8; ++j) o[j] = mfma(pp, expand8(nibbles(vw[j >> 1], j & 1)), o[j]);
        } else {   // the two A operands of the value-group pairs, rows (head, group in pair, part), through LDS
            uint4 *pvw = reinterpret_cast<uint4 *>(smem + LDS_PV) + PV_PAIR * (g >> 1) + 16 * kc + 4 * hl + 2 * (g & 1);
            pvw[0] = uh;
            pvw[1] = ul;
            wave_lds_order();
            const uint4 *pvr = reinterpret_cast<const uint4 *>(smem + LDS_PV) + l;
            const h8 pa0 = __builtin_bit_cast(h8, pvr[0]);
            const h8 pa1 = __builtin_bit_cast(h8, pvr[PV_PAIR]);
#pragma unroll
            for (int j = 0; j < 8; ++j) o[j] = mfma(j < 4 ? pa0 : pa1, expand8(nibbles(vw[j >> 1], j & 1)), o[j]);
        }
        asm volatile("" : "+s"(next_s));   // the base again from scalar registers (this is a later block)
        vw = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<g_u32x4 *>(next_s) + 64 + l));
        if constexpr (SPARSE) {   // head kc's value-outlier sums of channels n + 16 j, then cleared (G1: row 0 only)
            wave_lds_order();
            // channel n + 16 j of head kc: group j / 2, index n + 16 (j % 2) within it
            int64_t *vr = vacc + VROW * 4 * kc + n;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float corr = fix_join(vr[VROW * (j >> 1) + 16 * (j & 1)]);
                if (!G1 || kc == 0) o[j][G1 ? (j >> 1) : 2 * ((j >> 1) & 1)] += corr;
            }
            wave_lds_order();
#pragma unroll
            for (int j = 0; j < 8; ++j) vr[VROW * (j >> 1) + 16 * (j & 1)] = 0;
        }
        // every LDS read of this tile has been issued: overwrite with the next tile (after the last tile, with
        // that tile again; unconditional, so no load sits on only one path of the loop)
        ci[0] = stage(sw, ow);
    }

    // ------------------------------------------------------------------ residual (fp16) tiles
    // The same contraction with A = q' (high part; the low part zero) and B = the fp16 key rows, loaded
    // straight into registers at the top of each iteration. The value rows of a tile are copied into LDS by LDS-DMA
    // loads (issued for the next tile once PV has read the current one) and reach the PV B layout through transpose
    // reads; p~ = p (no scales). Window tiles (at most four per split in the normal case) and all-fp16 caches (the
    // fp16 comparator, bandwidth-bound: 16 KB per tile and wavefront) share this loop.
    const int w0 = max(v0, n_qtiles);
    if (w0 < v1) {
        h8 qw[4];
        __syncthreads();
        *reinterpret_cast<h8 *>(qt_lds + QT_ROW * kc + 8 * n) = qf;
        *reinterpret_cast<h8 *>(qt_lds + QT_ROW * (4 + kc) + 8 * n) = h8{};
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qw[ks] = *reinterpret_cast<const h8 *>(qta + 32 * ks);
        wait_lgkmcnt0();    // the query rows are in registers: the LDS below may be overwritten
        const _Float16 *kres = a.k_res + ((int64_t)b * a.kv_heads + hkv) * a.res_cap * D;
        const _Float16 *vres = a.v_res + ((int64_t)b * a.kv_heads + hkv) * a.res_cap * D;
        const uint32_t vt_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char *)smem;
        // 32 value rows of tile v (8 KB, contiguous in the window; rows past the window's length are read from
        // the buffer's capacity, which is a multiple of 32 rows, and zeroed in LDS before use)
        auto v_dma = [&](int v) {
            const unsigned char *src =
                reinterpret_cast<const unsigned char *>(vres + (int64_t)(v - n_qtiles) * 32 * D) + 16 * l;
#pragma unroll
            for (int i = 0; i < 8; ++i) lds_dma16(src + 1024 * i, vt_base + 1024 * i);
        };
        // key rows of tokens n and 16 + n (clamped to the window's length), channels 32 ks + 8 kc ..
        // MODE 2: the appended token's row comes from the input
        const _Float16 *knew_row = (MODE == 2 && new_row >= 0) ? a.k_new + b * a.new_sb + hkv * a.new_sh : nullptr;
        auto krow = [&](int row) -> const _Float16 * {
            if constexpr (MODE == 2) {
                if (row == new_row) return knew_row;
            }
            return kres + (int64_t)row * D;
        };
        auto k_load = [&](int v, h8 kr[8]) {
            const int r0 = (v - n_qtiles) * 32;
            const int nv = min(32, n_resid - r0);
            const _Float16 *k0 = krow(r0 + min(n, nv - 1)) + 8 * kc;
            const _Float16 *k1 = krow(r0 + min(16 + n, nv - 1)) + 8 * kc;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                kr[ks] = __builtin_bit_cast(h8, load_stream(k0 + 32 * ks, 0));
                kr[4 + ks] = __builtin_bit_cast(h8, load_stream(k1 + 32 * ks, 0));
            }
        };
        // transpose-read addressing: lane (n, kc) reads token 4 TQ + n / 4, channels 16 j + 4 (n % 4) .. + 3 and
        // receives tokens 4 TQ .. 4 TQ + 3 of channel 16 j + n; TQ = kc (tokens 4 kc ..) and 4 + kc (16 + 4 kc ..)
        const _Float16 *vt0 = vres_lds + (4 * kc + (n >> 2)) * 128 + 4 * (n & 3);
        const _Float16 *vt1 = vt0 + 16 * 128;
        v_dma(w0);
        for (int v = w0; v < v1; ++v) {
            const int r0 = (v - n_qtiles) * 32;
            const int nv = min(32, n_resid - r0);
            h8 kr[8];
            k_load(v, kr);
            const f4 ci = {-mr, 0.0f, 0.0f, 0.0f};
            f4 acc0 = ci, acc1 = ci;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                acc0 = mfma(qw[ks], kr[ks], acc0);
                acc1 = mfma(qw[ks], kr[4 + ks], acc1);
            }
            float s0 = (n < nv) ? acc0[0] + acc0[1] : -__builtin_inff();
            float s1 = (16 + n < nv) ? acc1[0] + acc1[1] : -__builtin_inff();
            if (!seen || __any(fmaxf(s0, s1) > 0.0f)) rescale(s0, s1);
            const float p0 = __builtin_amdgcn_exp2f(s0 * C), p1 = __builtin_amdgcn_exp2f(s1 * C);
            lsum += p0 + p1;
            float p[8];
            exchange(p0, p1, p);
            h8 phi, plo;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                phi[i] = (_Float16)p[i];
                plo[i] = (_Float16)(p[i] - (float)phi[i]);
            }
            wait_vmcnt<0>();    // this tile's value rows have landed
            if (nv < 32) {      // zero the rows past the window's length (their p is 0, their contents arbitrary)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int idx = l + 64 * i;   // 16-byte chunk: row idx / 16
                    if ((idx >> 4) >= nv) reinterpret_cast<uint4 *>(vres_lds)[idx] = uint4{0u, 0u, 0u, 0u};
                }
                wait_lgkmcnt0();
            }
            if constexpr (MODE == 2) {   // the appended token's value row, from the input
                if (new_row >= r0 && new_row < r0 + 32) {
                    if (l < 16)
                        reinterpret_cast<uint4 *>(vres_lds + (new_row - r0) * D)[l] =
                            reinterpret_cast<const uint4 *>(a.v_new + b * a.new_sb + hkv * a.new_sh)[l];
                    wait_lgkmcnt0();
                }
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const h4 lo4 = read_tr16(vt0 + 16 * j);
                const h4 hi4 = read_tr16(vt1 + 16 * j);
                const h8 bv = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
                if constexpr (G1) {
                    o[j] = mfma((hl & 1) ? plo : phi, bv, o[j]);
                } else {   // row n: part n % 2 of head n / 4 (p~ = p, the same for both groups of a pair)
                    o[j] = mfma((n & 1) ? plo : phi, bv, o[j]);
                }
            }
            wait_lgkmcnt0();    // PV has read the value rows: the next tile may overwrite them
            if (v + 1 < v1) v_dma(v + 1);
        }
        wait_vmcnt<0>();
    }

    // ------------------------------------------------------------------ partials of this split
    lsum = row16_sum(lsum);    // head kc
    gam = rows_sum(gam);       // (head hl, group g)
    float gr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) gr[r] = __shfl(gam, 4 * kc + r);
    if constexpr (G1) {   // lane (n, 0) adds the low parts held by lane (n, 1)
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j][j >> 1] += __shfl(o[j][j >> 1], (l & 15) + 16);
    } else {              // high and low part of channel block j's group (row 2 (group % 2) + part of head kc)
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j][j >> 1] = o[j][2 * ((j >> 1) & 1)] + o[j][2 * ((j >> 1) & 1) + 1];
    }
    const int64_t S = nsplit;
    if (kc < gc) {   // lane (n, kc) holds head h0 + kc, channels n + 16 j
        const int hq = h0 + kc;
        float *po = a.part_o + (((int64_t)b * a.q_heads + hq) * S + split) * D;
        float *pm = a.part_ml + (((int64_t)b * a.q_heads + hq) * S + split) * 2;
        const float m_out = seen ? mr * C : -__builtin_inff();
        if constexpr (MODE == 2) {   // read by the merging workgroup of this launch
#pragma unroll
            for (int j = 0; j < 8; ++j) coherent_store(po + n + 16 * j, o[j][j >> 1] + gr[j >> 1]);
            if (n == 0) {
                coherent_store(pm, m_out);
                coherent_store(pm + 1, lsum);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) po[n + 16 * j] = o[j][j >> 1] + gr[j >> 1];
            if (n == 0) {
                pm[0] = m_out;
                pm[1] = lsum;
            }
        }
    }

    if constexpr (MODE == 2) {
        // count this split once its partial stores are complete (and every load of this workgroup, so the cache
        // state it read may be overwritten once all are counted); the last one merges the chunk's heads
        wait_vmcnt<0>();
        uint32_t *cnt = a.sync + a.batch + ((int64_t)b * a.kv_heads + hkv) * a.chunks + chunk;
        uint32_t prev = 0u;
        if (l == 0) prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        prev = __shfl(prev, 0);
        if (prev + 1u != (uint32_t)S) return;
        if (l == 0) *cnt = 0u;
        float *wts = reinterpret_cast<float *>(smem);   // S <= PASS2_MAX_SPLITS floats + 8 zero weights
        __syncthreads();
        for (int k = 0; k < gc; ++k) {
            merge_splits<true>(a.part_o, a.part_ml, a.out, (int)S, (int64_t)b * a.q_heads + h0 + k, wts, true);
            __syncthreads();
        }
        // with one chunk per KV head, every reader of the window of KV head hkv is counted by now (its splits here,
        // its block workgroup reads no window row at or past the token's), so this workgroup writes the token's rows;
        // otherwise the sequence's last count writes all. Nothing in this launch reads the outputs or window rows
        // stored here, so their stores need not be complete before the sequence ticket; the end of the launch makes
        // them visible.
        if (a.chunks == 1 && new_row >= 0) write_rows(hkv);
        sequence_ticket();
    }
}

template <int MODE, bool G1>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(4, 4))) void decode_pass1_kernel(DecodeArgs a) {
    __shared__ __align__(16) unsigned char smem[lds_total<false>()];
    decode_pass1_body<MODE, G1, false>(a, smem);
}

// dense-and-sparse records: three wavefronts per SIMD (12.7 KB of LDS, up to 168 registers)
template <bool G1>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3, 3))) void decode_pass1_sparse_kernel(DecodeArgs a) {
    __shared__ __align__(16) unsigned char smem[lds_total<true>()];
    decode_pass1_body<0, G1, true>(a, smem);
}

// ------------------------------------------------------------------------------------------------ decode pass 2
// One wavefront per (batch row, query head): out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s. The splits'
// (m, l) are read by all lanes at once (lane l takes splits l, l + 64, ...), M and the weighted sum of l are wave
// reductions, and the weights go through LDS to the lanes that sum the partial outputs (lane l: channels 2l, 2l+1),
// eight splits per batch of loads. Empty splits carry m = -inf and weight 0.
// Ragged caches: a sequence with no token gives zeros, and with `commit` the workgroup of each sequence's first query
// head makes the appended token visible in its lengths (every pass-1 read of them is complete by now).
template <bool RAGGED>
__global__ __launch_bounds__(64) void decode_pass2_kernel(const float *part_o, const float *part_ml, float *out,
                                                          int splits, int32_t *lens, int q_heads, int res_cap,
                                                          int commit) {
    __shared__ float wts[PASS2_MAX_SPLITS + 32];   // + zero weights after the last split
    const int64_t bh = blockIdx.x;
    if constexpr (RAGGED) {
        if (commit && threadIdx.x == 0 && bh % q_heads == 0) {
            int32_t *ln = lens + 4 * (bh / q_heads);
            int nq, nr;
            ragged_after_append(ln, res_cap, nq, nr);
            ln[0] = nq;
            ln[1] = nr;
        }
    }
    merge_splits<false, 24>(part_o, part_ml, out, splits, bh, wts, RAGGED);
}

// ------------------------------------------------------------------------------------------------ launchers
hipError_t launch_quant_keys(const TokSrc &src, int64_t t_begin, int64_t n_tiles, int batch, int kv_heads,
                             uint8_t *tiles, int64_t max_tiles, int64_t tile0, bool sparse, hipStream_t st) {
    dim3 grid((unsigned)n_tiles, (unsigned)kv_heads, (unsigned)batch);
    if (sparse)
        hipLaunchKernelGGL(quant_keys_kernel<true>, grid, dim3(64), 0, st, src, t_begin, kv_heads, tiles, max_tiles, tile0);
    else
        hipLaunchKernelGGL(quant_keys_kernel<false>, grid, dim3(64), 0, st, src, t_begin, kv_heads, tiles, max_tiles, tile0);
    return hipGetLastError();
}

hipError_t launch_quant_values(const TokSrc &src, int64_t t_begin, int64_t n_tiles, int batch, int kv_heads,
                               uint8_t *tiles, int64_t max_tiles, int64_t tile0, bool sparse, hipStream_t st) {
    dim3 grid((unsigned)n_tiles, (unsigned)kv_heads, (unsigned)batch);
    if (sparse)
        hipLaunchKernelGGL(quant_values_kernel<true>, grid, dim3(64), 0, st, src, t_begin, kv_heads, tiles, max_tiles, tile0);
    else
        hipLaunchKernelGGL(quant_values_kernel<false>, grid, dim3(64), 0, st, src, t_begin, kv_heads, tiles, max_tiles, tile0);
    return hipGetLastError();
}

hipError_t launch_copy_rows(const TokSrc &ksrc, const TokSrc &vsrc, int64_t t_begin, int64_t n, int batch,
                            int kv_heads, _Float16 *kres, _Float16 *vres, int res_cap, int dst0, hipStream_t st) {
    dim3 grid((unsigned)((n + 3) / 4), (unsigned)kv_heads, (unsigned)batch);
    hipLaunchKernelGGL(copy_rows_kernel, grid, dim3(64), 0, st, ksrc, vsrc, t_begin, n, kv_heads, kres, vres,
                       res_cap, dst0);
    return hipGetLastError();
}

hipError_t launch_pass2(const float *part_o, const float *part_ml, float *out, int rows, int splits, hipStream_t st) {
    hipLaunchKernelGGL(decode_pass2_kernel<false>, dim3((unsigned)rows), dim3(64), 0, st, part_o, part_ml, out, splits,
                       nullptr, 1, 0, 0);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs &a, int splits, hipStream_t st) {
    const int units = a.batch * a.kv_heads * a.chunks;
    const dim3 grid((unsigned)units, (unsigned)splits);
    if (a.sparse && a.q_heads == a.kv_heads)
        hipLaunchKernelGGL((decode_pass1_sparse_kernel<true>), grid, dim3(64), 0, st, a);
    else if (a.sparse)
        hipLaunchKernelGGL((decode_pass1_sparse_kernel<false>), grid, dim3(64), 0, st, a);
    else if (a.q_heads == a.kv_heads)
        hipLaunchKernelGGL((decode_pass1_kernel<0, true>), grid, dim3(64), 0, st, a);
    else
        hipLaunchKernelGGL((decode_pass1_kernel<0, false>), grid, dim3(64), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_pass2(a.part_o, a.part_ml, a.out, a.batch * a.q_heads, splits, st);
}

hipError_t launch_decode_ragged(const DecodeArgs &a, int splits, int32_t *lens, int commit, hipStream_t st) {
    const int units = a.batch * a.kv_heads * a.chunks;
    if (a.q_heads == a.kv_heads)
        hipLaunchKernelGGL((decode_pass1_kernel<1, true>), dim3((unsigned)units, (unsigned)splits), dim3(64), 0, st, a);
    else
        hipLaunchKernelGGL((decode_pass1_kernel<1, false>), dim3((unsigned)units, (unsigned)splits), dim3(64), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_pass2_kernel<true>, dim3((unsigned)(a.batch * a.q_heads)), dim3(64), 0, st, a.part_o,
                       a.part_ml, a.out, splits, lens, a.q_heads, a.res_cap, commit);
    return hipGetLastError();
}

hipError_t launch_decode_step(const DecodeArgs &a, int splits, hipStream_t st) {
    const int units = a.batch * a.kv_heads * a.chunks;
    const dim3 grid((unsigned)units, (unsigned)splits + 1u);   // last row: the block workgroups
    if (a.q_heads == a.kv_heads)
        hipLaunchKernelGGL((decode_pass1_kernel<2, true>), grid, dim3(64), 0, st, a);
    else
        hipLaunchKernelGGL((decode_pass1_kernel<2, false>), grid, dim3(64), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_ragged_flush_append(const TokSrc &knew, const TokSrc &vnew, int batch, int kv_heads,
                                      uint8_t *tiles, int64_t max_tiles, _Float16 *k_res, _Float16 *v_res,
                                      int res_cap, int32_t *lens, hipStream_t st) {
    dim3 grid((unsigned)(res_cap / 32), (unsigned)kv_heads, (unsigned)batch);
    hipLaunchKernelGGL(ragged_flush_append_kernel, grid, dim3(64), 0, st, knew, vnew, kv_heads, tiles, max_tiles,
                       k_res, v_res, res_cap, lens);
    return hipGetLastError();
}

hipError_t launch_ragged_commit(int32_t *lens, int batch, int res_cap, hipStream_t st) {
    hipLaunchKernelGGL(ragged_commit_kernel, dim3((unsigned)((batch + 255) / 256)), dim3(256), 0, st, lens, batch,
                       res_cap);
    return hipGetLastError();
}

hipError_t launch_ragged_set(int32_t *lens, int b, int nq, int nr, int ns, hipStream_t st) {
    hipLaunchKernelGGL(ragged_set_kernel, dim3(1), dim3(1), 0, st, lens, b, nq, nr, ns);
    return hipGetLastError();
}

}  // namespace kvq
