// HIP kernels for gfx950 (CDNA4): the 4-bit KVQuant-style variant of the cache. Keys are quantized per channel and
// values per token with 4-bit codes in 5120-byte tile records; keys may be cached before the rotary embedding and are
// then rotated at decode time by their absolute position; token 0 may be held apart as an attention sink whose key
// stays in fp16. Decode pass 2 (the split merge) is shared with the 2-bit path.
//
// Sources: synthetic.wiki "KV cache quantization: putting the bits in the cached vectors, not the weights",
// section "Keys are harder than values" (per-channel keys, per-token values, keys quantized before RoPE with the
// rotation applied after dequantization) and section "What they report" (the first token's keys kept in full
// precision: attention sink); RoFormer form of the rotary
// embedding for the pair layout (adjacent channels 2i, 2i+1, angle m * base^(-2i/D)).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_kernels.h"
#include "kvq_lanes.h"
#include "kvq_quantizer.h"

namespace kvq {

namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int HD = 128;
constexpr int REC4 = 5120;
constexpr int K4_SCALE = 4096, K4_ZERO = 4352;
constexpr int V4_CODES = 2048, V4_SCALE = 4608, V4_ZERO = 4864;
constexpr int SINK_REC = 512;
constexpr float L4 = 15.0f;   // highest 4-bit level
// dense-and-sparse records: the 5120 bytes above, then the outlier section
constexpr int REC4S = 5888;
constexpr int K4_OUT = 5120, K4_IDX = 5376, V4_OUT = 5504, V4_IDX = 5760;
constexpr int SINK_VOUT = 336, SINK_VIDX = 344;

template <bool SPARSE>
constexpr int record_bytes() { return SPARSE ? REC4S : REC4; }

// Order key of an element for the outlier choice of a 32-element group: the binary16 magnitude (the binary32 bits
// of |x| shifted by 13 keep every bit of a binary16 value and its order) above the reversed index, so the largest
// key is the largest magnitude and, among equal magnitudes, the lowest index.
__device__ __forceinline__ uint32_t outlier_key(float x, uint32_t idx) {
    return ((__builtin_bit_cast(uint32_t, __builtin_fabsf(x)) >> 13) << 5) | (31u - idx);
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_xmax_u32(uint32_t v) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
    return v > o ? v : o;
}
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
    v = dpp_xmax_u32<DPP_QUAD_1032>(v);
    v = dpp_xmax_u32<DPP_QUAD_2301>(v);
    v = dpp_xmax_u32<DPP_ROW_HALF_MIRROR>(v);
    return dpp_xmax_u32<DPP_ROW_MIRROR>(v);
}

}  // namespace

// ------------------------------------------------------------------------------------------------ quantizers
// Keys: one workgroup of 64 lanes per tile; lane l owns channels 2l, 2l+1 over the tile's 32 tokens. Key code of
// token t, channel c sits in word 8 (c/8 + 16 (t/8)) + t%8 at bit 4 (c%8): the two channels of lane l fill byte
// l%4 of that word, so the four lanes of a quad make one word, written once into LDS.
// SPARSE (dense-and-sparse groups; synthetic.wiki "KV cache quantization", section "What they report"): each
// channel's token of largest magnitude (the first on ties) is kept apart as its fp16 value and token index; min and
// max run over the other 31 tokens and the outlier's code is 0.
template <bool SPARSE>
__global__ __launch_bounds__(64) void quant_keys_b4_kernel(TokSrc src, int64_t t_begin, int kv_heads, uint8_t *tiles,
                                                           int64_t max_tiles, int64_t tile0) {
    __shared__ __align__(16) uint32_t words[512];
    const int l = threadIdx.x;
    const int64_t tile = blockIdx.x;
    const int h = blockIdx.y, b = blockIdx.z;
    uint8_t *rec = tiles + ((int64_t)(b * kv_heads + h) * max_tiles + tile0 + tile) * record_bytes<SPARSE>();

    if constexpr (!SPARSE) {   // packed binary16 pairs: min/max without conversion, x - z by one mixed fma
        uint32_t xw[32];
        load_pairs32_packed(src, t_begin + tile * 32, b, h, 2 * l, xw);
        h2v mn, mx;
        minmax_pairs32(xw, mn, mx);
        _Float16 s0, z0, s1, z1;
        group_params((float)mn[0], (float)mx[0], L4, s0, z0);
        group_params((float)mn[1], (float)mx[1], L4, s1, z1);
        const float fs0 = (float)s0, fz0 = (float)z0, fs1 = (float)s1, fz1 = (float)z1;
        const float rs0 = fs0 > 0.0f ? __builtin_amdgcn_rcpf(fs0) : 0.0f;   // s = 0: t' = 0, code 0
        const float rs1 = fs1 > 0.0f ? __builtin_amdgcn_rcpf(fs1) : 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const uint32_t c0 = code_from_diff(diff_half<false>(xw[i], fz0), fs0, rs0, 15u);
            const uint32_t c1 = code_from_diff(diff_half<true>(xw[i], fz1), fs1, rs1, 15u);
            const uint32_t word = quad_or((c0 | (c1 << 4)) << (8 * (l & 3)));
            const int w = 8 * ((l >> 2) + 16 * (i >> 3)) + (i & 7);
            if ((l & 3) == 0) words[w] = word;
        }
        __syncthreads();
        reinterpret_cast<uint4 *>(rec)[2 * l] = reinterpret_cast<const uint4 *>(words)[2 * l];
        reinterpret_cast<uint4 *>(rec)[2 * l + 1] = reinterpret_cast<const uint4 *>(words)[2 * l + 1];
        const h2 sp = {s0, s1}, zp = {z0, z1};
        reinterpret_cast<h2 *>(rec + K4_SCALE)[l] = sp;
        reinterpret_cast<h2 *>(rec + K4_ZERO)[l] = zp;
        return;
    }

    float x0[32], x1[32];
    load_pairs32(src, t_begin + tile * 32, b, h, 2 * l, x0, x1);
    int i0 = -1, i1 = -1;   // outlier tokens (SPARSE)
    float o0 = 0.0f, o1 = 0.0f;
    float mn0 = x0[0], mx0 = x0[0], mn1 = x1[0], mx1 = x1[0];
    if constexpr (SPARSE) {
        float b0 = __builtin_fabsf(x0[0]), b1 = __builtin_fabsf(x1[0]);
        i0 = 0; i1 = 0; o0 = x0[0]; o1 = x1[0];
#pragma unroll
        for (int i = 1; i < 32; ++i) {
            const float a0 = __builtin_fabsf(x0[i]), a1 = __builtin_fabsf(x1[i]);
            if (a0 > b0) { b0 = a0; i0 = i; o0 = x0[i]; }
            if (a1 > b1) { b1 = a1; i1 = i; o1 = x1[i]; }
        }
        const float inf = __builtin_inff();
        mn0 = inf; mx0 = -inf; mn1 = inf; mx1 = -inf;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            mn0 = fminf(mn0, i == i0 ? inf : x0[i]); mx0 = fmaxf(mx0, i == i0 ? -inf : x0[i]);
            mn1 = fminf(mn1, i == i1 ? inf : x1[i]); mx1 = fmaxf(mx1, i == i1 ? -inf : x1[i]);
        }
    } else {
#pragma unroll
        for (int i = 1; i < 32; ++i) {
            mn0 = fminf(mn0, x0[i]); mx0 = fmaxf(mx0, x0[i]);
            mn1 = fminf(mn1, x1[i]); mx1 = fmaxf(mx1, x1[i]);
        }
    }
    _Float16 s0, z0, s1, z1;
    group_params(mn0, mx0, L4, s0, z0);
    group_params(mn1, mx1, L4, s1, z1);
    const float fs0 = (float)s0, fz0 = (float)z0, fs1 = (float)s1, fz1 = (float)z1;
    const float rs0 = fs0 > 0.0f ? __builtin_amdgcn_rcpf(fs0) : 0.0f;   // s = 0: t' = 0, code 0
    const float rs1 = fs1 > 0.0f ? __builtin_amdgcn_rcpf(fs1) : 0.0f;
    // the word of token i and channels 8 (l/4) .. 8 (l/4) + 7 takes one byte from each lane of the quad: OR over
    // the quad, the quad's first lane writes it
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        uint32_t c0 = code_fast(x0[i], fz0, fs0, rs0, L4), c1 = code_fast(x1[i], fz1, fs1, rs1, L4);
        if constexpr (SPARSE) {
            c0 = i == i0 ? 0u : c0;
            c1 = i == i1 ? 0u : c1;
        }
        const uint32_t word = quad_or((c0 | (c1 << 4)) << (8 * (l & 3)));
        const int w = 8 * ((l >> 2) + 16 * (i >> 3)) + (i & 7);
        if ((l & 3) == 0) words[w] = word;
    }
    __syncthreads();
    reinterpret_cast<uint4 *>(rec)[2 * l] = reinterpret_cast<const uint4 *>(words)[2 * l];
    reinterpret_cast<uint4 *>(rec)[2 * l + 1] = reinterpret_cast<const uint4 *>(words)[2 * l + 1];
    const h2 sp = {s0, s1}, zp = {z0, z1};
    reinterpret_cast<h2 *>(rec + K4_SCALE)[l] = sp;
    reinterpret_cast<h2 *>(rec + K4_ZERO)[l] = zp;
    if constexpr (SPARSE) {
        const h2 op = {(_Float16)o0, (_Float16)o1};
        reinterpret_cast<h2 *>(rec + K4_OUT)[l] = op;
        reinterpret_cast<uint16_t *>(rec + K4_IDX)[l] = (uint16_t)(i0 | (i1 << 8));
    }
}

// Values: groups are 32 channels of one token. Parameters: lane l reduces the groups (token l / 4 and 16 + l / 4,
// channel group l % 4) from their own 64-byte rows (packed binary16 min/max) into {s, z, 1/s} per (token, group) in
// LDS. Codes: lane l owns channels 2l, 2l+1 (group l/16); the value code of channel c, token t sits in word
// 4c + t/8 at bit 4 (t%8), so lane l owns words 8l .. 8l+7 whole and builds them in registers.
// SPARSE: the group's outlier (largest magnitude, lowest channel on ties) is the maximum of an order key (|x| bits,
// then the lower channel, then the sign bit, which recovers the value); min/max over the other 31 elements run with
// the outlier's half replaced by the other half of its 32-bit word (an element of the same group, so the extremes
// are unchanged), and the outlier's code is 0.
template <bool SPARSE>
__global__ __launch_bounds__(64) void quant_values_b4_kernel(TokSrc src, int64_t t_begin, int kv_heads,
                                                             uint8_t *tiles, int64_t max_tiles, int64_t tile0) {
    __shared__ __align__(16) _Float16 sv[128], zv[128], ov[128];   // [g][t]
    __shared__ __align__(16) uint8_t oi[128];                        // [g][t]
    __shared__ __align__(16) float gp[512];                          // [t][g] {s, z, 1/s, 0}
    const int l = threadIdx.x;
    const int64_t tile = blockIdx.x;
    const int h = blockIdx.y, b = blockIdx.z;
    const int g = l >> 4;
    const uint32_t c0 = 2 * (l & 15);   // the lane's first channel within its group
    uint8_t *rec = tiles + ((int64_t)(b * kv_heads + h) * max_tiles + tile0 + tile) * record_bytes<SPARSE>();
    uint32_t xw[32];
    load_pairs32_packed(src, t_begin + tile * 32, b, h, 2 * l, xw);
    const int gq = l & 3;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int tk = (l >> 2) + 16 * k;
        const uint4 *row = reinterpret_cast<const uint4 *>(tok_row(src, b, h, t_begin + tile * 32 + tk) + 32 * gq);
        uint32_t rw[16];   // word e: channels 2e (low half) and 2e + 1 of the group
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 r = row[q];
            rw[4 * q] = r.x; rw[4 * q + 1] = r.y; rw[4 * q + 2] = r.z; rw[4 * q + 3] = r.w;
        }
        h2v mn = __builtin_bit_cast(h2v, rw[0]), mx = mn;
        if constexpr (SPARSE) {
            uint32_t kmax = 0u;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const uint32_t klo = ((rw[e] & 0x7FFFu) << 6) | ((31u - 2u * e) << 1) | ((rw[e] >> 15) & 1u);
                const uint32_t khi = (((rw[e] >> 16) & 0x7FFFu) << 6) | ((30u - 2u * e) << 1) | (rw[e] >> 31);
                kmax = max(kmax, max(klo, khi));
            }
            const uint32_t w = 31u - ((kmax >> 1) & 31u);
            const uint32_t sel = (w & 1u) ? 0x01000100u : 0x03020302u;   // both halves = the partner half
            ov[32 * gq + tk] = __builtin_bit_cast(_Float16, (uint16_t)(((kmax >> 6) & 0x7FFFu) | ((kmax & 1u) << 15)));
            oi[32 * gq + tk] = (uint8_t)w;
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if ((uint32_t)e == (w >> 1)) rw[e] = __builtin_amdgcn_perm(rw[e], rw[e], sel);
            mn = __builtin_bit_cast(h2v, rw[0]);
            mx = mn;
        }
#pragma unroll
        for (int e = 1; e < 16; ++e) {
            const h2v v = __builtin_bit_cast(h2v, rw[e]);
            mn = __builtin_elementwise_min(mn, v);
            mx = __builtin_elementwise_max(mx, v);
        }
        _Float16 sh, zh;
        group_params((float)__builtin_fminf16(mn[0], mn[1]), (float)__builtin_fmaxf16(mx[0], mx[1]), L4, sh, zh);
        sv[32 * gq + tk] = sh;
        zv[32 * gq + tk] = zh;
        const float fs = (float)sh;
        reinterpret_cast<f4 *>(gp)[4 * tk + gq] = f4{fs, (float)zh, fs > 0.0f ? __builtin_amdgcn_rcpf(fs) : 0.0f, 0.0f};
    }
    __syncthreads();
    uint32_t w[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const f4 prm = reinterpret_cast<const f4 *>(gp)[4 * i + g];
        uint32_t q0 = code_from_diff(diff_half<false>(xw[i], prm[1]), prm[0], prm[2], 15u);
        uint32_t q1 = code_from_diff(diff_half<true>(xw[i], prm[1]), prm[0], prm[2], 15u);
        if constexpr (SPARSE) {
            const uint32_t oc = oi[32 * g + i];
            q0 = oc == c0 ? 0u : q0;
            q1 = oc == c0 + 1 ? 0u : q1;
        }
        w[i >> 3] |= q0 << (4 * (i & 7));
        w[4 + (i >> 3)] |= q1 << (4 * (i & 7));
    }
    uint4 *dst = reinterpret_cast<uint4 *>(rec + V4_CODES);
    dst[2 * l] = uint4{w[0], w[1], w[2], w[3]};
    dst[2 * l + 1] = uint4{w[4], w[5], w[6], w[7]};
    reinterpret_cast<uint32_t *>(rec + V4_SCALE)[l] = reinterpret_cast<const uint32_t *>(sv)[l];
    reinterpret_cast<uint32_t *>(rec + V4_ZERO)[l] = reinterpret_cast<const uint32_t *>(zv)[l];
    if constexpr (SPARSE) {
        reinterpret_cast<uint32_t *>(rec + V4_OUT)[l] = reinterpret_cast<const uint32_t *>(ov)[l];
        reinterpret_cast<uint16_t *>(rec + V4_IDX)[l] = reinterpret_cast<const uint16_t *>(oi)[l];
    }
}

// Sink record of one slice from token 0 of the sources: the key copied as fp16 into bytes [0, 256), the value
// quantized per token (4 groups of 32 channels) with codes at byte 256 + c/2 (bit 4 (c%2)), scales at 320 + 2g,
// zeros at 328 + 2g; bytes [336, 512) zero. SPARSE: each value group's outlier value at 336 + 2g and its channel
// within the group at 344 + g (its code 0); zero from byte 348. One wavefront per slice, lane l owns channels 2l,
// 2l+1.
template <bool SPARSE>
__global__ __launch_bounds__(64) void sink_b4_kernel(TokSrc ksrc, TokSrc vsrc, int kv_heads, uint8_t *sink) {
    const int l = threadIdx.x;
    const int h = blockIdx.x, b = blockIdx.y;
    const int g = l >> 4;
    const uint32_t c0 = 2 * (l & 15);
    uint8_t *out = sink + (int64_t)(b * kv_heads + h) * SINK_REC;
    const _Float16 *krow = tok_row(ksrc, b, h, 0);
    const _Float16 *vrow = tok_row(vsrc, b, h, 0);
    reinterpret_cast<uint32_t *>(out)[l] = reinterpret_cast<const uint32_t *>(krow)[l];
    const h2 v = *reinterpret_cast<const h2 *>(vrow + 2 * l);
    const float a0 = (float)v[0], a1 = (float)v[1];
    bool is0 = false, is1 = false;
    uint32_t w = 0u;
    if constexpr (SPARSE) {
        const uint32_t k0 = outlier_key(a0, c0), k1 = outlier_key(a1, c0 + 1);
        w = 31u - (row16_max_u32(k0 > k1 ? k0 : k1) & 31u);
        is0 = w == c0;
        is1 = w == c0 + 1;
    }
    const float inf = __builtin_inff();
    float mn = fminf(is0 ? inf : a0, is1 ? inf : a1), mx = fmaxf(is0 ? -inf : a0, is1 ? -inf : a1);
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
        mn = fminf(mn, __shfl_xor(mn, off, 16));
        mx = fmaxf(mx, __shfl_xor(mx, off, 16));
    }
    _Float16 s, z;
    group_params(mn, mx, L4, s, z);
    const float fs = (float)s, fz = (float)z;
    const uint32_t q0 = is0 ? 0u : code_of(a0, fz, fs, L4), q1 = is1 ? 0u : code_of(a1, fz, fs, L4);
    out[256 + l] = (uint8_t)(q0 | (q1 << 4));
    if ((l & 15) == 0) {
        reinterpret_cast<_Float16 *>(out + 320)[g] = s;
        reinterpret_cast<_Float16 *>(out + 328)[g] = z;
    }
    if constexpr (SPARSE) {
        if (is0 || is1) {
            reinterpret_cast<_Float16 *>(out + SINK_VOUT)[g] = is0 ? v[0] : v[1];
            out[SINK_VIDX + g] = (uint8_t)w;
        }
        if (l < 41) reinterpret_cast<uint32_t *>(out + 348)[l] = 0u;
    } else {
        if (l < 44) reinterpret_cast<uint32_t *>(out + 336)[l] = 0u;
    }
}

// ------------------------------------------------------------------------------------------------ decode pass 1
namespace {

// sin(pi x) and cos(pi x) for x = hi + lo (|hi| < 2^21, |lo| small beside the reduced argument), inline and
// branch-free: hi = n/2 + r with n = rint(2 hi) and |r| <= 1/4 (r exact), y = pi (r + lo), the Taylor series of
// sin y and cos y to the y^9 and y^10 terms (the next terms are below 2^-28 for |y| <= pi/4), then the quarter turns
// n mod 4. Absolute error a few units of 2^-24.
__device__ __forceinline__ void sincospi2(float hi, float lo, float &sn, float &cs) {
    const float n = __builtin_rintf(2.0f * hi);
    const float y = (fmaf(n, -0.5f, hi) + lo) * 3.14159265358979323846f;
    const float y2 = y * y;
    float ps = fmaf(y2, 2.75573192239858906526e-6f, -1.98412698412698412698e-4f);
    ps = fmaf(y2, ps, 8.33333333333333333333e-3f);
    ps = fmaf(y2, ps, -1.66666666666666666667e-1f);
    const float sy = fmaf(y * y2, ps, y);
    float pc = fmaf(y2, -2.75573192239858906526e-7f, 2.48015873015873015873e-5f);
    pc = fmaf(y2, pc, -1.38888888888888888889e-3f);
    pc = fmaf(y2, pc, 4.16666666666666666667e-2f);
    pc = fmaf(y2, pc, -0.5f);
    const float cy = fmaf(y2, pc, 1.0f);
    const int q = (int)n;
    const float a = (q & 1) ? cy : sy, b = (q & 1) ? sy : cy;   // sin, cos of y + (q & 1) pi/2, up to sign
    sn = (q & 2) ? -a : a;
    cs = ((q + 1) & 2) ? -b : b;
}

// cos and sin of pi * m * thp: the product reduced modulo 2 into [-1, 1] in binary64 (m up to 2^31), then passed
// on as a binary32 pair, so the argument keeps about 2^-48 absolute precision instead of binary32's 2^-25
__device__ __forceinline__ void half_turns(double m, double thp, float &c, float &s) {
    double t = m * thp;
    t -= 2.0 * __builtin_rint(0.5 * t);
    const float hi = (float)t;
    sincospi2(hi, (float)(t - (double)hi), s, c);
}

// Two 4-bit codes held in bytes 2 sel and 2 sel + 1 of w (each byte < 16) as exact fp32 values: a byte b < 16
// read as fp8 e4m3 is b * 2^-9 (subnormal for b < 8, exponent 1 otherwise), and the converter's scale 2^9 makes it b.
typedef float f2 __attribute__((ext_vector_type(2)));
template <bool SEL>
__device__ __forceinline__ f2 codes2(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 512.0f, SEL);
}

__device__ __forceinline__ f4 mfma(h8 a, h8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }

// Eight 4-bit codes of one word as fp16, in the order of nibbles 0, 2, 4, 6, 1, 3, 5, 7. The even and odd nibbles
// are spread into bytes; a byte b < 16 read as an fp8 e4m3 value is b * 2^-9 (subnormal for b < 8, exponent 1
// otherwise), so the gfx950 fp8 converter with scale 2^9 yields b exactly.
__device__ __forceinline__ h8 expand8_b4(uint32_t w) {
    const uint32_t ev = w & 0x0F0F0F0Fu, od = (w >> 4) & 0x0F0F0F0Fu;
    const h2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(ev, 512.0f, false);
    const h2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(ev, 512.0f, true);
    const h2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(od, 512.0f, false);
    const h2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(od, 512.0f, true);
    h8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
    return r;
}

// x = (pa * sa.lo, pb * sb.lo) (HI: the high halves of sa, sb), hi = RN16(x), then RN16(x - w hi) packed: the high
// parts for w = 0, the low parts (x - hi is exact) for w = 1. x in binary32 (one mixed-precision fma each), hi by one
// packed conversion, x - w hi by mixed fmas that read hi's halves, the result by a second packed conversion (six
// instructions at the full vector rate).
template <bool HI>
__device__ __forceinline__ uint32_t split_part(float pa, float pb, uint32_t sa, uint32_t sb, float w) {
    uint32_t part, hi;
    float x0, x1;
    if constexpr (HI)
        asm("v_fma_mix_f32 %1, %4, %6, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]\n\t"
            "v_fma_mix_f32 %2, %5, %7, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]\n\t"
            "v_cvt_pk_f16_f32 %3, %1, %2\n\t"
            "v_fma_mix_f32 %1, -%3, %8, %1 op_sel_hi:[1,0,0]\n\t"
            "v_fma_mix_f32 %2, -%3, %8, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
            "v_cvt_pk_f16_f32 %0, %1, %2"
            : "=&v"(part), "=&v"(x0), "=&v"(x1), "=&v"(hi)
            : "v"(pa), "v"(pb), "v"(sa), "v"(sb), "v"(w));
    else
        asm("v_fma_mix_f32 %1, %4, %6, 0 op_sel_hi:[0,1,0]\n\t"
            "v_fma_mix_f32 %2, %5, %7, 0 op_sel_hi:[0,1,0]\n\t"
            "v_cvt_pk_f16_f32 %3, %1, %2\n\t"
            "v_fma_mix_f32 %1, -%3, %8, %1 op_sel_hi:[1,0,0]\n\t"
            "v_fma_mix_f32 %2, -%3, %8, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
            "v_cvt_pk_f16_f32 %0, %1, %2"
            : "=&v"(part), "=&v"(x0), "=&v"(x1), "=&v"(hi)
            : "v"(pa), "v"(pb), "v"(sa), "v"(sb), "v"(w));
    return part;
}

}  // namespace

// One wavefront per (batch row, query head, token split). Virtual tiles of a slice: the quantized tiles
// 0 .. n_qtiles - 1, then the window tiles (32 rows each, the last one partial); token u of virtual tile v sits at
// absolute position n_sink + 32 v + u. Split 0 also takes the sink token (position 0) when there is one.
//
// Staging. Quantized tiles are copied whole into an LDS ring of three 5120-byte slots by global-to-LDS DMA, two
// tiles ahead of the one being computed, so a wavefront keeps up to 10 KB of loads in flight without spending
// registers on them. The key codes are scattered on the way in so that lane l later reads its 32 bytes as two
// bank-conflict-free 16-byte reads.
//
// Scores (VALU). Lane l = pq + 16 to owns channels 8pq .. 8pq+7 (rotation pairs i = 4pq .. 4pq+3) of tokens
// 8to .. 8to+7: key-code words 8l .. 8l+7. For a pair (x0, x1) of codes with per-channel scales (s0, s1) and zeros
// (z0, z1), and the query pair (q0, q1) rotated back by the tile start position m0 (qr = R(-m0 theta) q), the
// pair's share of the score of token u is
//     cos(u theta) (a0 x0 + a1 x1 + alpha) + sin(u theta) (b0 x0 + b1 x1 + beta)
// with a0 = qr0 s0, a1 = qr1 s1, alpha = qr0 z0 + qr1 z1, b0 = qr1 s0, b1 = -qr0 s1, beta = qr1 z0 - qr0 z1: the
// dot product of the query with the dequantized key rotated by m0 + u, expanded by angle addition. Lane l computes the
// six coefficients of pair l once per tile and shares them through LDS. The cos/sin of u theta for a lane's 32 (token,
// pair) combinations are the same for every tile and stay in registers; the rotation by the tile start advances by 32
// theta per tile (recomputed from the position every 16 tiles). Window tiles use the same expansion with the fp16 keys
// (s = 1, z = 0). Partial sums of the 16 lanes of a token are added through LDS. The query carries the softmax scale
// times log2(e), so scores are in the log2 domain.
//
// Softmax. Lagged maximum: the running maximum is raised (and every accumulator rescaled) only when some score of
// the tile exceeds it.
//
// PV (MFMA). 16x16x32 fp16: B = the value codes of 16 channels (column n = channel 16j + n) and the tile's 32
// tokens, one code word per lane (expanded exactly by the fp8 converter); A row g = the fp16 high part of
// p~[t] = p[t] s_V[g][t] for value group g and row 4 + g its low part (rows 8..15 are zero), one MFMA per channel
// block. For channel block j only rows g = j/2 and 4 + g are kept, and they are added once per split. The
// zero-point term sum_t p z_V[g][t] is accumulated on the VALU; window tiles and the sink add their values on the
// VALU.
//
// Dense-and-sparse records (SPARSE). The outlier of a key channel's group decodes as its zero point z (code 0), so
// the score of its token u misses d (dq/dk_c) with d = o - z: for pair l this is d (cos(u theta) qr0 + sin(u theta)
// qr1) for the even channel and d (cos(u theta) qr1 - sin(u theta) qr0) for the odd one. Lane l computes the two
// corrections of pair l with the tile's coefficients; a value outlier adds p[t] (o - z) to its channel. Both are
// scattered (to tokens, to channels) through LDS as exact integer sums: each correction is split against a power of
// two 2^K above every correction it can be, x = H 2^(K-23) + L 2^(K-46) with integers |H|, |L| < 2^23 (error below
// 2^(K-46)), and H and L are added with integer LDS atomics (a float LDS atomic costs some thirty times an integer
// one on this chip). The bounds need no per-tile reduction: |o - z| <= 2 * 65504 for binary16 o and z, a rotation
// keeps the length of a query pair, and p <= 1 under the lagged maximum, so 2^K comes from the wavefront's largest
// query pair (keys) or is 2^17 (values); the resolution 2^(K-46) stays far below binary32 rounding of a score or an
// output. Integer sums do not depend on the order of the adds, so the result is deterministic. The sink's value
// outliers replace the decoded value of their channels.
namespace {
constexpr int NBUF = 3;   // LDS ring slots (tiles in flight + the one being computed)
template <bool SPARSE>
struct B4Lds {
    static constexpr int REC = record_bytes<SPARSE>();
    static constexpr int RING = 0;                  // [NBUF][REC]: K codes scattered (see dma_tile), rest as stored
    static constexpr int RED = NBUF * REC;          // f32 rows of 16 (one per token, row 9 (u/8) + u%8); reused for
                                                    // the output at the end
    static constexpr int PBUF = RED + 36 * 64;      // f32 [32]; reused for the zero-point sums at the end
    // f32x4 [4 (pair % 4)][16 (pair / 4)]: a0 a1 alpha b0, and f32x2 [4][16]: b1 beta. Dense records: after PBUF.
    // Sparse records (the ring is larger): inside RED, whose rows are dead while the coefficients are shared.
    static constexpr int COEF4 = SPARSE ? RED : PBUF + 128;
    static constexpr int COEF2 = COEF4 + 1024;
    // SPARSE: value-outlier sums, int32 (H, L) [128 channels], inside RED (used between P V and the coefficients);
    // key-outlier sums, int32 (H, L) [32 tokens], filled with the coefficients and read by the next softmax step
    static constexpr int VACC = RED;
    static constexpr int KACC = PBUF + 128;
    // f32 [32] zeros: the P V operand's unused rows (4..15) read their probabilities here
    static constexpr int ZERO = SPARSE ? KACC + 256 : COEF2 + 512;
    static constexpr int BYTES = ZERO + 128;
    static constexpr int ND = SPARSE ? 6 : 5;       // LDS-DMA loads per tile
    static constexpr int NC = SPARSE ? 2 : 1;       // the first NC of them hold what the coefficients need
};
static_assert(B4Lds<true>::COEF2 + 512 <= B4Lds<true>::PBUF && B4Lds<true>::VACC + 1024 <= B4Lds<true>::PBUF,
              "coefficients and value sums inside the reduction rows");
static_assert(B4Lds<true>::BYTES <= 20480 && B4Lds<false>::BYTES <= 20480, "eight wavefronts per CU");

__device__ __forceinline__ void lds_add(int32_t *p, int32_t v) {
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ float exp2i(int n) { return __builtin_bit_cast(float, (uint32_t)(n + 127) << 23); }

// Fixed-point parts of values x against 2^K > m (m = the wavefront's largest |x|, K clamped to [-60, 100] so every
// factor below is a normal binary32 power of two): x = H 2^(K-23) + L 2^(K-46) + e, |H|, |L| < 2^23, |e| < 2^(K-46).
// x 2^(23-K) and H 2^(K-23) are exact, and so is the remainder x - H 2^(K-23) (it keeps the low bits of x).
struct FixScale {
    float f1, f2, g1, g2;   // 2^(23-K), 2^(46-K), 2^(K-23), 2^(K-46)
};
__device__ __forceinline__ FixScale fix_scale(float m) {
    int K = (int)((__builtin_bit_cast(uint32_t, m) >> 23) & 0xFFu) - 126;
    K = K < -60 ? -60 : (K > 100 ? 100 : K);
    return FixScale{exp2i(23 - K), exp2i(46 - K), exp2i(K - 23), exp2i(K - 46)};
}
__device__ __forceinline__ void fix_split(float x, const FixScale &f, int32_t &H, int32_t &L) {
#pragma clang fp contract(off)
    H = (int32_t)(x * f.f1);
    const float r = fmaf(-(float)H, f.g1, x);
    L = (int32_t)(r * f.f2);
}
__device__ __forceinline__ float fix_join(int32_t H, int32_t L, const FixScale &f) {
    return fmaf((float)H, f.g1, (float)L * f.g2);
}
constexpr float OUTLIER_SPAN = 131008.0f;   // |o - z| <= 2 * 65504 for binary16 o, z
}  // namespace

template <bool ROPE, bool SPARSE>
__global__ __launch_bounds__(64) void decode_b4_pass1_kernel(DecodeB4Args a) {
    typedef B4Lds<SPARSE> L;
    constexpr int REC = L::REC;
    __shared__ __align__(16) unsigned char smem[L::BYTES];
    float *red = reinterpret_cast<float *>(smem + L::RED);
    float *pbuf = reinterpret_cast<float *>(smem + L::PBUF);
    if (threadIdx.x < 32) reinterpret_cast<float *>(smem + L::ZERO)[threadIdx.x] = 0.0f;
    float4 *coef4 = reinterpret_cast<float4 *>(smem + L::COEF4);
    float2 *coef2 = reinterpret_cast<float2 *>(smem + L::COEF2);
    const uint32_t ring_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char *)smem + L::RING;

    const int l = threadIdx.x;
    const int pq = l & 15, to = l >> 4;
    const int n = l & 15, kg = l >> 4;
    const int u = l >> 1, uh = l & 1;
    const int bh = blockIdx.x;
    const int split = blockIdx.y;
    const int S = gridDim.y;
    // the workgroup's indices and tile range are uniform: kept in scalar registers (integer division runs on the
    // vector unit, and its results would otherwise make the tile loop's counter, branches and addresses vector work)
    auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
    const int b = uni(bh / a.q_heads), hq = uni(bh - b * a.q_heads);
    const int G = a.q_heads / a.kv_heads;
    const int64_t slice = (int64_t)b * a.kv_heads + uni(hq / G);
    const int n_vt = a.n_qtiles + (a.n_resid + 31) / 32;
    const int v0 = uni(split * a.tiles_per_split);
    const int v1 = uni(min(n_vt, v0 + a.tiles_per_split));
    const float C = a.sm_log2;
    const float NEG_INF = -__builtin_inff();

    // ---- query pair l (channels 2l, 2l+1) in log2 units: the pair whose coefficients this lane computes
    const _Float16 *qrow = a.q + (int64_t)bh * HD;
    const h2 qq = reinterpret_cast<const h2 *>(qrow)[l];
    const float qp0 = C * (float)qq[0], qp1 = C * (float)qq[1];

    // ---- rotation state: cos/sin of (8to + t) theta_i for the lane's score pairs i = 4pq + j (fixed tables); the
    // tile-start rotation of pair l and its per-tile step
    float tc[8][4], ts[8][4], ec = 1.0f, es = 0.0f, rc = 1.0f, rs = 0.0f;
    double thl = 0.0;   // theta_l / pi
    float thl_hi = 0.0f, thl_lo = 0.0f;   // theta_l / pi as hi (14 significant bits, so u * hi is exact) + lo
    if constexpr (ROPE) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const double th = exp2(-(2.0 * (4 * pq + j) / HD) * a.log2_base) * 0.31830988618379067154;
            float c1, s1;
            half_turns(1.0, th, c1, s1);
            half_turns(8.0 * to, th, tc[0][j], ts[0][j]);
#pragma unroll
            for (int t = 1; t < 8; ++t) {
                tc[t][j] = tc[t - 1][j] * c1 - ts[t - 1][j] * s1;
                ts[t][j] = ts[t - 1][j] * c1 + tc[t - 1][j] * s1;
            }
        }
        thl = exp2(-(2.0 * l / HD) * a.log2_base) * 0.31830988618379067154;
        thl_hi = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, (float)thl) & 0xFFFFFC00u);
        thl_lo = (float)(thl - (double)thl_hi);
        half_turns(32.0, thl, rc, rs);
        half_turns((double)a.n_sink + 32.0 * v0, thl, ec, es);
    }
    auto advance = [&](int v_next) {   // rotation of pair l for the start of tile v_next
        if constexpr (ROPE) {
            if (((v_next - v0) & 15) == 0) {
                half_turns((double)a.n_sink + 32.0 * v_next, thl, ec, es);
            } else {
                const float c = ec * rc - es * rs;
                es = es * rc + ec * rs;
                ec = c;
            }
        }
    };

    // coefficients of pair l for the current tile (scales/zeros of its two channels) -> LDS; then the lane's four
    // score pairs are read back
    float a0[4], a1[4], al[4], b0[4], b1[4], be[4];
    auto share_coefficients = [&](float s0, float s1, float z0, float z1, float &r0, float &r1) {
        r0 = qp0 * ec + qp1 * es;
        r1 = qp1 * ec - qp0 * es;
        const int at = (l & 3) * 16 + (l >> 2);
        coef4[at] = float4{r0 * s0, r1 * s1, r0 * z0 + r1 * z1, r1 * s0};
        coef2[at] = float2{-(r0 * s1), r1 * z0 - r0 * z1};
        wave_lds_order();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 c0 = coef4[j * 16 + pq];
            const float2 c1 = coef2[j * 16 + pq];
            a0[j] = c0.x; a1[j] = c0.y; al[j] = c0.z; b0[j] = c0.w; b1[j] = c1.x; be[j] = c1.y;
        }
    };

    // partial score of token 8to + t from x pairs (x0, x1) of the lane's four pairs
    auto token_score = [&](int t, const float (&x0)[4], const float (&x1)[4]) -> float {
        if constexpr (ROPE) {
            float sacc = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float P = fmaf(a1[j], x1[j], fmaf(a0[j], x0[j], al[j]));
                const float Q = fmaf(b1[j], x1[j], fmaf(b0[j], x0[j], be[j]));
                sacc = (j == 0) ? fmaf(tc[t][0], P, ts[t][0] * Q) : fmaf(tc[t][j], P, fmaf(ts[t][j], Q, sacc));
            }
            return sacc;
        } else {
            float sacc = (al[0] + al[1]) + (al[2] + al[3]);
#pragma unroll
            for (int j = 0; j < 4; ++j) sacc = fmaf(a1[j], x1[j], fmaf(a0[j], x0[j], sacc));
            return sacc;
        }
    };

    // ---- online softmax state
    float m = NEG_INF, lsum = 0.0f, gam = 0.0f, ws = 0.0f, ow0 = 0.0f, ow1 = 0.0f, vs0 = 0.0f, vs1 = 0.0f;
    f4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f4{0.0f, 0.0f, 0.0f, 0.0f};

    if (split == 0 && a.n_sink) {   // sink token at position 0 (no rotation); lane l: channels 2l, 2l+1
        const uint8_t *sk = a.sink + slice * SINK_REC;
        const h2 kk = reinterpret_cast<const h2 *>(sk)[l];
        const float d = rows_sum(row16_sum(qp0 * (float)kk[0] + qp1 * (float)kk[1]));
        const uint32_t byte = sk[256 + l];
        const int g = l >> 4;
        const float s = (float)reinterpret_cast<const _Float16 *>(sk + 320)[g];
        const float z = (float)reinterpret_cast<const _Float16 *>(sk + 328)[g];
        vs0 = fmaf((float)(byte & 15u), s, z);
        vs1 = fmaf((float)(byte >> 4), s, z);
        if constexpr (SPARSE) {   // the group's outlier replaces its channel's decoded value
            const float so = (float)reinterpret_cast<const _Float16 *>(sk + SINK_VOUT)[g];
            const uint32_t si = sk[SINK_VIDX + g] & 31u, c0 = 2 * (l & 15);
            vs0 = si == c0 ? so : vs0;
            vs1 = si == c0 + 1 ? so : vs1;
        }
        m = d;
        ws = 1.0f;
        lsum = (l == 0) ? 1.0f : 0.0f;
    }

    // partial scores -> full score of token u in lanes 2u, 2u+1 (tokens >= nv masked), then the softmax step
    // SPARSE: key-outlier score corrections of the coming tile, per token as int32 (H, L) in KACC; their scale bounds
    // |o - z| |query pair| over the wavefront, the value corrections' bounds p |o - z|
    int2 *kacc = reinterpret_cast<int2 *>(smem + L::KACC);
    FixScale kfix{0.0f, 0.0f, 0.0f, 0.0f}, vfix{0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (SPARSE) {
        kfix = fix_scale(OUTLIER_SPAN * sqrtf(rows_max(row16_max(qp0 * qp0 + qp1 * qp1))));
        vfix = fix_scale(OUTLIER_SPAN);
        if (l < 32) kacc[l] = int2{0, 0};
        wave_lds_order();
    }
    auto softmax_step = [&](const float (&part)[8], int nv, bool key_outliers) {
        // token 8to + t in row 9to + t: the 16 lanes of each `to` group land in distinct banks
#pragma unroll
        for (int t = 0; t < 8; ++t) red[(9 * to + t) * 16 + pq] = part[t];
        wave_lds_order();
        const float *rr = red + (9 * (u >> 3) + (u & 7)) * 16 + 4 * uh;   // partials 4uh..4uh+3 and 8+4uh..11+4uh
        const float4 r0 = *reinterpret_cast<const float4 *>(rr);
        const float4 r1 = *reinterpret_cast<const float4 *>(rr + 8);
        float s = ((r0.x + r0.y) + (r0.z + r0.w)) + ((r1.x + r1.y) + (r1.z + r1.w));
        s = dpp_xadd<DPP_QUAD_1032>(s);
        if constexpr (SPARSE) {
            if (key_outliers) {   // token u's key-outlier sum, then cleared for the next tile
                const int2 hl = kacc[u];
                s += fix_join(hl.x, hl.y, kfix);
                wave_lds_order();
                if (uh == 0) kacc[u] = int2{0, 0};
            }
        }
        if (u >= nv) s = NEG_INF;
        if (__any(s > m)) {
            const float mn = fmaxf(m, rows_max(row16_max(s)));
            const float sc = __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] *= sc;
            gam *= sc; lsum *= sc; ws *= sc; ow0 *= sc; ow1 *= sc;
            m = mn;
        }
        const float p = __builtin_amdgcn_exp2f(s - m);
        lsum += uh ? 0.0f : p;
        pbuf[u] = p;
        wave_lds_order();
    };

    const uint8_t *recs = a.tiles + slice * a.max_tiles * REC;
    const int vq_end = min(v1, a.n_qtiles);

    // one tile record -> ring slot, scales and zeros first (the coefficients of a tile need only those): key-code
    // bytes [32 l, 32 l + 16) go to slot + 16 l and [32 l + 16, 32 l + 32) to slot + 1024 + 16 l; value codes,
    // scales and zeros at their record offsets
    // SPARSE: the outlier section (768 bytes, lanes 0..47) right after the scales
    auto dma_tile = [&](int v, int slot) {   // v and slot are uniform: the record base stays in scalar registers
        const uint64_t rec = reinterpret_cast<uint64_t>(recs + (int64_t)v * REC);
        const uint32_t base = ring_base + slot * REC;
        lds_dma16_s(rec + K4_SCALE, 16 * l, base + K4_SCALE);
        if constexpr (SPARSE) {
            if (l < 48) lds_dma16_s(rec + K4_OUT, 16 * l, base + K4_OUT);
        }
        lds_dma16_s(rec, 32 * l, base);
        lds_dma16_s(rec + 16, 32 * l, base + 1024);
        lds_dma16_s(rec + V4_CODES, 16 * l, base + V4_CODES);
        lds_dma16_s(rec + V4_CODES + 1024, 16 * l, base + V4_CODES + 1024);
    };
    auto tile_coefficients = [&](int slot) {
        const unsigned char *tl = smem + L::RING + slot * REC;
        const h2 skp = reinterpret_cast<const h2 *>(tl + K4_SCALE)[l];
        const h2 zkp = reinterpret_cast<const h2 *>(tl + K4_ZERO)[l];
        const float z0 = (float)zkp[0], z1 = (float)zkp[1];
        float r0, r1;
        share_coefficients((float)skp[0], (float)skp[1], z0, z1, r0, r1);
        if constexpr (SPARSE) {   // key outliers of channels 2l, 2l+1
            const h2 kop = reinterpret_cast<const h2 *>(tl + K4_OUT)[l];
            const uint32_t ki = reinterpret_cast<const uint16_t *>(tl + K4_IDX)[l];
            const uint32_t u0 = ki & 31u, u1 = (ki >> 8) & 31u;
            const float d0 = (float)kop[0] - z0, d1 = (float)kop[1] - z1;
            float kc0, kc1;
            if constexpr (ROPE) {
                float c0, s0, c1, s1;
                sincospi2((float)u0 * thl_hi, (float)u0 * thl_lo, s0, c0);
                sincospi2((float)u1 * thl_hi, (float)u1 * thl_lo, s1, c1);
                kc0 = d0 * fmaf(c0, r0, s0 * r1);
                kc1 = d1 * fmaf(c1, r1, -(s1 * r0));
            } else {
                kc0 = d0 * r0;
                kc1 = d1 * r1;
            }
            int32_t h0, l0, h1, l1;
            fix_split(kc0, kfix, h0, l0);
            fix_split(kc1, kfix, h1, l1);
            int32_t *ka = reinterpret_cast<int32_t *>(kacc);
            wave_lds_order();
            lds_add(ka + 2 * u0, h0);
            lds_add(ka + 2 * u0 + 1, l0);
            lds_add(ka + 2 * u1, h1);
            lds_add(ka + 2 * u1 + 1, l1);
        }
    };

    // ---- quantized tiles: two tiles in flight; the coefficients of tile v + 1 are shared at the end of
    // iteration v (after its scales, the first chunk of its DMA, have landed)
    int v = v0;
    if (v < vq_end) {
        dma_tile(v, 0);
        if (v + 1 < vq_end) {
            dma_tile(v + 1, 1);
            wait_vmcnt<2 * L::ND - L::NC>();
        } else {
            wait_vmcnt<L::ND - L::NC>();
        }
        tile_coefficients(0);
        advance(v + 1);
    }
    int slot = 0;
    for (; v < vq_end; ++v) {
        // issue tile v + 2 into the slot tile v - 1 used (its reads are complete), then wait for tile v (DMA loads
        // complete in order)
        const bool ahead2 = v + 2 < vq_end, ahead1 = v + 1 < vq_end;
        if (ahead2) {
            dma_tile(v + 2, slot == 0 ? 2 : slot - 1);
            wait_vmcnt<2 * L::ND>();
        } else if (ahead1) {
            wait_vmcnt<L::ND>();
        } else {
            wait_vmcnt<0>();
        }
        const unsigned char *tl = smem + L::RING + slot * REC;
        slot = (slot == NBUF - 1) ? 0 : slot + 1;

        const uint4 k03 = reinterpret_cast<const uint4 *>(tl)[l];
        const uint4 k47 = reinterpret_cast<const uint4 *>(tl + 1024)[l];
        const uint32_t kw[8] = {k03.x, k03.y, k03.z, k03.w, k47.x, k47.y, k47.z, k47.w};
        float part[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            // even channels in the bytes of ev, odd channels in the bytes of od; two bytes per fp8 convert
            const uint32_t ev = kw[t] & 0x0F0F0F0Fu, od = (kw[t] >> 4) & 0x0F0F0F0Fu;
            const f2 e01 = codes2<false>(ev), e23 = codes2<true>(ev), o01 = codes2<false>(od), o23 = codes2<true>(od);
            const float x0[4] = {e01[0], e01[1], e23[0], e23[1]};
            const float x1[4] = {o01[0], o01[1], o23[0], o23[1]};
            part[t] = token_score(t, x0, x1);
        }
        softmax_step(part, 32, true);

        // SPARSE: value outliers of entries 2l, 2l+1 ([g][t]): p[t] (o - z) into channel 32 g + idx, added into the
        // (H, L) sums before P V and read back after it, so the adds complete under the MFMAs
        int32_t *vacc = reinterpret_cast<int32_t *>(smem + L::VACC);
        if constexpr (SPARSE) {
            const h2 vo = reinterpret_cast<const h2 *>(tl + V4_OUT)[l];
            const h2 vz = reinterpret_cast<const h2 *>(tl + V4_ZERO)[l];
            const uint32_t vi = reinterpret_cast<const uint16_t *>(tl + V4_IDX)[l];
            const float2 pp = reinterpret_cast<const float2 *>(pbuf)[l & 15];
            const float w0 = pp.x * ((float)vo[0] - (float)vz[0]), w1 = pp.y * ((float)vo[1] - (float)vz[1]);
            int32_t h0, l0, h1, l1;
            fix_split(w0, vfix, h0, l0);
            fix_split(w1, vfix, h1, l1);
            int32_t *cg = vacc + 2 * 32 * (l >> 4);
            wave_lds_order();
            reinterpret_cast<int4 *>(vacc)[l] = int4{0, 0, 0, 0};
            wave_lds_order();
            lds_add(cg + 2 * (vi & 31u), h0);
            lds_add(cg + 2 * (vi & 31u) + 1, l0);
            lds_add(cg + 2 * ((vi >> 8) & 31u), h1);
            lds_add(cg + 2 * ((vi >> 8) & 31u) + 1, l1);
        }

        // PV: A row g = the high part of p~ of value group g, row 4 + g its low part, over tokens 8kg .. 8kg+7 in the
        // expand8_b4 order (t0 t2 t4 t6 t1 t3 t5 t7); rows 8..15 (outputs never used) are zero: zero operands draw
        // less power than repeated ones
        const int gA = n & 3;
        const float *pz = n < 8 ? pbuf : reinterpret_cast<const float *>(smem + L::ZERO);
        const float wpart = n < 4 ? 0.0f : 1.0f;
        const uint4 svr = *reinterpret_cast<const uint4 *>(tl + V4_SCALE + 2 * (32 * gA + 8 * kg));
        const h8 zvh = __builtin_bit_cast(h8, *reinterpret_cast<const uint4 *>(tl + V4_ZERO + 2 * (32 * gA + 8 * kg)));
        const float4 pa = *reinterpret_cast<const float4 *>(pz + 8 * kg);
        const float4 pb = *reinterpret_cast<const float4 *>(pz + 8 * kg + 4);
        const h8 A = __builtin_bit_cast(h8, uint4{split_part<false>(pa.x, pa.z, svr.x, svr.y, wpart),
                                                  split_part<false>(pb.x, pb.z, svr.z, svr.w, wpart),
                                                  split_part<true>(pa.y, pa.w, svr.x, svr.y, wpart),
                                                  split_part<true>(pb.y, pb.w, svr.z, svr.w, wpart)});
        // (lanes 4..7 repeat the zero-point sums of lanes 0..3; only those of lanes 0..3 are stored at the end)
        gam += ((pa.x * (float)zvh[0] + pa.y * (float)zvh[1]) + (pa.z * (float)zvh[2] + pa.w * (float)zvh[3])) +
               ((pb.x * (float)zvh[4] + pb.y * (float)zvh[5]) + (pb.z * (float)zvh[6] + pb.w * (float)zvh[7]));
        const uint32_t *vwl = reinterpret_cast<const uint32_t *>(tl + V4_CODES);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = mfma(A, expand8_b4(vwl[4 * (16 * j + n) + kg]), acc[j]);
        if constexpr (SPARSE) {   // the value-outlier sums of channels 2l, 2l+1
            wave_lds_order();
            const int4 cv = reinterpret_cast<const int4 *>(vacc)[l];
            ow0 += fix_join(cv.x, cv.y, vfix);
            ow1 += fix_join(cv.z, cv.w, vfix);
        }
        if (ahead1) {   // coefficients of tile v + 1: its first NC loads are the oldest still counted
            if (ahead2)
                wait_vmcnt<2 * L::ND - L::NC>();
            else
                wait_vmcnt<L::ND - L::NC>();
            tile_coefficients(slot);
            advance(v + 2);
        }
    }

    // ---- window tiles (fp16 rows; keys rotated like the quantized ones)
    for (; v < v1; ++v) {
        const int w = v - a.n_qtiles;
        const int nv = min(32, a.n_resid - 32 * w);
        const _Float16 *kr = a.k_res + (slice * a.res_cap + 32 * w) * HD;
        const _Float16 *vr = a.v_res + (slice * a.res_cap + 32 * w) * HD;
        h8 kx[8];
#pragma unroll
        for (int t = 0; t < 8; ++t)
            kx[t] = __builtin_bit_cast(h8, *reinterpret_cast<const uint4 *>(kr + (8 * to + t) * HD + 8 * pq));
        float r0, r1;
        share_coefficients(1.0f, 1.0f, 0.0f, 0.0f, r0, r1);
        advance(v + 1);
        float part[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            float x0[4], x1[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x0[j] = (float)kx[t][2 * j];
                x1[j] = (float)kx[t][2 * j + 1];
            }
            part[t] = token_score(t, x0, x1);
        }
        softmax_step(part, nv, false);
        for (int t = 0; t < nv; ++t) {   // lane l: channels 2l, 2l+1
            const float p = pbuf[t];
            const h2 vv = reinterpret_cast<const h2 *>(vr + t * HD)[l];
            ow0 = fmaf(p, (float)vv[0], ow0);
            ow1 = fmaf(p, (float)vv[1], ow1);
        }
    }

    // ---- partials of this split: channel 16j + n of the MFMA sums is the high-part row j / 2 in acc[j][j / 2] of
    // lane n plus the low-part row 4 + j / 2 in the same register of lane 16 + n
    float *obuf = red;
    float *gbuf = pbuf;
    lsum = rows_sum(row16_sum(lsum));
    gam = rows_sum(gam);   // lane n (any row): value group n & 3
    wave_lds_order();
    if (l < 32) {
#pragma unroll
        for (int j = 0; j < 8; ++j) obuf[128 * (l >> 4) + 16 * j + (l & 15)] = acc[j][j >> 1];
    }
    if (l < 4) gbuf[l] = gam;
    wave_lds_order();
    const float2 oh = reinterpret_cast<const float2 *>(obuf)[l];
    const float2 olo = reinterpret_cast<const float2 *>(obuf)[64 + l];
    const float2 ov = {oh.x + olo.x, oh.y + olo.y};
    const float gz = gbuf[l >> 4];
    const int64_t row = (int64_t)bh * S + split;
    float2 res;
    res.x = ov.x + gz + ws * vs0 + ow0;
    res.y = ov.y + gz + ws * vs1 + ow1;
    reinterpret_cast<float2 *>(a.part_o + row * HD)[l] = res;
    if (l == 0) {
        a.part_ml[2 * row] = m;
        a.part_ml[2 * row + 1] = lsum;
    }
}

// ------------------------------------------------------------------------------------------------ launchers
hipError_t launch_quant_keys_b4(const TokSrc &src, int64_t t_begin, int64_t n_tiles, int batch, int kv_heads,
                                uint8_t *tiles, int64_t max_tiles, int64_t tile0, bool sparse, hipStream_t st) {
    dim3 grid((unsigned)n_tiles, (unsigned)kv_heads, (unsigned)batch);
    if (sparse)
        hipLaunchKernelGGL(quant_keys_b4_kernel<true>, grid, dim3(64), 0, st, src, t_begin, kv_heads, tiles,
                           max_tiles, tile0);
    else
        hipLaunchKernelGGL(quant_keys_b4_kernel<false>, grid, dim3(64), 0, st, src, t_begin, kv_heads, tiles,
                           max_tiles, tile0);
    return hipGetLastError();
}

hipError_t launch_quant_values_b4(const TokSrc &src, int64_t t_begin, int64_t n_tiles, int batch, int kv_heads,
                                  uint8_t *tiles, int64_t max_tiles, int64_t tile0, bool sparse, hipStream_t st) {
    dim3 grid((unsigned)n_tiles, (unsigned)kv_heads, (unsigned)batch);
    if (sparse)
        hipLaunchKernelGGL(quant_values_b4_kernel<true>, grid, dim3(64), 0, st, src, t_begin, kv_heads, tiles,
                           max_tiles, tile0);
    else
        hipLaunchKernelGGL(quant_values_b4_kernel<false>, grid, dim3(64), 0, st, src, t_begin, kv_heads, tiles,
                           max_tiles, tile0);
    return hipGetLastError();
}

hipError_t launch_sink_b4(const TokSrc &ksrc, const TokSrc &vsrc, int batch, int kv_heads, uint8_t *sink,
                          bool sparse, hipStream_t st) {
    const dim3 grid((unsigned)kv_heads, (unsigned)batch);
    if (sparse)
        hipLaunchKernelGGL(sink_b4_kernel<true>, grid, dim3(64), 0, st, ksrc, vsrc, kv_heads, sink);
    else
        hipLaunchKernelGGL(sink_b4_kernel<false>, grid, dim3(64), 0, st, ksrc, vsrc, kv_heads, sink);
    return hipGetLastError();
}

hipError_t launch_decode_b4(const DecodeB4Args &a, float *out, int splits, hipStream_t st) {
    const dim3 grid((unsigned)(a.batch * a.q_heads), (unsigned)splits);
    if (a.sparse) {
        if (a.rope)
            hipLaunchKernelGGL((decode_b4_pass1_kernel<true, true>), grid, dim3(64), 0, st, a);
        else
            hipLaunchKernelGGL((decode_b4_pass1_kernel<false, true>), grid, dim3(64), 0, st, a);
    } else {
        if (a.rope)
            hipLaunchKernelGGL((decode_b4_pass1_kernel<true, false>), grid, dim3(64), 0, st, a);
        else
            hipLaunchKernelGGL((decode_b4_pass1_kernel<false, false>), grid, dim3(64), 0, st, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_pass2(a.part_o, a.part_ml, out, a.batch * a.q_heads, splits, st);
}

}  // namespace kvq
