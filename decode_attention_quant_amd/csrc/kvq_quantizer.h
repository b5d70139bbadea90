// Device helpers shared by the 2-bit and 4-bit kernels: token-row addressing of a two-source token range and the
// asymmetric min/max group quantizer (KIVI page, paragraph on the cache contents; the exact rounding rule is the one
// stated in include/kvq.h for kv_quant_keys_per_channel, with L = 2^bits - 1).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_kernels.h"

namespace kvq {

typedef _Float16 h2v __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------------------------------------ token sources
__device__ __forceinline__ const _Float16 *tok_row(const TokSrc &s, int b, int h, int64_t t) {
    if (t < s.n_a) return s.a + b * s.a_sb + h * s.a_sh + t * s.a_st;
    t -= s.n_a;
    return s.b + b * s.b_sb + h * s.b_sh + t * s.b_st;
}

// ------------------------------------------------------------------------------------------------ group quantizer
// Asymmetric min/max quantizer with binary16 scale/zero (see kvq.h for the exact rule). Contraction is switched
// off so every binary32 operation rounds on its own.
__device__ __forceinline__ void group_params(float mn, float mx, float levels, _Float16 &s_out, _Float16 &z_out) {
#pragma clang fp contract(off)
    float r = mx - mn;
    float s32 = r / levels;
    _Float16 s = (_Float16)s32;
    if ((levels + 0.5f) * (float)s < r) {
        uint16_t bits = __builtin_bit_cast(uint16_t, s);
        s = __builtin_bit_cast(_Float16, (uint16_t)(bits + 1));
    }
    _Float16 z = (_Float16)mn;
    if (mn == 0.0f) z = (_Float16)0.0f;
    s_out = s;
    z_out = z;
}

// Channels c, c + 1 of the tokens t0 .. t0 + 31 of slice (b, h): x0[i], x1[i]. A tile normally lies in one source
// (one pointer walk); a tile that straddles the two sources selects per row.
__device__ __forceinline__ void load_pairs32(const TokSrc &s, int64_t t0, int b, int h, int c, float (&x0)[32],
                                             float (&x1)[32]) {
    const int64_t lim = s.n_a - t0;   // rows i < lim come from source a
    if (lim >= 32 || lim <= 0) {
        const bool in_a = lim >= 32;
        const _Float16 *p = in_a ? s.a + b * s.a_sb + h * s.a_sh + t0 * s.a_st + c
                                 : s.b + b * s.b_sb + h * s.b_sh + (t0 - s.n_a) * s.b_st + c;
        const int64_t st = in_a ? s.a_st : s.b_st;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const h2v v = *reinterpret_cast<const h2v *>(p);
            x0[i] = (float)v[0];
            x1[i] = (float)v[1];
            p += st;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const h2v v = *reinterpret_cast<const h2v *>(tok_row(s, b, h, t0 + i) + c);
            x0[i] = (float)v[0];
            x1[i] = (float)v[1];
        }
    }
}

// The level of one element, equal to code_of (the stated rule) for s > 0, with the division replaced by a product
// with rs ~ 1/s (within 1 ulp): t' = RN32(d * rs) is within 4 * 2^-24 * t' of the correctly rounded quotient t, at
// most 2^-18 for t <= 16, so rint(t') = rint(t) unless t' lies within 2^-16 of a half-integer, where the correctly
// rounded division decides.
// The division sits behind a wavefront vote, so it is a scalar branch taken only when some lane needs it (a lane-level
// condition lets the compiler compute the division for every element and select).
__device__ __forceinline__ uint32_t code_fast(float x, float z, float s, float rs, float levels) {
#pragma clang fp contract(off)
    const float d = x - z;
    float t = d * rs;
    const float f = t - __builtin_floorf(t);
    const bool near = __builtin_fabsf(f - 0.5f) < 0x1p-16f;
    if (__builtin_amdgcn_ballot_w64(near) != 0) {
        const float te = d / s;
        t = near ? te : t;
    }
    float q = __builtin_rintf(t);
    q = fminf(fmaxf(q, 0.0f), levels);
    return (uint32_t)q;
}

// The same tile load with each token's channel pair kept as one packed binary16 word (channel c in the low half).
__device__ __forceinline__ void load_pairs32_packed(const TokSrc &s, int64_t t0, int b, int h, int c,
                                                    uint32_t (&xw)[32]) {
    const int64_t lim = s.n_a - t0;   // rows i < lim come from source a
    if (lim >= 32 || lim <= 0) {
        const bool in_a = lim >= 32;
        const _Float16 *p = in_a ? s.a + b * s.a_sb + h * s.a_sh + t0 * s.a_st + c
                                 : s.b + b * s.b_sb + h * s.b_sh + (t0 - s.n_a) * s.b_st + c;
        const int64_t st = in_a ? s.a_st : s.b_st;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            xw[i] = *reinterpret_cast<const uint32_t *>(p);
            p += st;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) xw[i] = *reinterpret_cast<const uint32_t *>(tok_row(s, b, h, t0 + i) + c);
    }
}

// Element-wise minimum and maximum of 32 packed binary16 pairs (exact: the results are elements).
__device__ __forceinline__ void minmax_pairs32(const uint32_t (&xw)[32], h2v &mn, h2v &mx) {
    mn = __builtin_bit_cast(h2v, xw[0]);
    mx = mn;
#pragma unroll
    for (int i = 1; i < 32; ++i) {
        const h2v v = __builtin_bit_cast(h2v, xw[i]);
        mn = __builtin_elementwise_min(mn, v);
        mx = __builtin_elementwise_max(mx, v);
    }
}

// RN32(x - z) for the binary16 x in the low (HI = false) or high half of w: one mixed-precision fma x * 1 - z,
// exact product and a single rounding.
template <bool HI>
__device__ __forceinline__ float diff_half(uint32_t w, float z) {
    float d;
    if constexpr (HI)
        asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(w), "v"(z));
    else
        asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel_hi:[1,0,0]" : "=v"(d) : "v"(w), "v"(z));
    return d;
}

// code_fast from d = RN32(x - z): the same level, the same near-half test (t within 2^-16 of a half-integer, judged
// from t - rint(t)) and the same correctly rounded division there, with rint shared by the test and the level.
__device__ __forceinline__ uint32_t code_from_diff(float d, float s, float rs, uint32_t levels) {
#pragma clang fp contract(off)
    float t = d * rs;
    float r = __builtin_rintf(t);
    const bool near = __builtin_fabsf(t - r) > 0.5f - 0x1p-16f;
    if (__builtin_amdgcn_ballot_w64(near) != 0) {
        const float te = d / s;
        t = near ? te : t;
        r = __builtin_rintf(t);
    }
    const uint32_t q = (uint32_t)r;   // r >= 0 (d >= 0, rs >= 0)
    return q < levels ? q : levels;
}

__device__ __forceinline__ uint32_t code_of(float x, float z, float s, float levels) {
#pragma clang fp contract(off)
    if (s == 0.0f) return 0u;
    float d = x - z;
    float t = d / s;
    float q = __builtin_rintf(t);
    q = fminf(fmaxf(q, 0.0f), levels);
    return (uint32_t)q;
}

}  // namespace kvq
