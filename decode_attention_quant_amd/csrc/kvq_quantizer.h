// Device helpers shared by the 2-bit and 4-bit kernels: token-row addressing of a two-source token range and the
// asymmetric min/max group quantizer (KIVI page, paragraph on the cache contents; the exact rounding rule is the one
// stated in include/kvq.h for kv_quant_keys_per_channel, with L = 2^bits - 1).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_kernels.h"

namespace kvq {

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
