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

namespace kvq {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;
constexpr int REC = 3072;

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

// Keys: one workgroup of 64 lanes per tile; lane l owns channels 2l and 2l+1 over the tile's 32 tokens.
__global__ __launch_bounds__(64) void quant_keys_kernel(TokSrc src, int64_t t_begin, int kv_heads, uint8_t *tiles,
                                                        int64_t max_tiles, int64_t tile0) {
    __shared__ uint32_t words[256];
    const int l = threadIdx.x;
    const int64_t tile = blockIdx.x;
    const int h = blockIdx.y, b = blockIdx.z;
    for (int i = l; i < 256; i += 64) words[i] = 0u;

    float x0[32], x1[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const _Float16 *row = tok_row(src, b, h, t_begin + tile * 32 + i);
        h2 v = *reinterpret_cast<const h2 *>(row + 2 * l);
        x0[i] = (float)v[0];
        x1[i] = (float)v[1];
    }
    float mn0 = x0[0], mx0 = x0[0], mn1 = x1[0], mx1 = x1[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) {
        mn0 = fminf(mn0, x0[i]); mx0 = fmaxf(mx0, x0[i]);
        mn1 = fminf(mn1, x1[i]); mx1 = fmaxf(mx1, x1[i]);
    }
    _Float16 s0, z0, s1, z1;
    group_params(mn0, mx0, 3.0f, s0, z0);
    group_params(mn1, mx1, 3.0f, s1, z1);
    const float fs0 = (float)s0, fz0 = (float)z0, fs1 = (float)s1, fz1 = (float)z1;
    __syncthreads();

    // channel c = 2l: ks = c / 32, kc = (c % 32) / 8, e = c % 8 (even, so c + 1 sits in the next nibble)
    const int c = 2 * l, ks = c >> 5, kc = (c & 31) >> 3, e = c & 7;
    const int shift = 4 * e + 2 * (ks & 1);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const int m = i >> 4, n = i & 15;
        const int w = 4 * (n + 16 * kc) + 2 * m + (ks >> 1);
        uint32_t bits = (code_of(x0[i], fz0, fs0, 3.0f) << shift) | (code_of(x1[i], fz1, fs1, 3.0f) << (shift + 4));
        atomicOr(&words[w], bits);
    }
    __syncthreads();
    uint8_t *rec = tiles + ((int64_t)(b * kv_heads + h) * max_tiles + tile0 + tile) * REC;
    reinterpret_cast<uint4 *>(rec)[l] = reinterpret_cast<const uint4 *>(words)[l];
    h2 sp = {s0, s1}, zp = {z0, z1};
    reinterpret_cast<h2 *>(rec + 2048)[l] = sp;
    reinterpret_cast<h2 *>(rec + 2304)[l] = zp;
}

// Values: one workgroup of 64 lanes per tile; for each token, lane l owns channels 2l and 2l+1 and the 16 lanes
// of row g = l / 16 together own channel group g (channels 32g .. 32g+31).
__global__ __launch_bounds__(64) void quant_values_kernel(TokSrc src, int64_t t_begin, int kv_heads,
                                                          uint8_t *tiles, int64_t max_tiles, int64_t tile0) {
    __shared__ uint32_t words[256];
    __shared__ _Float16 sv[128], zv[128];
    const int l = threadIdx.x;
    const int64_t tile = blockIdx.x;
    const int h = blockIdx.y, b = blockIdx.z;
    for (int i = l; i < 256; i += 64) words[i] = 0u;
    __syncthreads();

    const int c = 2 * l, j = c >> 4, cc = c & 15, g = l >> 4;
#pragma unroll 4
    for (int i = 0; i < 32; ++i) {
        const _Float16 *row = tok_row(src, b, h, t_begin + tile * 32 + i);
        h2 v = *reinterpret_cast<const h2 *>(row + c);
        const float a0 = (float)v[0], a1 = (float)v[1];
        float mn = fminf(a0, a1), mx = fmaxf(a0, a1);
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            mn = fminf(mn, __shfl_xor(mn, off, 16));
            mx = fmaxf(mx, __shfl_xor(mx, off, 16));
        }
        _Float16 s, z;
        group_params(mn, mx, 3.0f, s, z);
        const float fs = (float)s, fz = (float)z;
        int kc, e;
        if (i < 16) { kc = i >> 2; e = i & 3; } else { kc = (i - 16) >> 2; e = 4 + ((i - 16) & 3); }
        const int w0 = 4 * (cc + 16 * kc) + (j >> 1);
        const int shift = 4 * e + 2 * (j & 1);
        atomicOr(&words[w0], code_of(a0, fz, fs, 3.0f) << shift);
        atomicOr(&words[w0 + 4], code_of(a1, fz, fs, 3.0f) << shift);
        if ((l & 15) == 0) { sv[32 * g + i] = s; zv[32 * g + i] = z; }
    }
    __syncthreads();
    uint8_t *rec = tiles + ((int64_t)(b * kv_heads + h) * max_tiles + tile0 + tile) * REC;
    reinterpret_cast<uint4 *>(rec + 1024)[l] = reinterpret_cast<const uint4 *>(words)[l];
    reinterpret_cast<uint32_t *>(rec + 2560)[l] = reinterpret_cast<const uint32_t *>(sv)[l];
    reinterpret_cast<uint32_t *>(rec + 2816)[l] = reinterpret_cast<const uint32_t *>(zv)[l];
}

// ------------------------------------------------------------------------------------------------ window append
// Copies n tokens (source tokens t_begin ..) of every slice into window rows dst0 .. ; 16 lanes move one 256-byte
// row, a workgroup of 64 lanes moves 4 rows.
__global__ __launch_bounds__(64) void copy_rows_kernel(TokSrc src, int64_t t_begin, int64_t n, int kv_heads,
                                                       _Float16 *res, int res_cap, int dst0) {
    const int l = threadIdx.x;
    const int64_t r = blockIdx.x * 4 + (l >> 4);
    const int h = blockIdx.y, b = blockIdx.z;
    if (r >= n) return;
    const _Float16 *row = tok_row(src, b, h, t_begin + r);
    _Float16 *dst = res + ((int64_t)(b * kv_heads + h) * res_cap + dst0 + r) * D;
    reinterpret_cast<uint4 *>(dst)[l & 15] = reinterpret_cast<const uint4 *>(row)[l & 15];
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

// Cross-row reductions over the four 16-lane rows of a wavefront with the gfx950 row swaps. Two compiler traps
// are avoided here: the second operand goes through an empty asm statement (a swap whose operands the compiler
// can prove equal is folded into the identity), and the result pair is copied into named integers before use
// (reading element 1 of the pair through a bit cast was lowered as element 0).
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}
__device__ __forceinline__ void swap16(uint32_t u, uint32_t &a, uint32_t &b) {
    auto p = __builtin_amdgcn_permlane16_swap(u, opaque(u), false, false);   // rows (0,1) and (2,3)
    a = p[0];
    b = p[1];
}
__device__ __forceinline__ void swap32(uint32_t u, uint32_t &a, uint32_t &b) {
    auto p = __builtin_amdgcn_permlane32_swap(u, opaque(u), false, false);   // halves (0,1) and (2,3)
    a = p[0];
    b = p[1];
}
__device__ __forceinline__ float rows_max(float v) {
    uint32_t a, b;
    swap16(__builtin_bit_cast(uint32_t, v), a, b);
    v = fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
    swap32(__builtin_bit_cast(uint32_t, v), a, b);
    return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float rows_sum(float v) {
    uint32_t a, b;
    swap16(__builtin_bit_cast(uint32_t, v), a, b);
    v = __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
    swap32(__builtin_bit_cast(uint32_t, v), a, b);
    return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// One wavefront per (split, batch row, KV head, chunk of up to 4 query heads of that KV head).
//
// Lane l = n + 16 kc (n = 0..15, kc = 0..3). Scores are computed transposed, S^T[t][n] = sum_c code[t][c] q~[c][n],
// with 16x16x32 fp16 MFMAs: the A operand is a 16-token block of key codes (exact small integers), the B operand
// holds the query with the tile's key scales folded in (q~ = q' * s_K, split into an fp16 high part and an fp16
// low part that are contracted one after the other), and a leading contraction with A = z_K (rows broadcast) and
// B = q' adds the zero-point term sum_c q' z_K. Column n carries query head n / 4 of the chunk, replicated over
// the four value channel groups g = n % 4, so that lane n's probabilities are exactly the PV A-operand row
// (head n / 4, group n % 4): P~[n][t] = p[t] * s_V[g][t] (fp16 high + low), contracted against the value codes of
// all 128 channels (8 N-blocks of 16); for channel block j only row group g = j / 2 is kept. The value zero-point
// term sum_t p[t] z_V[g][t] is accumulated on the VALU and added at the end.
//
// Per-wavefront LDS: the tile's 1 KB of scales/zeros and the 2 KB folded query (high and low parts, computed once
// per (head, channel) rather than once per replicated column). Both are written for tile v + 1 at the end of
// iteration v, after every read of tile v has been issued (a wavefront's LDS operations complete in order), so
// the next iteration starts with its operands in place. The fp16 window tiles reuse the same 8 KB.
constexpr int LDS_SZ = 0;            // 256 x uint32: s_K[128], z_K[128], s_V[4][32], z_V[4][32] (fp16)
constexpr int LDS_QT = 1024;         // fp16 [2 (high, low)][4 heads][128 channels]
constexpr int LDS_BYTES = 8192;      // also the fp16 window tile [32][128]

__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(4, 4))) void decode_pass1_kernel(DecodeArgs a) {
    __shared__ __align__(16) unsigned char smem[LDS_BYTES];
    uint32_t *sz_lds = reinterpret_cast<uint32_t *>(smem + LDS_SZ);
    const _Float16 *szh = reinterpret_cast<const _Float16 *>(smem + LDS_SZ);
    _Float16 *qt_lds = reinterpret_cast<_Float16 *>(smem + LDS_QT);
    _Float16 *vres_lds = reinterpret_cast<_Float16 *>(smem);

    const int l = threadIdx.x;
    const int n = l & 15, kc = l >> 4, hl = n >> 2, g = n & 3;
    const int unit = blockIdx.x;
    const int split = blockIdx.y;
    const int chunk = unit % a.chunks;
    const int hkv = (unit / a.chunks) % a.kv_heads;
    const int b = unit / (a.chunks * a.kv_heads);
    const int G = a.q_heads / a.kv_heads;
    const int gc = min(4, G - 4 * chunk);
    const int h0 = hkv * G + 4 * chunk;
    const bool col_valid = hl < gc;

    // ---- query, two layouts. MFMA B layout (column n, channels 32 ks + 8 kc + e): used for the zero-point term and
    // the window tiles. Folding layout (head kc, channels 8 n .. 8 n + 7): one (head, channel) per lane slot.
    const _Float16 *qp = a.q + ((int64_t)b * a.q_heads + h0 + (col_valid ? hl : 0)) * D;
    h8 qv[4];
    float qmax = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        qv[ks] = *reinterpret_cast<const h8 *>(qp + 32 * ks + 8 * kc);
#pragma unroll
        for (int e = 0; e < 8; ++e) qmax = fmaxf(qmax, fabsf((float)qv[ks][e]));
    }
    qmax = rows_max(qmax);
    // q' = q * 2^-E with 2^E > max |q|: |q'| < 1 keeps q' * s_K within binary16 range for any fp16 scale
    int E = 0;   // qmax is a float16 value widened, hence a normal binary32 number: read its exponent field
    if (qmax > 0.0f) E = (int)((__builtin_bit_cast(uint32_t, qmax) >> 23) & 0xffu) - 127 + 1;
    const float qsc = pow2(-E);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[ks][e] = col_valid ? (_Float16)((float)qv[ks][e] * qsc) : (_Float16)0.0f;
    // folding layout: lane (n, kc) holds head kc of the chunk (if valid), channels 8n .. 8n+7; its own scale 2^-E_kc
    h8 qf = {};
    {
        const bool fv = kc < gc;
        const _Float16 *qfp = a.q + ((int64_t)b * a.q_heads + h0 + (fv ? kc : 0)) * D + 8 * n;
        const h8 raw = *reinterpret_cast<const h8 *>(qfp);
        // after rows_max, lane 4 kc (column 4 kc, head kc) holds the maximum of head kc
        const float qm_head = __shfl(qmax, 4 * kc);
        int Eh = 0;
        if (qm_head > 0.0f) Eh = (int)((__builtin_bit_cast(uint32_t, qm_head) >> 23) & 0xffu) - 127 + 1;
        const float sch = pow2(-Eh);
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[e] = fv ? (_Float16)((float)raw[e] * sch) : (_Float16)0.0f;
    }
    const float C = a.sm_log2 * pow2(E);   // score (in q' units) -> log2 domain

    float m = -__builtin_inff();
    float lsum = 0.0f, gam = 0.0f;
    f4 o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = f4{0.0f, 0.0f, 0.0f, 0.0f};

    const int n_vt = a.n_qtiles + (a.n_resid + 31) / 32;
    const int v0 = split * a.tiles_per_split;
    const int v1 = min(v0 + a.tiles_per_split, n_vt);
    const int qend = min(v1, a.n_qtiles);
    const uint8_t *base = a.tiles + ((int64_t)b * a.kv_heads + hkv) * a.max_tiles * (int64_t)REC;

    // stage a tile's scales/zeros and its folded query (high, low) into LDS
    auto stage = [&](const uint4 &sw) {
        reinterpret_cast<uint4 *>(sz_lds)[l] = sw;
        __syncthreads();
        const h8 sk = *reinterpret_cast<const h8 *>(szh + 8 * n);
        const h8 hi = qf * sk;
        const h8 lo = __builtin_elementwise_fma(qf, sk, -hi);
        *reinterpret_cast<h8 *>(qt_lds + 128 * kc + 8 * n) = hi;
        *reinterpret_cast<h8 *>(qt_lds + 512 + 128 * kc + 8 * n) = lo;
        __syncthreads();
    };

    // ------------------------------------------------------------------ quantized tiles
    uint4 kw, vw, sw;
    if (v0 < qend) {
        const uint8_t *rec = base + (int64_t)v0 * REC;
        kw = reinterpret_cast<const uint4 *>(rec)[l];
        vw = reinterpret_cast<const uint4 *>(rec + 1024)[l];
        sw = reinterpret_cast<const uint4 *>(rec + 2048)[l];
        stage(sw);
    }
    for (int v = v0; v < qend; ++v) {
        const uint32_t kwa[4] = {kw.x, kw.y, kw.z, kw.w};
        const uint32_t vwa[4] = {vw.x, vw.y, vw.z, vw.w};
        const bool more = v + 1 < qend;
        if (more) {    // prefetch the next tile
            const uint8_t *rec = base + (int64_t)(v + 1) * REC;
            kw = reinterpret_cast<const uint4 *>(rec)[l];
            vw = reinterpret_cast<const uint4 *>(rec + 1024)[l];
            sw = reinterpret_cast<const uint4 *>(rec + 2048)[l];
        }

        // zero-point term: acc0[t][n] = sum_c z_K[c] q'[c][n] (the same for every token row)
        f4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const h8 zk = *reinterpret_cast<const h8 *>(szh + 128 + 32 * ks + 8 * kc);
            acc0 = mfma(zk, qv[ks], acc0);
        }
        f4 acc1 = acc0;
        const _Float16 *qth = qt_lds + 128 * hl + 8 * kc;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const h8 hi = *reinterpret_cast<const h8 *>(qth + 32 * ks);
            const h8 lo = *reinterpret_cast<const h8 *>(qth + 512 + 32 * ks);
            const h8 a0 = expand8(nibbles(kwa[ks >> 1], ks & 1));
            const h8 a1 = expand8(nibbles(kwa[2 + (ks >> 1)], ks & 1));
            acc0 = mfma(a0, hi, acc0);
            acc1 = mfma(a1, hi, acc1);
            acc0 = mfma(a0, lo, acc0);
            acc1 = mfma(a1, lo, acc1);
        }
        // acc0[r]: token 4 kc + r; acc1[r]: token 16 + 4 kc + r; column n. C > 0, so the maximum is taken on the
        // raw accumulators and scaled once.
        float mx = fmaxf(fmaxf(fmaxf(acc0[0], acc0[1]), fmaxf(acc0[2], acc0[3])),
                         fmaxf(fmaxf(acc1[0], acc1[1]), fmaxf(acc1[2], acc1[3])));
        mx = rows_max(mx) * C;
        const float mnew = fmaxf(m, mx);
        if (__any(mnew > m)) {
            const float alpha = __builtin_amdgcn_exp2f(m - mnew);
            lsum *= alpha;
            gam *= alpha;
            float ar[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * kc + r);
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) o[j][r] *= ar[r];
            m = mnew;
        }
        float p[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc0[r], C, -m));
            p[4 + r] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc1[r], C, -m));
        }
        lsum += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));

        // value scales/zeros of tokens 4kc..4kc+3 and 16+4kc..16+4kc+3, channel group g
        const h4 sv0 = *reinterpret_cast<const h4 *>(szh + 256 + 32 * g + 4 * kc);
        const h4 sv1 = *reinterpret_cast<const h4 *>(szh + 256 + 32 * g + 16 + 4 * kc);
        const h4 zv0 = *reinterpret_cast<const h4 *>(szh + 384 + 32 * g + 4 * kc);
        const h4 zv1 = *reinterpret_cast<const h4 *>(szh + 384 + 32 * g + 16 + 4 * kc);
        h8 phi, plo;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float t0 = p[i] * (float)sv0[i];
            const float t1 = p[4 + i] * (float)sv1[i];
            phi[i] = (_Float16)t0;
            phi[4 + i] = (_Float16)t1;
            plo[i] = (_Float16)(t0 - (float)phi[i]);
            plo[4 + i] = (_Float16)(t1 - (float)phi[4 + i]);
            gam = __builtin_fmaf(p[i], (float)zv0[i], gam);
            gam = __builtin_fmaf(p[4 + i], (float)zv1[i], gam);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const h8 bv = expand8(nibbles(vwa[j >> 1], j & 1));
            o[j] = mfma(phi, bv, o[j]);
            o[j] = mfma(plo, bv, o[j]);
        }
        if (more) stage(sw);   // every LDS read of this tile has been issued: overwrite with the next tile
    }

    // ------------------------------------------------------------------ residual (fp16) tiles
    const _Float16 *kres = a.k_res + ((int64_t)b * a.kv_heads + hkv) * a.res_cap * D;
    const _Float16 *vres = a.v_res + ((int64_t)b * a.kv_heads + hkv) * a.res_cap * D;
    for (int v = max(v0, a.n_qtiles); v < v1; ++v) {
        const int r0 = (v - a.n_qtiles) * 32;
        const int nv = min(32, a.n_resid - r0);
        __syncthreads();
        // stage the value rows (zeros beyond the valid ones) for the transposed PV operand
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int idx = l + 64 * i;        // 16-byte chunk: token idx / 16, channels 8 (idx % 16) ..
            const int tok = idx >> 4;
            uint4 val = {0u, 0u, 0u, 0u};
            if (tok < nv) val = reinterpret_cast<const uint4 *>(vres + (int64_t)(r0 + tok) * D)[idx & 15];
            reinterpret_cast<uint4 *>(vres_lds)[idx] = val;
        }
        f4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = acc0;
        const int t0 = min(n, nv - 1), t1 = min(16 + n, nv - 1);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const h8 k0 = *reinterpret_cast<const h8 *>(kres + (int64_t)(r0 + t0) * D + 32 * ks + 8 * kc);
            const h8 k1 = *reinterpret_cast<const h8 *>(kres + (int64_t)(r0 + t1) * D + 32 * ks + 8 * kc);
            acc0 = mfma(k0, qv[ks], acc0);
            acc1 = mfma(k1, qv[ks], acc1);
        }
        float x[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            x[r] = (4 * kc + r < nv) ? acc0[r] * C : -__builtin_inff();
            x[4 + r] = (16 + 4 * kc + r < nv) ? acc1[r] * C : -__builtin_inff();
        }
        float mx = x[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
        mx = rows_max(mx);
        const float mnew = fmaxf(m, mx);
        if (__any(mnew > m)) {
            const float alpha = __builtin_amdgcn_exp2f(m - mnew);
            lsum *= alpha;
            gam *= alpha;
            float ar[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * kc + r);
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) o[j][r] *= ar[r];
            m = mnew;
        }
        h8 phi, plo;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float p = __builtin_amdgcn_exp2f(x[i] - m);
            lsum += p;
            phi[i] = (_Float16)p;
            plo[i] = (_Float16)(p - (float)phi[i]);
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            h8 bv;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int tok = (e < 4) ? (4 * kc + e) : (16 + 4 * kc + e - 4);
                bv[e] = vres_lds[tok * 128 + n + 16 * j];
            }
            o[j] = mfma(phi, bv, o[j]);
            o[j] = mfma(plo, bv, o[j]);
        }
    }

    // ------------------------------------------------------------------ partials of this split
    lsum = rows_sum(lsum);
    gam = rows_sum(gam);
    float gr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) gr[r] = __shfl(gam, 4 * kc + r);
    const int64_t S = gridDim.y;
    if (kc < gc) {   // lane (n, kc) holds head h0 + kc, channels n + 16 j
        const int hq = h0 + kc;
        float *po = a.part_o + (((int64_t)b * a.q_heads + hq) * S + split) * D;
#pragma unroll
        for (int j = 0; j < 8; ++j) po[n + 16 * j] = o[j][j >> 1] + gr[j >> 1];
    }
    if (kc == 0 && g == 0 && col_valid) {
        const int hq = h0 + hl;
        float *pm = a.part_ml + (((int64_t)b * a.q_heads + hq) * S + split) * 2;
        pm[0] = m;
        pm[1] = lsum;
    }
}

// ------------------------------------------------------------------------------------------------ decode pass 2
// One wavefront per (batch row, query head): out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
__global__ __launch_bounds__(64) void decode_pass2_kernel(const float *part_o, const float *part_ml, float *out,
                                                          int splits) {
    const int64_t bh = blockIdx.x;
    const int l = threadIdx.x;
    const float *pm = part_ml + bh * splits * 2;
    float M = -__builtin_inff();
    for (int s = 0; s < splits; ++s) M = fmaxf(M, pm[2 * s]);
    float L = 0.0f, o0 = 0.0f, o1 = 0.0f;
    for (int s = 0; s < splits; ++s) {
        const float ms = pm[2 * s];
        const float w = (ms == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(ms - M);
        L += w * pm[2 * s + 1];
        const float2 ov = reinterpret_cast<const float2 *>(part_o + (bh * splits + s) * D)[l];
        o0 += w * ov.x;
        o1 += w * ov.y;
    }
    reinterpret_cast<float2 *>(out + bh * D)[l] = float2{o0 / L, o1 / L};
}

// ------------------------------------------------------------------------------------------------ launchers
hipError_t launch_quant_keys(const TokSrc &src, int64_t t_begin, int64_t n_tiles, int batch, int kv_heads,
                             uint8_t *tiles, int64_t max_tiles, int64_t tile0, hipStream_t st) {
    dim3 grid((unsigned)n_tiles, (unsigned)kv_heads, (unsigned)batch);
    hipLaunchKernelGGL(quant_keys_kernel, grid, dim3(64), 0, st, src, t_begin, kv_heads, tiles, max_tiles, tile0);
    return hipGetLastError();
}

hipError_t launch_quant_values(const TokSrc &src, int64_t t_begin, int64_t n_tiles, int batch, int kv_heads,
                               uint8_t *tiles, int64_t max_tiles, int64_t tile0, hipStream_t st) {
    dim3 grid((unsigned)n_tiles, (unsigned)kv_heads, (unsigned)batch);
    hipLaunchKernelGGL(quant_values_kernel, grid, dim3(64), 0, st, src, t_begin, kv_heads, tiles, max_tiles, tile0);
    return hipGetLastError();
}

hipError_t launch_copy_rows(const TokSrc &src, int64_t t_begin, int64_t n, int batch, int kv_heads, _Float16 *res,
                            int res_cap, int dst0, hipStream_t st) {
    dim3 grid((unsigned)((n + 3) / 4), (unsigned)kv_heads, (unsigned)batch);
    hipLaunchKernelGGL(copy_rows_kernel, grid, dim3(64), 0, st, src, t_begin, n, kv_heads, res, res_cap, dst0);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs &a, int splits, hipStream_t st) {
    const int units = a.batch * a.kv_heads * a.chunks;
    hipLaunchKernelGGL(decode_pass1_kernel, dim3((unsigned)units, (unsigned)splits), dim3(64), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_pass2_kernel, dim3((unsigned)(a.batch * a.q_heads)), dim3(64), 0, st, a.part_o,
                       a.part_ml, a.out, splits);
    return hipGetLastError();
}

}  // namespace kvq
