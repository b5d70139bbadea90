// Internal interface between the C-ABI entry points (kvq_api.hip) and the HIP kernels (kvq_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

// Tokens 0 .. n_a - 1 come from `a`, tokens n_a .. from `b` (element strides; the channel stride is 1). Lets one
// kernel read a flush block that starts in the residual window and continues in the new tokens.
struct TokSrc {
    const _Float16 *a;
    int64_t a_sb, a_sh, a_st;
    int64_t n_a;
    const _Float16 *b;
    int64_t b_sb, b_sh, b_st;
};

struct DecodeArgs {
    const uint8_t *tiles;
    const _Float16 *k_res;
    const _Float16 *v_res;
    const _Float16 *q;
    float *part_o;   // [B][Hq][splits][128]
    float *part_ml;  // [B][Hq][splits][2]: maximum (log2 domain) and exponent sum
    float *out;      // [B][Hq][128]
    int64_t max_tiles;
    int n_qtiles;
    int n_resid;
    int res_cap;
    int batch;
    int kv_heads;
    int q_heads;
    int chunks;           // ceil(G / 4): query heads are processed four per wavefront
    int tiles_per_split;  // 32-token tiles (quantized, then residual) per split
    float sm_log2;        // softmax scale * log2(e)
    int sparse;           // dense-and-sparse records (3840 bytes; uniform lengths only)
    const int32_t *lens;  // ragged caches: per-sequence {n_quant, n_resid, n_sink, status}; else null
    int appended;         // ragged: the lengths predate the append of one token per sequence (decode step)
    // single-launch decode step (ragged caches): the new token of every (batch row, KV head) at
    // k_new/v_new + b new_sb + h new_sh; the launch flushes full windows, attends, merges the splits, writes the
    // new rows and commits the lengths, counting finished workgroups in `sync` (zero before and after)
    const _Float16 *k_new;
    const _Float16 *v_new;
    int64_t new_sb, new_sh;
    uint8_t *tiles_w;
    _Float16 *k_res_w;
    _Float16 *v_res_w;
    int32_t *lens_w;
    uint32_t *sync;
};

// 4-bit (KVQuant-style) decode: one wavefront per (batch row, query head, token split). Virtual tiles v of a
// slice: [0, n_sink) the sink token (position 0), then n_qtiles quantized tiles, then the window tiles.
struct DecodeB4Args {
    const uint8_t *tiles;   // [B][Hkv][max_tiles][5120, or 5888 with outliers]
    const uint8_t *sink;    // [B][Hkv][512] (read only when n_sink = 1)
    const _Float16 *k_res;
    const _Float16 *v_res;
    const _Float16 *q;
    float *part_o;          // [B][Hq][splits][128]
    float *part_ml;         // [B][Hq][splits][2]
    int64_t max_tiles;
    int n_sink;
    int n_qtiles;
    int n_resid;
    int res_cap;
    int batch;
    int kv_heads;
    int q_heads;
    int tiles_per_split;
    float sm_log2;
    int rope;               // keys are cached before RoPE: rotate by the absolute position
    int sparse;             // dense-and-sparse records (5888 bytes) and sink
    double log2_base;       // log2 of the RoPE base
};

hipError_t launch_quant_keys_b4(const TokSrc &src, int64_t t_begin, int64_t n_tiles, int batch, int kv_heads,
                                uint8_t *tiles, int64_t max_tiles, int64_t tile0, bool sparse, hipStream_t st);
hipError_t launch_quant_values_b4(const TokSrc &src, int64_t t_begin, int64_t n_tiles, int batch, int kv_heads,
                                  uint8_t *tiles, int64_t max_tiles, int64_t tile0, bool sparse, hipStream_t st);
hipError_t launch_sink_b4(const TokSrc &ksrc, const TokSrc &vsrc, int batch, int kv_heads, uint8_t *sink,
                          bool sparse, hipStream_t st);
hipError_t launch_decode_b4(const DecodeB4Args &a, float *out, int splits, hipStream_t st);
hipError_t launch_pass2(const float *part_o, const float *part_ml, float *out, int rows, int splits, hipStream_t st);

// 2-bit tiles (sparse: dense-and-sparse records of 3840 bytes)
hipError_t launch_quant_keys(const TokSrc &src, int64_t t_begin, int64_t n_tiles, int batch, int kv_heads,
                             uint8_t *tiles, int64_t max_tiles, int64_t tile0, bool sparse, hipStream_t st);
hipError_t launch_quant_values(const TokSrc &src, int64_t t_begin, int64_t n_tiles, int batch, int kv_heads,
                               uint8_t *tiles, int64_t max_tiles, int64_t tile0, bool sparse, hipStream_t st);
hipError_t launch_copy_rows(const TokSrc &ksrc, const TokSrc &vsrc, int64_t t_begin, int64_t n, int batch,
                            int kv_heads, _Float16 *kres, _Float16 *vres, int res_cap, int dst0, hipStream_t st);
hipError_t launch_decode(const DecodeArgs &a, int splits, hipStream_t st);

// Ragged caches (per-sequence lengths in device memory, see kvq_kernels.hip).
hipError_t launch_ragged_flush_append(const TokSrc &knew, const TokSrc &vnew, int batch, int kv_heads,
                                      uint8_t *tiles, int64_t max_tiles, _Float16 *k_res, _Float16 *v_res,
                                      int res_cap, int32_t *lens, hipStream_t st);
hipError_t launch_ragged_commit(int32_t *lens, int batch, int res_cap, hipStream_t st);
hipError_t launch_ragged_set(int32_t *lens, int b, int nq, int nr, int ns, hipStream_t st);
// pass 1 over per-sequence lengths, then pass 2 (which commits the appended token's lengths when `commit`)
hipError_t launch_decode_ragged(const DecodeArgs &a, int splits, int32_t *lens, int commit, hipStream_t st);
// the whole decode step (append with lazy flush, attention, merge, length commit) in one launch
hipError_t launch_decode_step(const DecodeArgs &a, int splits, hipStream_t st);

}  // namespace kvq
