// C-ABI entry points declared in include/kvq.h: host-side validation, the residual-window state machine and the
// split-K sizing; every step of the computation runs in the kernels of kvq_kernels.hip (2-bit) and
// kvq_kernels_b4.hip (4-bit).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "kvq.h"
#include "kvq_kernels.h"

// Scratch of the allocation-free decode entry point (kv_decode_attention_noalloc): the split partials of one call
// in a file-scope device array of KVQ_NOALLOC_SCRATCH_BYTES, one copy per GPU, held until the process ends. In
// host code the array's name is not a device address; each device's address comes from hipGetSymbolAddress on that
// device's first call and is the only form host code passes on.
__device__ __align__(256) unsigned char scratch[KVQ_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Address of the current device's scratch array (looked up once per device, with that device current).
int scratch_address(void **ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KVQ_E_LAUNCH;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVQ_E_LAUNCH;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return KVQ_OK;
}

// Split plans fill the chip in a single round, with no tail of partly filled rounds. The 2-bit decode kernel could
// hold four wavefronts per SIMD (its register budget, 4096 in all) but runs faster with three (3072: fewer
// concurrent read streams; the call's settled rate and the decode step both gain ~2% over four). The 4-bit kernel
// keeps its rotation tables in registers and holds two per SIMD.
constexpr int64_t kTargetWaves = 3072;
constexpr int64_t kTargetWavesB4 = 2048;
constexpr int64_t kTargetWavesSparse = 3072;   // 2-bit dense-and-sparse: three wavefronts per SIMD (LDS and registers)
constexpr int64_t kMinTilesPerSplit = 4;
constexpr int64_t kMaxSplits = 1024;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// decided on the bit pattern, so that it holds whatever floating-point assumptions the compiler is given
bool finite_above_one(double x) {
    uint64_t u;
    memcpy(&u, &x, sizeof u);
    if (((u >> 52) & 0x7ff) == 0x7ff) return false;   // infinity or NaN
    return x > 1.0;
}

int check_shape(const kvq_shape *s) {
    if (!s) return KVQ_E_NULL;
    if (s->bits != 2 && s->bits != 4) return KVQ_E_BITS;
    if (s->batch <= 0 || s->kv_heads <= 0 || s->q_heads <= 0 || s->head_dim != KVQ_HEAD_DIM ||
        s->group != KVQ_GROUP || s->q_heads % s->kv_heads != 0 || s->residual_cap <= 0 ||
        s->residual_cap % KVQ_TILE_TOKENS != 0 || s->max_tokens <= 0 || s->max_tokens % KVQ_TILE_TOKENS != 0 ||
        s->batch > 65535 || s->kv_heads > 65535 || (int64_t)s->batch * s->q_heads > 0x7fffffff)
        return KVQ_E_SHAPE;
    if ((s->flags & ~(KVQ_FLAG_SINK | KVQ_FLAG_PRE_ROPE | KVQ_FLAG_SPARSE)) != 0 ||
        (s->bits == 2 && s->flags != 0 && s->flags != KVQ_FLAG_SPARSE))   // 2-bit: dense-and-sparse groups only
        return KVQ_E_SHAPE;
    if ((s->flags & KVQ_FLAG_PRE_ROPE) && !finite_above_one(s->rope_base)) return KVQ_E_SHAPE;
    return KVQ_OK;
}

bool has_sink(const kvq_shape *s) { return (s->flags & KVQ_FLAG_SINK) != 0; }
bool is_sparse(const kvq_shape *s) { return (s->flags & KVQ_FLAG_SPARSE) != 0; }

int check_cache(const kvq_shape *s, const kvq_cache *c) {
    if (!c) return KVQ_E_NULL;
    if (!c->tiles || !c->k_res || !c->v_res) return KVQ_E_NULL;
    if (has_sink(s) && !c->sink) return KVQ_E_NULL;
    if (!aligned16(c->tiles) || !aligned16(c->k_res) || !aligned16(c->v_res)) return KVQ_E_ALIGN;
    if (has_sink(s) && !aligned16(c->sink)) return KVQ_E_ALIGN;
    if (c->n_quant < 0 || c->n_quant % KVQ_TILE_TOKENS != 0 || c->n_quant > s->max_tokens || c->n_resid < 0 ||
        c->n_resid > s->residual_cap)
        return KVQ_E_STATE;
    if (c->n_sink != 0 && c->n_sink != 1) return KVQ_E_STATE;
    if (!has_sink(s) && c->n_sink != 0) return KVQ_E_STATE;
    // with a sink, token 0 always goes to the sink first
    if (has_sink(s) && c->n_sink == 0 && (c->n_quant != 0 || c->n_resid != 0)) return KVQ_E_STATE;
    return KVQ_OK;
}

int check_src(const void *p, int64_t sb, int64_t sh, int64_t st) {
    if (!p) return KVQ_E_NULL;
    if (!aligned16(p) || sb % 8 != 0 || sh % 8 != 0 || st % 8 != 0) return KVQ_E_ALIGN;
    if (sb < 0 || sh < 0 || st < 0) return KVQ_E_ALIGN;
    return KVQ_OK;
}

int launched(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_E_LAUNCH; }

kvq::TokSrc single_src(const void *p, int64_t sb, int64_t sh, int64_t st) {
    kvq::TokSrc s;
    s.a = static_cast<const _Float16 *>(p);
    s.a_sb = sb; s.a_sh = sh; s.a_st = st;
    s.n_a = INT64_MAX;
    s.b = s.a; s.b_sb = sb; s.b_sh = sh; s.b_st = st;
    return s;
}

hipError_t quant_launch(const kvq_shape *shape, bool keys, const kvq::TokSrc &src, int64_t nt, uint8_t *tiles,
                        int64_t max_tiles, int64_t tile0, hipStream_t st) {
    const int B = shape->batch, H = shape->kv_heads;
    if (shape->bits == 4)
        return keys ? kvq::launch_quant_keys_b4(src, 0, nt, B, H, tiles, max_tiles, tile0, is_sparse(shape), st)
                    : kvq::launch_quant_values_b4(src, 0, nt, B, H, tiles, max_tiles, tile0, is_sparse(shape), st);
    return keys ? kvq::launch_quant_keys(src, 0, nt, B, H, tiles, max_tiles, tile0, is_sparse(shape), st)
                : kvq::launch_quant_values(src, 0, nt, B, H, tiles, max_tiles, tile0, is_sparse(shape), st);
}

int quant_common(const kvq_shape *shape, const void *x, int64_t sb, int64_t sh, int64_t st, int64_t n_tokens,
                 int64_t tile0, void *tiles, bool keys, void *stream) {
    int e = check_shape(shape);
    if (e) return e;
    if (!tiles) return KVQ_E_NULL;
    if ((e = check_src(x, sb, sh, st))) return e;
    if (!aligned16(tiles)) return KVQ_E_ALIGN;
    if (n_tokens <= 0 || n_tokens % KVQ_TILE_TOKENS != 0 || tile0 < 0) return KVQ_E_SHAPE;
    const int64_t max_tiles = shape->max_tokens / KVQ_TILE_TOKENS;
    if (tile0 + n_tokens / KVQ_TILE_TOKENS > max_tiles) return KVQ_E_CAPACITY;
    const kvq::TokSrc src = single_src(x, sb, sh, st);
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t *t = static_cast<uint8_t *>(tiles);
    const int64_t nt = n_tokens / KVQ_TILE_TOKENS;
    return launched(quant_launch(shape, keys, src, nt, t, max_tiles, tile0, s));
}

struct SplitPlan {
    int64_t n_vt;       // 32-token tiles to visit (quantized + residual)
    int32_t splits;
    int32_t tiles_per_split;
    int32_t chunks;
};

// Splits along the virtual tiles (quantized, then window). A work unit is one wavefront's (batch row, KV head,
// chunk of 4 query heads) in the 2-bit kernel and one (batch row, query head) in the 4-bit kernel; the sink token,
// when present, is taken by split 0 on top of its tiles.
SplitPlan plan(const kvq_shape *s, const kvq_cache *c) {
    SplitPlan p;
    p.n_vt = c->n_quant / KVQ_TILE_TOKENS + (c->n_resid + KVQ_TILE_TOKENS - 1) / KVQ_TILE_TOKENS;
    const int G = s->q_heads / s->kv_heads;
    p.chunks = (G + 3) / 4;
    const int64_t units = s->bits == 4 ? (int64_t)s->batch * s->q_heads : (int64_t)s->batch * s->kv_heads * p.chunks;
    const int64_t target = s->bits == 4 ? kTargetWavesB4 : (is_sparse(s) ? kTargetWavesSparse : kTargetWaves);
    int64_t S = (target + units - 1) / units;
    const int64_t by_len = (p.n_vt + kMinTilesPerSplit - 1) / kMinTilesPerSplit;
    if (S > by_len) S = by_len;
    if (S > kMaxSplits) S = kMaxSplits;
    if (S < 1) S = 1;
    int64_t tps = (p.n_vt + S - 1) / S;
    if (tps < 1) tps = 1;
    S = (p.n_vt + tps - 1) / tps;
    if (S < 1) S = 1;   // also a cache that holds only the sink token: one split, no tiles
    p.splits = (int32_t)S;
    p.tiles_per_split = (int32_t)tps;
    return p;
}

int check_ragged(const kvq_shape *s, const kvq_ragged *c) {
    int e = check_shape(s);
    if (e) return e;
    if (s->bits != 2 || s->flags != 0) return KVQ_E_BITS;
    if (!c) return KVQ_E_NULL;
    if (!c->tiles || !c->k_res || !c->v_res || !c->lens) return KVQ_E_NULL;
    if (!aligned16(c->tiles) || !aligned16(c->k_res) || !aligned16(c->v_res) || !aligned16(c->lens))
        return KVQ_E_ALIGN;
    if (s->max_tokens > 0x7fffffffLL - s->residual_cap) return KVQ_E_SHAPE;   // lengths are int32 on the device
    return KVQ_OK;
}

// Split plan of a ragged cache: fixed by the capacity (every sequence could be full), so a captured step stays
// valid as lengths grow; each sequence spreads its own tiles over these splits.
SplitPlan ragged_plan(const kvq_shape *s) {
    kvq_cache full{};
    full.n_quant = s->max_tokens;
    full.n_resid = s->residual_cap;
    return plan(s, &full);
}

kvq::DecodeArgs ragged_args(const kvq_shape *shape, const kvq_ragged *cache, const SplitPlan &p, const void *q,
                            float sm_scale, float *out, void *workspace, int appended) {
    kvq::DecodeArgs a;
    a.tiles = static_cast<const uint8_t *>(cache->tiles);
    a.k_res = static_cast<const _Float16 *>(cache->k_res);
    a.v_res = static_cast<const _Float16 *>(cache->v_res);
    a.q = static_cast<const _Float16 *>(q);
    a.part_o = static_cast<float *>(workspace);
    a.part_ml = a.part_o + (size_t)shape->batch * shape->q_heads * p.splits * KVQ_HEAD_DIM;
    a.out = out;
    a.max_tiles = shape->max_tokens / KVQ_TILE_TOKENS;
    a.n_qtiles = 0;
    a.n_resid = 0;
    a.res_cap = shape->residual_cap;
    a.batch = shape->batch;
    a.kv_heads = shape->kv_heads;
    a.q_heads = shape->q_heads;
    a.chunks = p.chunks;
    a.tiles_per_split = 0;
    a.sm_log2 = (sm_scale > 0.0f ? sm_scale : 1.0f / sqrtf((float)KVQ_HEAD_DIM)) * 1.4426950408889634f;
    a.sparse = 0;
    a.lens = cache->lens;
    a.appended = appended;
    a.k_new = nullptr;
    a.v_new = nullptr;
    a.new_sb = a.new_sh = 0;
    a.tiles_w = nullptr;
    a.k_res_w = nullptr;
    a.v_res_w = nullptr;
    a.lens_w = nullptr;
    a.sync = nullptr;
    return a;
}

int check_decode_io(const kvq_shape *shape, const SplitPlan &p, const void *q, const float *out, const void *ws,
                    size_t ws_bytes) {
    if (!q || !out) return KVQ_E_NULL;
    if (!aligned16(q) || !aligned16(out)) return KVQ_E_ALIGN;
    const size_t need = (size_t)shape->batch * shape->q_heads * p.splits * (KVQ_HEAD_DIM + 2) * sizeof(float);
    if (!ws || ws_bytes < need) return KVQ_E_WORKSPACE;
    if (!aligned16(ws)) return KVQ_E_ALIGN;
    return KVQ_OK;
}

}  // namespace

extern "C" {

const char *kvq_status_string(int status) {
    switch (status) {
        case KVQ_OK: return "ok";
        case KVQ_E_NULL: return "null pointer";
        case KVQ_E_SHAPE: return "unsupported shape or size";
        case KVQ_E_BITS: return "unsupported bit width";
        case KVQ_E_ALIGN: return "misaligned pointer or stride";
        case KVQ_E_CAPACITY: return "cache capacity exceeded";
        case KVQ_E_WORKSPACE: return "workspace missing or too small";
        case KVQ_E_EMPTY: return "attention over an empty cache";
        case KVQ_E_LAUNCH: return "HIP launch error";
        case KVQ_E_STATE: return "inconsistent cache state";
        case KVQ_E_SCRATCH: return "call needs more scratch than the static array holds";
        default: return "unknown status";
    }
}

int kv_quant_keys_per_channel(const kvq_shape *shape, const void *k, int64_t stride_b, int64_t stride_h,
                              int64_t stride_t, int64_t n_tokens, int64_t tile0, void *tiles, void *stream) {
    return quant_common(shape, k, stride_b, stride_h, stride_t, n_tokens, tile0, tiles, true, stream);
}

int kv_quant_values_per_token(const kvq_shape *shape, const void *v, int64_t stride_b, int64_t stride_h,
                              int64_t stride_t, int64_t n_tokens, int64_t tile0, void *tiles, void *stream) {
    return quant_common(shape, v, stride_b, stride_h, stride_t, n_tokens, tile0, tiles, false, stream);
}

int kv_append_and_flush(const kvq_shape *shape, kvq_cache *cache, const void *k_new, const void *v_new,
                        int64_t stride_b, int64_t stride_h, int64_t stride_t, int64_t n_tokens, void *stream) {
    int e = check_shape(shape);
    if (e) return e;
    if ((e = check_cache(shape, cache))) return e;
    if ((e = check_src(k_new, stride_b, stride_h, stride_t))) return e;
    if ((e = check_src(v_new, stride_b, stride_h, stride_t))) return e;
    if (n_tokens <= 0) return KVQ_E_SHAPE;
    // with a sink, the first token of an empty cache becomes the sink; the rest follows the window rule
    const int64_t take_sink = (has_sink(shape) && cache->n_sink == 0) ? 1 : 0;
    const int64_t n_rest = n_tokens - take_sink;
    const int64_t R = shape->residual_cap;
    const int64_t nr0 = cache->n_resid;
    const int64_t flushed = n_rest > 0 ? R * ((nr0 + n_rest - 1) / R) : 0;
    if (cache->n_quant + flushed > shape->max_tokens) return KVQ_E_CAPACITY;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const int B = shape->batch, H = shape->kv_heads;
    kvq::TokSrc knew = single_src(k_new, stride_b, stride_h, stride_t);
    kvq::TokSrc vnew = single_src(v_new, stride_b, stride_h, stride_t);
    if (take_sink) {
        if ((e = launched(kvq::launch_sink_b4(knew, vnew, B, H, static_cast<uint8_t *>(cache->sink), is_sparse(shape),
                                              s))))
            return e;
        cache->n_sink = 1;
        if (n_rest == 0) return KVQ_OK;
        knew = single_src(static_cast<const _Float16 *>(k_new) + stride_t, stride_b, stride_h, stride_t);
        vnew = single_src(static_cast<const _Float16 *>(v_new) + stride_t, stride_b, stride_h, stride_t);
    }
    const int64_t max_tiles = shape->max_tokens / KVQ_TILE_TOKENS;
    _Float16 *kres = static_cast<_Float16 *>(cache->k_res);
    _Float16 *vres = static_cast<_Float16 *>(cache->v_res);
    int64_t copy_from, dst0;
    if (flushed > 0) {
        // the flushed tokens: the whole window, then the first flushed - nr0 new tokens
        kvq::TokSrc ksrc = knew, vsrc = vnew;
        ksrc.a = kres; vsrc.a = vres;
        ksrc.a_sb = vsrc.a_sb = (int64_t)H * R * KVQ_HEAD_DIM;
        ksrc.a_sh = vsrc.a_sh = R * KVQ_HEAD_DIM;
        ksrc.a_st = vsrc.a_st = KVQ_HEAD_DIM;
        ksrc.n_a = vsrc.n_a = nr0;
        uint8_t *tiles = static_cast<uint8_t *>(cache->tiles);
        const int64_t tile0 = cache->n_quant / KVQ_TILE_TOKENS, nt = flushed / KVQ_TILE_TOKENS;
        if ((e = launched(quant_launch(shape, true, ksrc, nt, tiles, max_tiles, tile0, s)))) return e;
        if ((e = launched(quant_launch(shape, false, vsrc, nt, tiles, max_tiles, tile0, s)))) return e;
        copy_from = flushed - nr0;
        dst0 = 0;
    } else {
        copy_from = 0;
        dst0 = nr0;
    }
    const int64_t n_copy = n_rest - copy_from;
    if ((e = launched(kvq::launch_copy_rows(knew, vnew, copy_from, n_copy, B, H, kres, vres, (int)R, (int)dst0, s))))
        return e;
    cache->n_quant += flushed;
    cache->n_resid = (int32_t)(dst0 + n_copy);
    return KVQ_OK;
}

int32_t kv_decode_attention_splits(const kvq_shape *shape, const kvq_cache *cache) {
    if (check_shape(shape) || check_cache(shape, cache)) return 0;
    const SplitPlan p = plan(shape, cache);
    return (p.n_vt > 0 || cache->n_sink > 0) ? p.splits : 0;
}

size_t kv_decode_attention_workspace_bytes(const kvq_shape *shape, const kvq_cache *cache) {
    const int32_t S = kv_decode_attention_splits(shape, cache);
    if (S <= 0) return 0;
    return (size_t)shape->batch * shape->q_heads * S * (KVQ_HEAD_DIM + 2) * sizeof(float);
}

}  // extern "C"

namespace {

// Host checks shared by both decode entry points; on success `p` is the split plan and `need` the partials' bytes.
int decode_checks(const kvq_shape *shape, const kvq_cache *cache, const void *q, const float *out, SplitPlan &p,
                  size_t &need) {
    int e = check_shape(shape);
    if (e) return e;
    if ((e = check_cache(shape, cache))) return e;
    if (!q || !out) return KVQ_E_NULL;
    if (!aligned16(q) || !aligned16(out)) return KVQ_E_ALIGN;
    p = plan(shape, cache);
    if (p.n_vt == 0 && cache->n_sink == 0) return KVQ_E_EMPTY;
    need = (size_t)shape->batch * shape->q_heads * p.splits * (KVQ_HEAD_DIM + 2) * sizeof(float);
    return KVQ_OK;
}

// Both passes of one decode call with the split partials at `workspace` (validated by the caller).
int decode_launch(const kvq_shape *shape, const kvq_cache *cache, const SplitPlan &p, const void *q, float sm_scale,
                  float *out, void *workspace, void *stream) {
    if (!(sm_scale > 0.0f)) sm_scale = 1.0f / sqrtf((float)KVQ_HEAD_DIM);
    float *part_o = static_cast<float *>(workspace);
    float *part_ml = part_o + (size_t)shape->batch * shape->q_heads * p.splits * KVQ_HEAD_DIM;
    hipStream_t st = static_cast<hipStream_t>(stream);

    if (shape->bits == 4) {
        kvq::DecodeB4Args a;
        a.tiles = static_cast<const uint8_t *>(cache->tiles);
        a.sink = static_cast<const uint8_t *>(cache->sink);
        a.k_res = static_cast<const _Float16 *>(cache->k_res);
        a.v_res = static_cast<const _Float16 *>(cache->v_res);
        a.q = static_cast<const _Float16 *>(q);
        a.part_o = part_o;
        a.part_ml = part_ml;
        a.max_tiles = shape->max_tokens / KVQ_TILE_TOKENS;
        a.n_sink = cache->n_sink;
        a.n_qtiles = (int)(cache->n_quant / KVQ_TILE_TOKENS);
        a.n_resid = cache->n_resid;
        a.res_cap = shape->residual_cap;
        a.batch = shape->batch;
        a.kv_heads = shape->kv_heads;
        a.q_heads = shape->q_heads;
        a.tiles_per_split = p.tiles_per_split;
        a.sm_log2 = sm_scale * 1.4426950408889634f;
        a.rope = (shape->flags & KVQ_FLAG_PRE_ROPE) ? 1 : 0;
        a.sparse = is_sparse(shape) ? 1 : 0;
        a.log2_base = a.rope ? log2(shape->rope_base) : 0.0;
        return launched(kvq::launch_decode_b4(a, out, p.splits, st));
    }

    kvq::DecodeArgs a;
    a.tiles = static_cast<const uint8_t *>(cache->tiles);
    a.k_res = static_cast<const _Float16 *>(cache->k_res);
    a.v_res = static_cast<const _Float16 *>(cache->v_res);
    a.q = static_cast<const _Float16 *>(q);
    a.part_o = part_o;
    a.part_ml = part_ml;
    a.out = out;
    a.max_tiles = shape->max_tokens / KVQ_TILE_TOKENS;
    a.n_qtiles = (int)(cache->n_quant / KVQ_TILE_TOKENS);
    a.n_resid = cache->n_resid;
    a.res_cap = shape->residual_cap;
    a.batch = shape->batch;
    a.kv_heads = shape->kv_heads;
    a.q_heads = shape->q_heads;
    a.chunks = p.chunks;
    a.tiles_per_split = p.tiles_per_split;
    a.sm_log2 = sm_scale * 1.4426950408889634f;
    a.sparse = is_sparse(shape) ? 1 : 0;
    a.lens = nullptr;
    a.appended = 0;
    a.k_new = nullptr;
    a.v_new = nullptr;
    a.new_sb = a.new_sh = 0;
    a.tiles_w = nullptr;
    a.k_res_w = nullptr;
    a.v_res_w = nullptr;
    a.lens_w = nullptr;
    a.sync = nullptr;
    return launched(kvq::launch_decode(a, p.splits, st));
}

}  // namespace

extern "C" {

int kv_decode_attention(const kvq_shape *shape, const kvq_cache *cache, const void *q, float sm_scale, float *out,
                        void *workspace, size_t workspace_bytes, void *stream) {
    SplitPlan p;
    size_t need = 0;
    int e = decode_checks(shape, cache, q, out, p, need);
    if (e) return e;
    if (!workspace || workspace_bytes < need) return KVQ_E_WORKSPACE;
    if (!aligned16(workspace)) return KVQ_E_ALIGN;
    return decode_launch(shape, cache, p, q, sm_scale, out, workspace, stream);
}

int kv_decode_attention_noalloc(const kvq_shape *shape, const kvq_cache *cache, const void *q, float sm_scale,
                                float *out, void *stream) {
    SplitPlan p;
    size_t need = 0;
    int e = decode_checks(shape, cache, q, out, p, need);
    if (e) return e;
    if (need > (size_t)KVQ_NOALLOC_SCRATCH_BYTES) return KVQ_E_SCRATCH;   // before any runtime call
    void *ws = nullptr;
    if ((e = scratch_address(&ws))) return e;
    return decode_launch(shape, cache, p, q, sm_scale, out, ws, stream);
}

int kv_ragged_prefill(const kvq_shape *shape, const kvq_ragged *cache, int32_t b, const void *k, const void *v,
                      int64_t stride_h, int64_t stride_t, int64_t n_tokens, void *stream) {
    int e = check_ragged(shape, cache);
    if (e) return e;
    if (b < 0 || b >= shape->batch || n_tokens < 0) return KVQ_E_SHAPE;
    const int64_t R = shape->residual_cap;
    const int64_t flushed = n_tokens > 0 ? R * ((n_tokens - 1) / R) : 0;
    if (flushed > shape->max_tokens) return KVQ_E_CAPACITY;
    if (n_tokens > 0) {
        if ((e = check_src(k, 0, stride_h, stride_t))) return e;
        if ((e = check_src(v, 0, stride_h, stride_t))) return e;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int H = shape->kv_heads;
    const int64_t max_tiles = shape->max_tokens / KVQ_TILE_TOKENS;
    // sequence b alone, as a batch of one
    uint8_t *tiles = static_cast<uint8_t *>(cache->tiles) + (int64_t)b * H * max_tiles * KVQ_RECORD_BYTES;
    _Float16 *kres = static_cast<_Float16 *>(cache->k_res) + (int64_t)b * H * R * KVQ_HEAD_DIM;
    _Float16 *vres = static_cast<_Float16 *>(cache->v_res) + (int64_t)b * H * R * KVQ_HEAD_DIM;
    if (n_tokens > 0) {
        const kvq::TokSrc ks = single_src(k, 0, stride_h, stride_t), vs = single_src(v, 0, stride_h, stride_t);
        // the flushed tiles, then (written ahead, within the capacity) the complete 32-row blocks of the window:
        // tile i holds tokens 32 i .. 32 i + 31 either way
        const int64_t nt = std::min(n_tokens / KVQ_TILE_TOKENS, max_tiles);
        if (nt > 0) {
            if ((e = launched(kvq::launch_quant_keys(ks, 0, nt, 1, H, tiles, max_tiles, 0, false, s)))) return e;
            if ((e = launched(kvq::launch_quant_values(vs, 0, nt, 1, H, tiles, max_tiles, 0, false, s)))) return e;
        }
        const int64_t n_copy = n_tokens - flushed;
        if ((e = launched(kvq::launch_copy_rows(ks, vs, flushed, n_copy, 1, H, kres, vres, (int)R, 0, s)))) return e;
    }
    return launched(kvq::launch_ragged_set(cache->lens, b, (int)flushed, (int)(n_tokens - flushed), 0, s));
}

int kv_ragged_append(const kvq_shape *shape, const kvq_ragged *cache, const void *k_new, const void *v_new,
                     int64_t stride_b, int64_t stride_h, void *stream) {
    int e = check_ragged(shape, cache);
    if (e) return e;
    if ((e = check_src(k_new, stride_b, stride_h, 0))) return e;
    if ((e = check_src(v_new, stride_b, stride_h, 0))) return e;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const kvq::TokSrc kn = single_src(k_new, stride_b, stride_h, 0), vn = single_src(v_new, stride_b, stride_h, 0);
    if ((e = launched(kvq::launch_ragged_flush_append(
             kn, vn, shape->batch, shape->kv_heads, static_cast<uint8_t *>(cache->tiles),
             shape->max_tokens / KVQ_TILE_TOKENS, static_cast<_Float16 *>(cache->k_res),
             static_cast<_Float16 *>(cache->v_res), shape->residual_cap, cache->lens, s))))
        return e;
    return launched(kvq::launch_ragged_commit(cache->lens, shape->batch, shape->residual_cap, s));
}

int32_t kv_ragged_splits(const kvq_shape *shape) {
    if (check_shape(shape) || shape->bits != 2 || shape->flags != 0) return 0;
    return ragged_plan(shape).splits;
}

size_t kv_ragged_workspace_bytes(const kvq_shape *shape) {
    const int32_t S = kv_ragged_splits(shape);
    if (S <= 0) return 0;
    return (size_t)shape->batch * shape->q_heads * S * (KVQ_HEAD_DIM + 2) * sizeof(float);
}

int kv_ragged_decode_attention(const kvq_shape *shape, const kvq_ragged *cache, const void *q, float sm_scale,
                               float *out, void *workspace, size_t workspace_bytes, void *stream) {
    int e = check_ragged(shape, cache);
    if (e) return e;
    const SplitPlan p = ragged_plan(shape);
    if ((e = check_decode_io(shape, p, q, out, workspace, workspace_bytes))) return e;
    const kvq::DecodeArgs a = ragged_args(shape, cache, p, q, sm_scale, out, workspace, 0);
    return launched(kvq::launch_decode_ragged(a, p.splits, cache->lens, 0, static_cast<hipStream_t>(stream)));
}

int kv_ragged_decode_step(const kvq_shape *shape, const kvq_ragged *cache, const void *k_new, const void *v_new,
                          int64_t stride_b, int64_t stride_h, const void *q, float sm_scale, float *out,
                          void *workspace, size_t workspace_bytes, void *stream) {
    int e = check_ragged(shape, cache);
    if (e) return e;
    if ((e = check_src(k_new, stride_b, stride_h, 0))) return e;
    if ((e = check_src(v_new, stride_b, stride_h, 0))) return e;
    const SplitPlan p = ragged_plan(shape);
    if ((e = check_decode_io(shape, p, q, out, workspace, workspace_bytes))) return e;
    if (!cache->sync) return KVQ_E_NULL;
    if ((reinterpret_cast<uintptr_t>(cache->sync) & 3u) != 0) return KVQ_E_ALIGN;
    kvq::DecodeArgs a = ragged_args(shape, cache, p, q, sm_scale, out, workspace, 0);
    a.k_new = static_cast<const _Float16 *>(k_new);
    a.v_new = static_cast<const _Float16 *>(v_new);
    a.new_sb = stride_b;
    a.new_sh = stride_h;
    a.tiles_w = static_cast<uint8_t *>(cache->tiles);
    a.k_res_w = static_cast<_Float16 *>(cache->k_res);
    a.v_res_w = static_cast<_Float16 *>(cache->v_res);
    a.lens_w = cache->lens;
    a.sync = cache->sync;
    return launched(kvq::launch_decode_step(a, p.splits, static_cast<hipStream_t>(stream)));
}

size_t kv_ragged_sync_words(const kvq_shape *shape) {
    if (check_shape(shape) || shape->bits != 2 || shape->flags != 0) return 0;
    const int64_t chunks = (shape->q_heads / shape->kv_heads + 3) / 4;
    return (size_t)shape->batch * (size_t)(1 + (int64_t)shape->kv_heads * chunks);
}

}  // extern "C"
