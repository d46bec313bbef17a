// C ABI of libh2o.so (declared in include/h2o.h): argument validation on the
// host, workspace sizing, and kernel launches on the caller's stream.
// Nothing here allocates, frees or synchronises (unless H2O_SYNC_DEBUG=1 is
// set in the environment, which synchronises after every launch to pin a
// fault to its kernel).
#include "h2o.h"
#include "h2o_device.h"
#include "h2o_launch.h"

#include <math.h>
#include <stdlib.h>

#include <mutex>
#include <vector>

// Scratch of h2o_attn_chunk_static: one copy per device (the code object's
// globals are instantiated on every device it is loaded on).  Host code
// never uses this name as an address: it looks up each device's copy with
// hipGetSymbolAddress and passes that pointer to the kernels.
static __device__ __align__(256) unsigned char scratch[H2O_STATIC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t device_scratch(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p || ((uintptr_t)p & 255u)) return hipErrorInvalidValue;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

bool sync_debug() {
    static const bool on = [] {
        const char* e = getenv("H2O_SYNC_DEBUG");
        return e && e[0] == '1';
    }();
    return on;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Shape checks shared by every entry point.
h2o_status_t check_shape(const h2o_shape_t* s) {
    if (!s) return H2O_ERR_INVALID_ARG;
    if (s->batch < 1 || s->n_q_heads < 1 || s->n_kv_heads < 1 || s->cache_len < 1 ||
        s->chunk_len < 1)
        return H2O_ERR_INVALID_ARG;
    if (s->n_q_heads % s->n_kv_heads != 0) return H2O_ERR_INVALID_ARG;
    if (s->chunk_len > s->cache_len) return H2O_ERR_INVALID_ARG;
    if (s->n_valid < 0 || s->n_valid > s->cache_len) return H2O_ERR_INVALID_ARG;
    if (!(s->scale == s->scale)) return H2O_ERR_INVALID_ARG;   // NaN scale
    if (s->head_dim != 64 && s->head_dim != 128) return H2O_ERR_UNSUPPORTED;
    if (s->cache_len > (1 << 20)) return H2O_ERR_UNSUPPORTED;   // in-head indices stay 32-bit
    // 32-bit index limits used inside the kernels
    const long long BH = (long long)s->batch * s->n_kv_heads;
    const long long W = (long long)s->cache_len + s->chunk_len;
    if (BH * W >= (1ll << 31) || (long long)s->n_q_heads / s->n_kv_heads * s->chunk_len >= (1ll << 30) ||
        BH >= 65536)
        return H2O_ERR_UNSUPPORTED;
    return H2O_OK;
}

h2o_status_t from_hip(hipError_t e) { return e == hipSuccess ? H2O_OK : H2O_ERR_HIP; }

bool overlaps(const void* a, size_t a_bytes, const void* b, size_t b_bytes) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + b_bytes && y < x + a_bytes;
}

// Event timing of the attention kernels (diagnostics, one thread).
struct Timing {
    bool on = false;
    int max_calls = 0;
    int used = 0;
    std::vector<hipEvent_t> ev;
};
Timing g_timing;

hipEvent_t* timing_slot() {
    if (!g_timing.on || g_timing.used >= g_timing.max_calls) return nullptr;
    return &g_timing.ev[(size_t)5 * g_timing.used++];
}

}  // namespace

extern "C" {

size_t h2o_workspace_size(const h2o_shape_t* s) {
    if (check_shape(s) != H2O_OK) return 0;
    h2o::AttnPlan pl;
    h2o::make_attn_plan(s->batch, s->n_q_heads, s->n_kv_heads, s->head_dim, s->cache_len,
                        s->chunk_len, s->n_valid, s->scale, &pl);
    return pl.bytes;
}

h2o_status_t h2o_attn_chunk(const h2o_shape_t* s, const uint16_t* q, const uint16_t* k_cache,
                            const uint16_t* v_cache, const uint16_t* k_new,
                            const uint16_t* v_new, float* out, float* lse, float* wsum,
                            void* ws, size_t ws_bytes, void* stream) {
    h2o_status_t st = check_shape(s);
    if (st != H2O_OK) return st;
    if (!q || !k_cache || !v_cache || !k_new || !v_new || !out || !wsum)
        return H2O_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) ||
        !aligned16(v_new) || !aligned16(out) || !aligned16(wsum) || (lse && !aligned16(lse)))
        return H2O_ERR_INVALID_ARG;
    h2o::AttnPlan pl;
    h2o::make_attn_plan(s->batch, s->n_q_heads, s->n_kv_heads, s->head_dim, s->cache_len,
                        s->chunk_len, s->n_valid, s->scale, &pl);
    if (!ws || ((uintptr_t)ws & 255u) || ws_bytes < pl.bytes) return H2O_ERR_WORKSPACE;
    return from_hip(h2o::launch_attention(pl, q, k_cache, v_cache, k_new, v_new, out, lse,
                                          wsum, ws, (hipStream_t)stream, sync_debug(),
                                          timing_slot()));
}

h2o_status_t h2o_attn_chunk_static(const h2o_shape_t* s, const uint16_t* q,
                                   const uint16_t* k_cache, const uint16_t* v_cache,
                                   const uint16_t* k_new, const uint16_t* v_new, float* out,
                                   float* lse, float* wsum, void* stream) {
    h2o_status_t st = check_shape(s);
    if (st != H2O_OK) return st;
    if (!q || !k_cache || !v_cache || !k_new || !v_new || !out || !wsum)
        return H2O_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) ||
        !aligned16(v_new) || !aligned16(out) || !aligned16(wsum) || (lse && !aligned16(lse)))
        return H2O_ERR_INVALID_ARG;
    h2o::AttnPlan pl;
    h2o::make_attn_plan(s->batch, s->n_q_heads, s->n_kv_heads, s->head_dim, s->cache_len,
                        s->chunk_len, s->n_valid, s->scale, &pl);
    if (pl.bytes > H2O_STATIC_SCRATCH_BYTES) return H2O_ERR_WORKSPACE;
    void* ws = nullptr;
    st = from_hip(device_scratch(&ws));
    if (st != H2O_OK) return st;
    return from_hip(h2o::launch_attention(pl, q, k_cache, v_cache, k_new, v_new, out, lse,
                                          wsum, ws, (hipStream_t)stream, sync_debug(),
                                          timing_slot()));
}

h2o_status_t h2o_score_accumulate(const h2o_shape_t* s, float* scores, float* new_scores,
                                  const float* wsum, void* stream) {
    h2o_status_t st = check_shape(s);
    if (st != H2O_OK) return st;
    if (!scores || !new_scores || !wsum) return H2O_ERR_INVALID_ARG;
    if (!aligned16(scores) || !aligned16(new_scores) || !aligned16(wsum))
        return H2O_ERR_INVALID_ARG;
    hipError_t e = h2o::launch_score_accumulate(s->batch * s->n_kv_heads, s->cache_len,
                                                s->chunk_len, s->n_valid, scores, new_scores,
                                                wsum, (hipStream_t)stream);
    if (e == hipSuccess && sync_debug()) e = hipStreamSynchronize((hipStream_t)stream);
    return from_hip(e);
}

h2o_status_t h2o_evict_select(const h2o_shape_t* s, const float* scores, int32_t* evict_idx,
                              void* stream) {
    h2o_status_t st = check_shape(s);
    if (st != H2O_OK) return st;
    if (!scores || !evict_idx) return H2O_ERR_INVALID_ARG;
    if (!aligned16(scores) || !aligned16(evict_idx)) return H2O_ERR_INVALID_ARG;
    hipError_t e = h2o::launch_evict_select(s->batch * s->n_kv_heads, s->cache_len,
                                            s->chunk_len, s->n_valid, scores, evict_idx,
                                            (hipStream_t)stream);
    if (e == hipSuccess && sync_debug()) e = hipStreamSynchronize((hipStream_t)stream);
    return from_hip(e);
}

h2o_status_t kv_scatter(const h2o_shape_t* s, uint16_t* k_cache, uint16_t* v_cache,
                        float* scores, int64_t* pos, const uint16_t* k_new,
                        const uint16_t* v_new, const float* new_scores,
                        const int32_t* evict_idx, int64_t p0, void* stream) {
    h2o_status_t st = check_shape(s);
    if (st != H2O_OK) return st;
    if (!k_cache || !v_cache || !scores || !k_new || !v_new || !new_scores || !evict_idx)
        return H2O_ERR_INVALID_ARG;
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(scores) ||
        !aligned16(k_new) || !aligned16(v_new) || !aligned16(new_scores) ||
        !aligned16(evict_idx) || (pos && !aligned16(pos)))
        return H2O_ERR_INVALID_ARG;
    if (p0 < 0) return H2O_ERR_INVALID_ARG;
    hipError_t e = h2o::launch_kv_scatter(s->batch * s->n_kv_heads, s->head_dim, s->cache_len,
                                          s->chunk_len, k_cache, v_cache, scores, pos, k_new,
                                          v_new, new_scores, evict_idx, p0,
                                          (hipStream_t)stream);
    if (e == hipSuccess && sync_debug()) e = hipStreamSynchronize((hipStream_t)stream);
    return from_hip(e);
}

h2o_status_t h2o_step(const h2o_shape_t* s, const uint16_t* q, uint16_t* k_cache,
                      uint16_t* v_cache, const uint16_t* k_new, const uint16_t* v_new, float* out,
                      float* lse, float* wsum, float* scores, float* new_scores,
                      int32_t* evict_idx, int64_t* pos, int64_t p0, void* ws, size_t ws_bytes,
                      void* stream) {
    h2o_status_t st = check_shape(s);
    if (st != H2O_OK) return st;
    const void* req[] = {q, k_cache, v_cache, k_new, v_new, out, wsum, scores, new_scores,
                         evict_idx};
    for (const void* p : req)
        if (!p || !aligned16(p)) return H2O_ERR_INVALID_ARG;
    if ((lse && !aligned16(lse)) || (pos && !aligned16(pos)) || p0 < 0)
        return H2O_ERR_INVALID_ARG;
    h2o::AttnPlan pl;
    h2o::make_attn_plan(s->batch, s->n_q_heads, s->n_kv_heads, s->head_dim, s->cache_len,
                        s->chunk_len, s->n_valid, s->scale, &pl);
    if (!ws || ((uintptr_t)ws & 255u) || ws_bytes < pl.bytes) return H2O_ERR_WORKSPACE;
    const hipStream_t str = (hipStream_t)stream;
    if (h2o::decode_tail_applies(pl))
        return from_hip(h2o::launch_decode_step(pl, q, k_cache, v_cache, k_new, v_new, out, lse,
                                                wsum, scores, new_scores, evict_idx, pos, p0,
                                                ws, str, sync_debug(), timing_slot()));
    const int BH = s->batch * s->n_kv_heads;
    // the kernel that writes the summed weights also accumulates the scores;
    // the choice and the scatter share one kernel where the keys fit in
    // registers and the chunk is short
    hipError_t e = h2o::launch_attention(pl, q, k_cache, v_cache, k_new, v_new, out, lse, wsum,
                                         ws, str, sync_debug(), timing_slot(), scores,
                                         new_scores);
    if (e == hipSuccess && h2o::select_scatter_fuses(s->cache_len, s->chunk_len, s->head_dim)) {
        e = h2o::launch_select_scatter(BH, s->head_dim, s->cache_len, s->chunk_len, s->n_valid,
                                       scores, evict_idx, k_cache, v_cache, pos, k_new, v_new,
                                       new_scores, p0, str);
    } else {
        if (e == hipSuccess)
            e = h2o::launch_evict_select(BH, s->cache_len, s->chunk_len, s->n_valid, scores,
                                         evict_idx, str);
        if (e == hipSuccess)
            e = h2o::launch_kv_scatter(BH, s->head_dim, s->cache_len, s->chunk_len, k_cache,
                                       v_cache, scores, pos, k_new, v_new, new_scores, evict_idx,
                                       p0, str);
    }
    if (e == hipSuccess && sync_debug()) e = hipStreamSynchronize(str);
    return from_hip(e);
}

h2o_status_t h2o_attn_chunk_q8(const h2o_shape_t* s, const uint16_t* q, const int8_t* k_cache,
                               const float* k_scale, const int8_t* v_cache,
                               const float* v_scale, const uint16_t* k_new,
                               const uint16_t* v_new, float* out, float* lse, float* wsum,
                               void* ws, size_t ws_bytes, void* stream) {
    h2o_status_t st = check_shape(s);
    if (st != H2O_OK) return st;
    if (!q || !k_cache || !k_scale || !v_cache || !v_scale || !k_new || !v_new || !out || !wsum)
        return H2O_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(k_scale) || !aligned16(v_cache) ||
        !aligned16(v_scale) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out) ||
        !aligned16(wsum) || (lse && !aligned16(lse)))
        return H2O_ERR_INVALID_ARG;
    h2o::AttnPlan pl;
    h2o::make_attn_plan(s->batch, s->n_q_heads, s->n_kv_heads, s->head_dim, s->cache_len,
                        s->chunk_len, s->n_valid, s->scale, &pl);
    if (!ws || ((uintptr_t)ws & 255u) || ws_bytes < pl.bytes) return H2O_ERR_WORKSPACE;
    return from_hip(h2o::launch_attention_q8(pl, q, k_cache, k_scale, v_cache, v_scale, k_new,
                                             v_new, out, lse, wsum, ws, (hipStream_t)stream,
                                             sync_debug(), timing_slot()));
}

h2o_status_t kv_scatter_q8(const h2o_shape_t* s, int8_t* k_cache, float* k_scale,
                           int8_t* v_cache, float* v_scale, float* scores, int64_t* pos,
                           const uint16_t* k_new, const uint16_t* v_new,
                           const float* new_scores, const int32_t* evict_idx, int64_t p0,
                           void* stream) {
    h2o_status_t st = check_shape(s);
    if (st != H2O_OK) return st;
    if (!k_cache || !k_scale || !v_cache || !v_scale || !scores || !k_new || !v_new ||
        !new_scores || !evict_idx)
        return H2O_ERR_INVALID_ARG;
    if (!aligned16(k_cache) || !aligned16(k_scale) || !aligned16(v_cache) ||
        !aligned16(v_scale) || !aligned16(scores) || !aligned16(k_new) || !aligned16(v_new) ||
        !aligned16(new_scores) || !aligned16(evict_idx) || (pos && !aligned16(pos)))
        return H2O_ERR_INVALID_ARG;
    if (p0 < 0) return H2O_ERR_INVALID_ARG;
    hipError_t e = h2o::launch_kv_scatter_q8(s->batch * s->n_kv_heads, s->head_dim,
                                             s->cache_len, s->chunk_len, k_cache, k_scale,
                                             v_cache, v_scale, scores, pos, k_new, v_new,
                                             new_scores, evict_idx, p0, (hipStream_t)stream);
    if (e == hipSuccess && sync_debug()) e = hipStreamSynchronize((hipStream_t)stream);
    return from_hip(e);
}

h2o_status_t h2o_quantize_rows_q8(const uint16_t* x, int64_t n_rows, int32_t head_dim,
                                  int8_t* codes, float* scales, void* stream) {
    if (head_dim != 64 && head_dim != 128) return H2O_ERR_UNSUPPORTED;
    if (n_rows < 0 || n_rows >= (1ll << 31) / 16) return H2O_ERR_INVALID_ARG;
    if (!x || !codes || !scales || !aligned16(x) || !aligned16(codes) || !aligned16(scales))
        return H2O_ERR_INVALID_ARG;
    if (n_rows == 0) return H2O_OK;
    hipError_t e = h2o::launch_quantize_rows(x, (long)n_rows, head_dim, codes, scales,
                                             (hipStream_t)stream);
    if (e == hipSuccess && sync_debug()) e = hipStreamSynchronize((hipStream_t)stream);
    return from_hip(e);
}

h2o_status_t h2o_snapkv_select(const h2o_shape_t* s, const float* wsum, int32_t budget,
                               int32_t* keep_idx, void* stream) {
    h2o_status_t st = check_shape(s);
    if (st != H2O_OK) return st;
    if (budget < 0 || budget > s->n_valid) return H2O_ERR_INVALID_ARG;
    if (!wsum || (budget > 0 && !keep_idx)) return H2O_ERR_INVALID_ARG;
    if (!aligned16(wsum) || (keep_idx && !aligned16(keep_idx))) return H2O_ERR_INVALID_ARG;
    hipError_t e = h2o::launch_snapkv_select(s->batch * s->n_kv_heads, s->cache_len,
                                             s->chunk_len, s->n_valid, budget, wsum, keep_idx,
                                             (hipStream_t)stream);
    if (e == hipSuccess && sync_debug()) e = hipStreamSynchronize((hipStream_t)stream);
    return from_hip(e);
}

h2o_status_t h2o_snapkv_compact(const h2o_shape_t* s, const uint16_t* k_cache,
                                const uint16_t* v_cache, const int64_t* pos,
                                const uint16_t* k_new, const uint16_t* v_new, const float* wsum,
                                const int32_t* keep_idx, int32_t budget, int32_t out_len,
                                int64_t p0, uint16_t* k_out, uint16_t* v_out, int64_t* pos_out,
                                float* scores_out, void* stream) {
    h2o_status_t st = check_shape(s);
    if (st != H2O_OK) return st;
    if (budget < 0 || budget > s->n_valid) return H2O_ERR_INVALID_ARG;
    if (out_len < 1 || out_len > (1 << 20) || (long long)budget + s->chunk_len > out_len)
        return H2O_ERR_INVALID_ARG;
    if (!k_cache || !v_cache || !k_new || !v_new || !wsum || !k_out || !v_out ||
        (budget > 0 && !keep_idx) || (pos_out && !pos))
        return H2O_ERR_INVALID_ARG;
    if (p0 < 0) return H2O_ERR_INVALID_ARG;
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new) ||
        !aligned16(k_out) || !aligned16(v_out) || !aligned16(wsum) ||
        (keep_idx && !aligned16(keep_idx)) || (pos && !aligned16(pos)) ||
        (pos_out && !aligned16(pos_out)) || (scores_out && !aligned16(scores_out)))
        return H2O_ERR_INVALID_ARG;
    const size_t BH = (size_t)s->batch * s->n_kv_heads, D = s->head_dim;
    const size_t out_b = BH * out_len * D * 2, cache_b = BH * s->cache_len * D * 2,
                 new_b = BH * s->chunk_len * D * 2;
    const void* srcs[4] = {k_cache, v_cache, k_new, v_new};
    const size_t src_b[4] = {cache_b, cache_b, new_b, new_b};
    for (int i = 0; i < 4; ++i)
        if (overlaps(k_out, out_b, srcs[i], src_b[i]) || overlaps(v_out, out_b, srcs[i], src_b[i]))
            return H2O_ERR_INVALID_ARG;
    if (overlaps(k_out, out_b, v_out, out_b)) return H2O_ERR_INVALID_ARG;
    hipError_t e = h2o::launch_kv_compact((int)BH, s->head_dim, s->cache_len, s->chunk_len,
                                          budget, out_len, k_cache, v_cache, pos, k_new, v_new,
                                          wsum, keep_idx, p0, k_out, v_out, pos_out, scores_out,
                                          (hipStream_t)stream);
    if (e == hipSuccess && sync_debug()) e = hipStreamSynchronize((hipStream_t)stream);
    return from_hip(e);
}

}  // extern "C"

namespace {

h2o::BwdGeom bwd_geom(const h2o_shape_t* s) {
    h2o::BwdGeom g;
    g.B = s->batch;
    g.Hq = s->n_q_heads;
    g.Hkv = s->n_kv_heads;
    g.G = g.Hq / g.Hkv;
    g.D = s->head_dim;
    g.C = s->cache_len;
    g.S = s->chunk_len;
    g.n = s->n_valid;
    g.R = g.G * g.S;
    g.tau = s->scale > 0.f ? s->scale : 1.0f / sqrtf((float)g.D);
    g.c = g.tau * h2o::kLog2e;
    return g;
}

}  // namespace

extern "C" {

size_t h2o_attn_bwd_workspace_size(const h2o_shape_t* s) {
    if (check_shape(s) != H2O_OK) return 0;
    return (h2o::bwd_workspace_bytes(bwd_geom(s)) + 255) & ~(size_t)255;
}

h2o_status_t h2o_attn_chunk_bwd(const h2o_shape_t* s, const uint16_t* q,
                                const uint16_t* k_cache, const uint16_t* v_cache,
                                const uint16_t* k_new, const uint16_t* v_new,
                                const float* out, const float* lse, const uint16_t* dout,
                                float* dq, float* dk_cache, float* dv_cache, float* dk_new,
                                float* dv_new, void* ws, size_t ws_bytes, void* stream) {
    h2o_status_t st = check_shape(s);
    if (st != H2O_OK) return st;
    const void* ptrs[] = {q, k_cache, v_cache, k_new, v_new, out, lse, dout,
                          dq, dk_cache, dv_cache, dk_new, dv_new};
    for (const void* p : ptrs)
        if (!p || !aligned16(p)) return H2O_ERR_INVALID_ARG;
    const h2o::BwdGeom g = bwd_geom(s);
    const size_t need = (h2o::bwd_workspace_bytes(g) + 255) & ~(size_t)255;
    if (!ws || ((uintptr_t)ws & 255u) || ws_bytes < need) return H2O_ERR_WORKSPACE;
    return from_hip(h2o::launch_attention_bwd(g, q, k_cache, v_cache, k_new, v_new, out, lse,
                                              dout, dq, dk_cache, dv_cache, dk_new, dv_new, ws,
                                              (hipStream_t)stream, sync_debug(), timing_slot()));
}

h2o_status_t h2o_timing_start(int32_t max_calls) {
    if (max_calls < 1 || max_calls > (1 << 20) || g_timing.on) return H2O_ERR_INVALID_ARG;
    g_timing.ev.assign((size_t)5 * max_calls, nullptr);
    for (auto& e : g_timing.ev) {
        // timing only: no system-scope fence (cache write-back and
        // invalidation) when the event is recorded between the kernels
        if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) {
            for (auto& x : g_timing.ev)
                if (x) (void)hipEventDestroy(x);
            g_timing.ev.clear();
            return H2O_ERR_HIP;
        }
    }
    g_timing.max_calls = max_calls;
    g_timing.used = 0;
    g_timing.on = true;
    return H2O_OK;
}

h2o_status_t h2o_timing_stop(double* ms, int32_t* calls) {
    if (!g_timing.on || !ms || !calls) return H2O_ERR_INVALID_ARG;
    h2o_status_t st = H2O_OK;
    for (int k = 0; k < 4; ++k) ms[k] = 0.0;
    // the events carry no memory fence: wait for the device before reading them
    if (g_timing.used > 0 && hipDeviceSynchronize() != hipSuccess) st = H2O_ERR_HIP;
    for (int c = 0; c < g_timing.used && st == H2O_OK; ++c) {
        for (int k = 0; k < 4; ++k) {
            float t = 0.f;
            if (hipEventElapsedTime(&t, g_timing.ev[(size_t)5 * c + k],
                                    g_timing.ev[(size_t)5 * c + k + 1]) != hipSuccess) {
                st = H2O_ERR_HIP;
                break;
            }
            ms[k] += t;
        }
    }
    *calls = g_timing.used;
    for (auto& e : g_timing.ev) (void)hipEventDestroy(e);
    g_timing.ev.clear();
    g_timing.on = false;
    g_timing.used = 0;
    return st;
}

const char* h2o_status_string(h2o_status_t st) {
    switch (st) {
        case H2O_OK: return "ok";
        case H2O_ERR_INVALID_ARG: return "invalid argument";
        case H2O_ERR_UNSUPPORTED: return "unsupported shape";
        case H2O_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case H2O_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

}  // extern "C"
