/*
 * h2o.h -- C ABI of libh2o.so: one chunked step of Heavy-Hitter Oracle (H2O)
 * sparse attention over a fixed-size KV cache, for AMD Instinct MI355X
 * (gfx950).
 *
 * The method: "Learning how to Forget: Fine-tuning for Long-Context Sparse
 * Attention" (arXiv 2608.19920).  Its Chinese translation page, §1, keeps K/V
 * in a fixed number of cache slots and evicts slots by a policy once the cache
 * is full; §1 (contributions) gives H2O an attention kernel that also returns
 * the summed attention weights; §2 describes those summed weights as the
 * H2O-style score.  The Korean summary page's glossary describes H2O as
 * scoring entries by how often and how strongly they were attended to and
 * evicting the low scorers; its Table 1 / Table 5 captions process sequences
 * in chunks of S tokens.
 *
 * A step, for every (batch b, KV head h), with G = n_q_heads / n_kv_heads
 * query heads per KV head (query head a reads KV head a / G):
 *   1. h2o_attn_chunk       attention of the S chunk queries over the valid
 *                           cache slots [0, n_valid) plus the chunk keys t <= i
 *                           (causal inside the chunk); returns the output, the
 *                           log-sum-exp and the summed attention weights.
 *   2. h2o_score_accumulate scores[j] += wsum[j] for valid slots; the chunk
 *                           tokens' starting scores are their own columns.
 *   3. h2o_evict_select     the S slots to overwrite: empty slots first (slot
 *                           order), then the lowest (score, slot) valid slots;
 *                           listed in increasing slot order.
 *   4. kv_scatter           chunk token t -> slot evict_idx[t]: K, V, score
 *                           and absolute position.
 * The caller advances n_valid to min(cache_len, n_valid + chunk_len) after the
 * step.  All four calls use the same h2o_shape_t (same n_valid).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers to caller-owned memory, dense
 *     and row-major in the layouts given below, 16-byte aligned.  "bf16" is
 *     the 16-bit bfloat16 bit pattern (uint16_t).
 *   - Nothing allocates or frees memory and nothing synchronises: every call
 *     only enqueues kernels on `stream` (a hipStream_t; NULL = the legacy
 *     default stream) and returns.  The calls can be captured in a HIP graph.
 *   - Argument errors are found on the host before anything is enqueued; the
 *     call then returns a non-zero status and touches no buffer.
 *     H2O_ERR_HIP means a launch failed (hipGetLastError after the launch).
 *     Faults inside kernels surface at the caller's next synchronisation.
 *   - Supported: head_dim in {64, 128}; 1 <= chunk_len <= cache_len <= 2^20;
 *     0 <= n_valid <= cache_len; n_q_heads a multiple of n_kv_heads.
 *   - Calls are asynchronous and stream-ordered; two calls that share buffers
 *     must be ordered by the caller (same stream or events).
 */
#ifndef H2O_H
#define H2O_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    H2O_OK = 0,
    H2O_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, bad sizes        */
    H2O_ERR_UNSUPPORTED = 2,   /* valid but unsupported (e.g. head_dim 96)  */
    H2O_ERR_WORKSPACE = 3,     /* workspace missing or smaller than needed  */
    H2O_ERR_HIP = 4            /* a HIP launch failed                        */
} h2o_status_t;

typedef struct {
    int32_t batch;       /* B  >= 1                                        */
    int32_t n_q_heads;   /* Hq >= 1, multiple of n_kv_heads                */
    int32_t n_kv_heads;  /* Hkv >= 1                                       */
    int32_t head_dim;    /* D in {64, 128}                                 */
    int32_t cache_len;   /* C  >= 1: slots per (b, kv head)                */
    int32_t chunk_len;   /* S in [1, C]: tokens in this chunk              */
    int32_t n_valid;     /* n in [0, C]: filled slots before the step      */
    float   scale;       /* logit scale; <= 0 selects 1/sqrt(D)            */
} h2o_shape_t;

/* Bytes of device workspace h2o_attn_chunk needs for this shape.  Depends on
 * (B, Hq, Hkv, D, C, S) only, not on n_valid, so one allocation serves every
 * step of a run.  Returns 0 for an invalid shape. */
size_t h2o_workspace_size(const h2o_shape_t* shape);

/* Step 1 -- attention of the chunk plus summed attention weights.
 * ([LtF] Chinese page §1 contributions: an SDPA kernel that returns the summed
 * attention weights; §2: FlashInfer's few-queries-many-keys regime.)
 *   q        [B, Hq, S, D]   bf16  chunk queries
 *   k_cache  [B, Hkv, C, D]  bf16  cache keys; slots >= n_valid are ignored
 *   v_cache  [B, Hkv, C, D]  bf16  cache values
 *   k_new    [B, Hkv, S, D]  bf16  chunk keys
 *   v_new    [B, Hkv, S, D]  bf16  chunk values
 *   out      [B, Hq, S, D]   fp32  softmax-weighted values (written)
 *   lse      [B, Hq, S]      fp32  natural log-sum-exp of each query's scaled
 *                                  logits (written; may be NULL)
 *   wsum     [B, Hkv, C + S] fp32  summed weights (written): column j < n is
 *                                  cache slot j summed over the G query heads
 *                                  and S queries; n <= j < C is 0; column
 *                                  C + t is chunk token t
 *   ws, ws_bytes                   device workspace of at least
 *                                  h2o_workspace_size(shape) bytes, 256-byte
 *                                  aligned; its contents are scratch.
 * Logits are scale * <q, k>; visible keys of query i are the n cache slots and
 * chunk tokens t <= i.  Reductions run in a fixed order: repeated calls give
 * bit-identical results. */
h2o_status_t h2o_attn_chunk(const h2o_shape_t* shape,
                            const uint16_t* q, const uint16_t* k_cache,
                            const uint16_t* v_cache, const uint16_t* k_new,
                            const uint16_t* v_new, float* out, float* lse,
                            float* wsum, void* ws, size_t ws_bytes,
                            void* stream);

/* Step 2 -- score accumulation.
 * ([LtF] Korean page glossary: H2O scores entries by accumulated attention;
 * Chinese page §2: summed attention weights as the score.)
 *   scores     [B, Hkv, C]     fp32  in/out: scores[j] += wsum[j] for j < n;
 *                                    slots >= n are left untouched
 *   new_scores [B, Hkv, S]     fp32  out: new_scores[t] = wsum[C + t]
 *   wsum       [B, Hkv, C + S] fp32  in: from h2o_attn_chunk */
h2o_status_t h2o_score_accumulate(const h2o_shape_t* shape, float* scores,
                                  float* new_scores, const float* wsum,
                                  void* stream);

/* Step 3 -- choice of the S slots to overwrite, per (b, kv head).
 * ([LtF] Chinese page §1: evict by policy only when the cache is full;
 * Korean page glossary: the low scorers are evicted.)
 *   scores    [B, Hkv, C] fp32   in (after h2o_score_accumulate)
 *   evict_idx [B, Hkv, S] int32  out: slot indices in increasing order.
 * Empty slots n..C-1 are taken first; the rest are the valid slots with the
 * smallest (score, slot) pairs -- equal scores go to the lower slot, -0.0
 * equals +0.0 and NaN ranks above +inf.  While n + S <= C this is simply
 * n, n+1, ..., n+S-1. */
h2o_status_t h2o_evict_select(const h2o_shape_t* shape, const float* scores,
                              int32_t* evict_idx, void* stream);

/* Step 4 -- write the chunk into the chosen slots (in place).
 * ([LtF] Chinese page §1: the chunk's K/V replace the evicted slots.)
 *   k_cache, v_cache [B, Hkv, C, D] bf16   in/out
 *   scores           [B, Hkv, C]    fp32   in/out: scores[e_t] = new_scores[t]
 *   pos              [B, Hkv, C]    int64  in/out: pos[e_t] = p0 + t (may be
 *                                          NULL: positions not tracked)
 *   k_new, v_new     [B, Hkv, S, D] bf16   chunk rows
 *   new_scores       [B, Hkv, S]    fp32   from h2o_score_accumulate
 *   evict_idx        [B, Hkv, S]    int32  distinct slots in [0, C), from
 *                                          h2o_evict_select; an index outside
 *                                          [0, C) writes nothing for its token
 *   p0               absolute position of the chunk's first token */
h2o_status_t kv_scatter(const h2o_shape_t* shape, uint16_t* k_cache,
                        uint16_t* v_cache, float* scores, int64_t* pos,
                        const uint16_t* k_new, const uint16_t* v_new,
                        const float* new_scores, const int32_t* evict_idx,
                        int64_t p0, void* stream);

/* One whole step -- h2o_attn_chunk, h2o_score_accumulate, h2o_evict_select
 * and kv_scatter in that order, on one stream, with the same arguments and
 * results (the choice is written to evict_idx; scores ends as after
 * kv_scatter).  For one-token chunks (chunk_len == 1) with at most 32 query
 * heads per KV head -- the decode step, the few-queries-many-keys regime of
 * [LtF] Chinese page §2 -- everything after the streaming attention pass
 * (merging the key splits, the summed weights, the score update, the
 * lowest (score, slot) choice and the one-row scatter) runs as a single
 * kernel per (b, KV head) instead of five launches; its results are those of
 * the separate calls bit for bit.
 *   arguments as for the four calls; lse and pos may be NULL;
 *   ws, ws_bytes: at least h2o_workspace_size(shape) bytes, 256-byte aligned. */
h2o_status_t h2o_step(const h2o_shape_t* shape, const uint16_t* q, uint16_t* k_cache,
                      uint16_t* v_cache, const uint16_t* k_new, const uint16_t* v_new,
                      float* out, float* lse, float* wsum, float* scores,
                      float* new_scores, int32_t* evict_idx, int64_t* pos, int64_t p0,
                      void* ws, size_t ws_bytes, void* stream);

/* 8-bit KV cache (Q-Hitter-like H2O).  ([LtF] Chinese page §2: cache
 * buffers can be quantised to 8 bits or fewer; Q-Hitter combines H2O with
 * such quantisation.)  Reading used here: every cached (token, KV head) row
 * is stored as D int8 codes plus one fp32 scale, scale = amax / 127 (amax =
 * the row's largest |x|), code = round-half-even(x / scale), both correctly
 * rounded fp32 divisions, |code| <= 127; a row of zeros has scale 0.  Rows
 * must be finite.  Attention reads the cache rows as code * scale; the
 * chunk's own K/V are used unquantised in their step and quantised when
 * written into the cache.  Score accumulation and the slot choice are the
 * unchanged calls above.  The int8 cache halves the bytes attention reads
 * from HBM per cached key (2*(D + 4) instead of 4*D).
 *
 * h2o_attn_chunk_q8: as h2o_attn_chunk, with the cache given as
 *   k_cache, v_cache [B, Hkv, C, D] int8 codes
 *   k_scale, v_scale [B, Hkv, C]    fp32 per-row scales
 * and the same workspace (h2o_workspace_size).  Inside, a logit of a cache
 * key is (q . codes) * scale * tau with the codes converted exactly to bf16;
 * a value row enters the PV product as bf16(code * scale). */
h2o_status_t h2o_attn_chunk_q8(const h2o_shape_t* shape, const uint16_t* q,
                               const int8_t* k_cache, const float* k_scale,
                               const int8_t* v_cache, const float* v_scale,
                               const uint16_t* k_new, const uint16_t* v_new,
                               float* out, float* lse, float* wsum, void* ws,
                               size_t ws_bytes, void* stream);

/* Step 4 into an 8-bit cache: chunk token t is quantised (as above) and
 * written to slot evict_idx[t] -- codes, scale, score, position; arguments
 * as for kv_scatter with the cache as codes + scales. */
h2o_status_t kv_scatter_q8(const h2o_shape_t* shape, int8_t* k_cache, float* k_scale,
                           int8_t* v_cache, float* v_scale, float* scores,
                           int64_t* pos, const uint16_t* k_new,
                           const uint16_t* v_new, const float* new_scores,
                           const int32_t* evict_idx, int64_t p0, void* stream);

/* Quantise n_rows bf16 rows of head_dim values (x [n_rows, head_dim]) into
 * codes [n_rows, head_dim] int8 and scales [n_rows] fp32, as above: for
 * building an 8-bit cache from bf16 K/V (e.g. after a prefill). */
h2o_status_t h2o_quantize_rows_q8(const uint16_t* x, int64_t n_rows,
                                  int32_t head_dim, int8_t* codes,
                                  float* scales, void* stream);

/* SnapKV-style one-shot choice ([LtF] Chinese page §2: SnapKV scores cache
 * entries with H2O-like summed attention weights but makes the choice at a
 * single point of the generation).  Reading used here: the choice is made
 * once, from the summed weights that h2o_attn_chunk returns for one chunk --
 * the observation window, typically the prompt's last S tokens -- over the
 * n_valid cache slots holding the rest of the prompt.  Of those slots, the
 * n_valid - budget with the lowest (weight, slot) pairs are dropped, in the
 * same order as h2o_evict_select (equal weights drop the lower slot first,
 * -0.0 equals +0.0, NaN ranks above +inf), and the rest are kept.
 *   wsum     [B, Hkv, C + S] fp32  in: from h2o_attn_chunk with this shape
 *   budget   0 <= budget <= n_valid
 *   keep_idx [B, Hkv, budget] int32 out: the kept slots in increasing order
 *            (may be NULL when budget == 0)
 * Any cache_len allowed by the shape; rows are read from memory once per
 * radix pass (no register limit on their length). */
h2o_status_t h2o_snapkv_select(const h2o_shape_t* shape, const float* wsum,
                               int32_t budget, int32_t* keep_idx, void* stream);

/* The cache after a SnapKV choice, written to a separate output cache of
 * out_len slots (out_len >= budget + S):
 *   slot i < budget        <- input slot keep_idx[i]: K, V row, position
 *                             pos[keep_idx[i]], score wsum[keep_idx[i]]
 *   slot budget + t (t < S) <- chunk token t: k_new/v_new row, position
 *                             p0 + t, score wsum[C + t] (its own column)
 *   slots >= budget + S     not written.
 * The caller continues with n_valid = budget + S on the output cache.
 *   k_cache, v_cache [B, Hkv, C, D]       bf16  in (not modified)
 *   pos              [B, Hkv, C]          int64 in (NULL only if pos_out is)
 *   k_new, v_new     [B, Hkv, S, D]       bf16  the observation window
 *   wsum             [B, Hkv, C + S]      fp32  the window's summed weights
 *   keep_idx         [B, Hkv, budget]     int32 from h2o_snapkv_select; an
 *                                         index outside [0, C) leaves its
 *                                         output row unwritten
 *   k_out, v_out     [B, Hkv, out_len, D] bf16  out; must not overlap any
 *                                         input cache or chunk (checked)
 *   pos_out          [B, Hkv, out_len]    int64 out, may be NULL
 *   scores_out       [B, Hkv, out_len]    fp32  out, may be NULL */
h2o_status_t h2o_snapkv_compact(const h2o_shape_t* shape, const uint16_t* k_cache,
                                const uint16_t* v_cache, const int64_t* pos,
                                const uint16_t* k_new, const uint16_t* v_new,
                                const float* wsum, const int32_t* keep_idx,
                                int32_t budget, int32_t out_len, int64_t p0,
                                uint16_t* k_out, uint16_t* v_out, int64_t* pos_out,
                                float* scores_out, void* stream);

/* Backward of step 1 with the slot layout fixed: gradients of `out` of
 * h2o_attn_chunk with respect to q and to the keys and values it attended to.
 * ([LtF] Chinese page abstract and §1: the paper's fine-tuning computes
 * gradients through the sparse attention with the KV cache policy in place;
 * the eviction decisions that produced the slot layout are discrete and are
 * not differentiated.)  With P the forward's normalised weights:
 *   dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D),
 *   dq = scale * dS K,  dk = scale * dS^T q,  dv = P^T dO,
 * the G query heads of a KV head summed into its key and value gradients.
 *   q, k_cache, v_cache, k_new, v_new   as for h2o_attn_chunk (same shape,
 *                                 same n_valid: the forward's inputs)
 *   out      [B, Hq, S, D]   fp32  the forward's output
 *   lse      [B, Hq, S]      fp32  the forward's log-sum-exp (required here)
 *   dout     [B, Hq, S, D]   bf16  upstream gradient of out
 *   dq       [B, Hq, S, D]   fp32  written
 *   dk_cache, dv_cache [B, Hkv, C, D] fp32  written; 0 for slots >= n_valid
 *   dk_new,   dv_new   [B, Hkv, S, D] fp32  written
 *   ws, ws_bytes                   device workspace of at least
 *                                  h2o_attn_bwd_workspace_size(shape) bytes,
 *                                  256-byte aligned; contents are scratch.
 * Every output element is written.  Reductions run in a fixed order:
 * repeated calls give bit-identical results. */
size_t h2o_attn_bwd_workspace_size(const h2o_shape_t* shape);
h2o_status_t h2o_attn_chunk_bwd(const h2o_shape_t* shape, const uint16_t* q,
                                const uint16_t* k_cache, const uint16_t* v_cache,
                                const uint16_t* k_new, const uint16_t* v_new,
                                const float* out, const float* lse,
                                const uint16_t* dout, float* dq, float* dk_cache,
                                float* dv_cache, float* dk_new, float* dv_new,
                                void* ws, size_t ws_bytes, void* stream);

/* Diagnostics: per-kernel timing of h2o_attn_chunk with HIP events.
 * h2o_timing_start(max_calls) creates 5 * max_calls events (call it outside
 * any timed or captured region); until h2o_timing_stop, each h2o_attn_chunk
 * call records an event before its first kernel and after each of its four
 * kernels on its stream (pass 1: output and log-sum-exp; split merge; pass 2:
 * summed-weight partials; partial reduction), for the first max_calls calls.
 * The events are created without a system-scope memory fence (they only
 * time; recording them does not write back or invalidate the caches).
 * h2o_timing_stop(ms, calls) synchronizes the device, writes the
 * summed milliseconds of the four kernels to ms[0..3] and the number of timed
 * calls to *calls, and destroys the events.  h2o_attn_chunk_bwd calls are
 * timed the same way, with ms[0..2] its three kernels (row statistics; key,
 * value gradients; query gradients) and ms[3] = 0.  Not thread-safe; meant
 * for one benchmarking thread. */
h2o_status_t h2o_timing_start(int32_t max_calls);
h2o_status_t h2o_timing_stop(double* ms, int32_t* calls);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): h2o_attn_chunk without a
 * caller workspace.  The kernels' scratch (the key splits' partial outputs
 * and row statistics, the row tiles' partial summed weights or the few-row
 * path's stored logits) lives in a static device array of the library,
 * H2O_STATIC_SCRATCH_BYTES on every GPU the library runs on, held until the
 * process ends.  Nothing is allocated or freed by this call.
 *   Arguments and results: as h2o_attn_chunk, without ws / ws_bytes.
 *   Limit: shapes with h2o_workspace_size(shape) > H2O_STATIC_SCRATCH_BYTES
 *          return H2O_ERR_WORKSPACE before anything is enqueued (the
 *          Qwen3-4B-shaped 64k/128k layers, the 128-token chunks and 16-way
 *          decode at 16384 slots all fit).
 *   The first call on a device looks up that device's copy of the array
 *   (hipGetSymbolAddress, with the device current); make it outside any
 *   graph capture.  Every call on a GPU uses that GPU's one array and
 *   leaves its contents behind: calls that overlap on one GPU (different
 *   streams, or host threads without ordering) race and must be ordered by
 *   the caller.  No element of the scratch has to start at zero: every
 *   element a kernel reads was written earlier in the same call. */
#define H2O_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
h2o_status_t h2o_attn_chunk_static(const h2o_shape_t* shape, const uint16_t* q,
                                   const uint16_t* k_cache, const uint16_t* v_cache,
                                   const uint16_t* k_new, const uint16_t* v_new,
                                   float* out, float* lse, float* wsum, void* stream);

/* Static, human-readable name of a status code. */
const char* h2o_status_string(h2o_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* H2O_H */
