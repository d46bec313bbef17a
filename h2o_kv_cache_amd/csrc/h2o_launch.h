// Host-side launchers of the gfx950 kernels (internal to libh2o.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace h2o {

// Tiling shared by the attention kernels.
constexpr int kKeyTile = 64;        // keys per LDS tile
constexpr int kRowBlocks = 1;       // 32-row MFMA blocks per wave
constexpr int kRowsPerWave = 32 * kRowBlocks;   // query rows (head, query) per wave
constexpr int kWaves = 8;           // waves per workgroup (2 per SIMD)
constexpr int kRowsPerBlock = kRowsPerWave * kWaves;

// Rows of a (b, kv head) are r = i * G + g: query i of head h*G + g.
struct AttnGeom {
    int B, Hq, Hkv, G, D, C, S, n;
    int R;          // G * S rows per (b, kv head)
    int n_qt;       // row tiles: ceil(R / kRowsPerBlock)
    int rows_pad;   // n_qt * kRowsPerBlock
    float c;        // logit scale * log2(e)
};

struct AttnPlan {
    AttnGeom g;
    bool small;     // G * S <= 32: one row block, logits stored for the weights
    int split1;     // key splits of pass 1 (log-sum-exp and output)
    int split2;     // key splits of pass 2 (summed weights)
    // off_tail: per (b, kv head) state of the one-token step's tail (the
    // running minimum; 16 bytes each)
    size_t off_o, off_ml, off_l2, off_wp, off_tail, bytes;
};

bool make_attn_plan(int B, int Hq, int Hkv, int D, int C, int S, int n,
                    float scale, AttnPlan* plan);

// With non-null `scores` the kernel that writes the summed weights also does
// the score accumulation (scores[j] += wsum[j] for j < n, new_scores[t] =
// wsum[C + t]), with the results of launch_score_accumulate.
hipError_t launch_attention(const AttnPlan& plan, const uint16_t* q,
                            const uint16_t* kc, const uint16_t* vc,
                            const uint16_t* kn, const uint16_t* vn, float* out,
                            float* lse, float* wsum, void* ws,
                            hipStream_t stream, bool sync_debug,
                            hipEvent_t* ev5 /* nullable: 5 timing events */,
                            float* scores = nullptr, float* new_scores = nullptr);

// A whole one-token step on the few-row path (decode_tail_applies): the
// streaming attention pass, one kernel for the split merge, the summed
// weights, the score accumulation and the running minimum, and one for the
// choice and the scatter.  Same results as launch_attention +
// launch_score_accumulate + launch_evict_select + launch_kv_scatter.
bool decode_tail_applies(const AttnPlan& plan);
hipError_t launch_decode_step(const AttnPlan& plan, const uint16_t* q, uint16_t* kc,
                              uint16_t* vc, const uint16_t* kn, const uint16_t* vn, float* out,
                              float* lse, float* wsum, float* scores, float* new_scores,
                              int32_t* evict, int64_t* pos, int64_t p0, void* ws,
                              hipStream_t stream, bool sync_debug,
                              hipEvent_t* ev5 /* nullable: 5 timing events */);

// The same attention over an 8-bit cache: int8 codes [B, Hkv, C, D] and one
// float scale per row [B, Hkv, C] for K and V; same plan and workspace.
hipError_t launch_attention_q8(const AttnPlan& plan, const uint16_t* q, const int8_t* kc,
                               const float* ks, const int8_t* vc, const float* vs,
                               const uint16_t* kn, const uint16_t* vn, float* out, float* lse,
                               float* wsum, void* ws, hipStream_t stream, bool sync_debug,
                               hipEvent_t* ev5 /* nullable: 5 timing events */);

// Backward of the attention (bwd.hip).
struct BwdGeom {
    int B, Hq, Hkv, G, D, C, S, n;
    int R;          // G * S packed rows per (b, kv head)
    float c;        // logit scale * log2(e)
    float tau;      // logit scale
};

size_t bwd_rows_padded(const BwdGeom& g);
size_t bwd_workspace_bytes(const BwdGeom& g);
hipError_t launch_attention_bwd(const BwdGeom& g, const uint16_t* q, const uint16_t* kc,
                                const uint16_t* vc, const uint16_t* kn, const uint16_t* vn,
                                const float* out, const float* lse, const uint16_t* dout,
                                float* dq, float* dkc, float* dvc, float* dkn, float* dvn,
                                void* ws, hipStream_t stream, bool sync_debug,
                                hipEvent_t* ev5 /* nullable: 5 timing events */);

hipError_t launch_score_accumulate(int BH, int C, int S, int n, float* scores,
                                   float* new_scores, const float* wsum,
                                   hipStream_t stream);

hipError_t launch_evict_select(int BH, int C, int S, int n,
                               const float* scores, int32_t* evict_idx,
                               hipStream_t stream);

// launch_evict_select followed by launch_kv_scatter in one kernel (same
// results), for rows whose keys fit in registers and short chunks
// (select_scatter_fuses).
bool select_scatter_fuses(int C, int S, int D);
hipError_t launch_select_scatter(int BH, int D, int C, int S, int n, float* scores,
                                 int32_t* evict_idx, uint16_t* kc, uint16_t* vc, int64_t* pos,
                                 const uint16_t* kn, const uint16_t* vn,
                                 const float* new_scores, int64_t p0, hipStream_t stream);

hipError_t launch_kv_scatter(int BH, int D, int C, int S, uint16_t* kc,
                             uint16_t* vc, float* scores, int64_t* pos,
                             const uint16_t* kn, const uint16_t* vn,
                             const float* new_scores, const int32_t* evict_idx,
                             int64_t p0, hipStream_t stream);

// 8-bit cache rows (one scale per row) from bf16 rows, and the scatter of a
// chunk into an 8-bit cache.
hipError_t launch_quantize_rows(const uint16_t* x, long rows, int D, int8_t* codes,
                                float* scales, hipStream_t stream);
hipError_t launch_kv_scatter_q8(int BH, int D, int C, int S, int8_t* kc, float* ks, int8_t* vc,
                                float* vs, float* scores, int64_t* pos, const uint16_t* kn,
                                const uint16_t* vn, const float* new_scores,
                                const int32_t* evict_idx, int64_t p0, hipStream_t stream);

// SnapKV one-shot choice: keep_idx[bh][0..budget) = the budget valid slots
// (of n) that are not among the n - budget lowest (wsum, slot), ascending.
// wsum rows are C + S floats.
hipError_t launch_snapkv_select(int BH, int C, int S, int n, int budget, const float* wsum,
                                int32_t* keep_idx, hipStream_t stream);

hipError_t launch_kv_compact(int BH, int D, int C, int S, int budget, int out_len,
                             const uint16_t* kc, const uint16_t* vc, const int64_t* pos,
                             const uint16_t* kn, const uint16_t* vn, const float* wsum,
                             const int32_t* keep_idx, int64_t p0, uint16_t* ko, uint16_t* vo,
                             int64_t* pos_out, float* scores_out, hipStream_t stream);

}  // namespace h2o
