// Attention of a query chunk over (valid cache slots) + (causal chunk), with
// the summed attention weights per key, for gfx950.
//
// Method: "Learning how to Forget: Fine-tuning for Long-Context Sparse
// Attention" -- Chinese translation page, §1 contributions (an SDPA kernel
// that returns summed attention weights) and §2 (H2O-like summed attention
// weights; grouped query heads; the few-queries-many-keys regime).
//
// The column sums W_j = sum_i exp(s_ij - L_i) need every row's final
// log-sum-exp L_i before any column can be summed, so the work runs in two
// passes over the keys:
//
//   pass 1 (attn_fwd_kernel)    S^T = K Q^T on MFMA, online softmax in base 2,
//                               O^T += V^T P^T on MFMA.  Writes per-split
//                               partial (O, m, l).  In the S^T orientation a
//                               lane owns one query row and 16 keys, so the
//                               row max / row sum stay in-lane and P^T feeds
//                               the PV MFMA straight from the accumulators.
//   combine                     merges the key splits: O, L (natural log for
//                               the caller, base 2 for pass 2).
//   pass 2 (attn_colsum_kernel) S = Q K^T on MFMA (the other orientation: a
//                               lane owns one key and 16 query rows), so the
//                               column sums of P = exp2(S*c - L2) reduce
//                               in-lane, then across the two wave halves, then
//                               across the 4 waves through LDS in a fixed
//                               order.  Writes one partial row of column sums
//                               per 128-row tile.
//   wsum reduce                 sums the row-tile partials in tile order.
//
// Rows of a (b, kv head) pack the G query heads of its group: row r is query
// i = r / G of head h*G + r % G, so one K/V tile read serves the whole group.
// Every reduction has a fixed order, so results are bit-reproducible.
#include "h2o_device.h"
#include "h2o_launch.h"

#include <math.h>

namespace h2o {
namespace {

constexpr int KT = kKeyTile;
constexpr int KPAD = 8;   // bf16 pad per K row in LDS (bank spread)
constexpr int VPAD = 8;   // bf16 pad per V^T row in LDS

// Key tiles seen by one row tile: cache tiles [0, n_ct), then the chunk tiles
// up to the last query of the row tile (causal).
struct TileRange {
    int n_ct, total;
};

__device__ __forceinline__ TileRange tile_range(const AttnGeom& g, int qt) {
    TileRange t;
    t.n_ct = (g.n + KT - 1) / KT;
    const int r_last = min((qt + 1) * kRowsPerBlock, g.R) - 1;
    const int i_max = r_last / g.G;
    t.total = t.n_ct + i_max / KT + 1;
    return t;
}

// Cooperative copy of a KT x D bf16 key tile into LDS (rows >= lim -> 0).
template <int D>
__device__ __forceinline__ void load_k_tile(uint16_t (*Ks)[D + KPAD],
                                            const uint16_t* __restrict__ base,
                                            int key0, int lim, int tid) {
    constexpr int CPR = D / 8;  // 16-byte chunks per row
#pragma unroll
    for (int c = tid; c < KT * CPR; c += kWaves * 64) {
        const int kr = c / CPR, dc = c % CPR;
        const int key = key0 + kr;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (key < lim) v = *(const u32x4*)(base + (size_t)key * D + dc * 8);
        *(u32x4*)&Ks[kr][dc * 8] = v;
    }
}

// Cooperative transposed copy of a KT x D bf16 value tile: Vt[d][key].
// Each unit moves 4 keys x 8 dims with 4 16-byte loads and 8 8-byte stores.
template <int D>
__device__ __forceinline__ void load_vt_tile(uint16_t (*Vt)[KT + VPAD],
                                             const uint16_t* __restrict__ base,
                                             int key0, int lim, int tid) {
    constexpr int UNITS = (KT / 4) * (D / 8);
#pragma unroll
    for (int u = tid; u < UNITS; u += kWaves * 64) {
        const int kg = u % (KT / 4), dg = u / (KT / 4);
        u32x4 r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int key = key0 + 4 * kg + e;
            r[e] = (key < lim) ? *(const u32x4*)(base + (size_t)key * D + dg * 8)
                               : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) {   // dword w holds dims 2w, 2w+1
            u32x2 even = {pack_lo(r[0][w], r[1][w]), pack_lo(r[2][w], r[3][w])};
            u32x2 odd = {pack_hi(r[0][w], r[1][w]), pack_hi(r[2][w], r[3][w])};
            *(u32x2*)&Vt[dg * 8 + 2 * w][4 * kg] = even;
            *(u32x2*)&Vt[dg * 8 + 2 * w + 1][4 * kg] = odd;
        }
    }
}

// ---------------------------------------------------------------------------
// pass 1: partial (O, m, l) per key split
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(
    const AttnGeom g, const int nsplit, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn,
    float* __restrict__ o_part, float* __restrict__ ml_part) {
    __shared__ __attribute__((aligned(16))) uint16_t Ks[KT][D + KPAD];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[D][KT + VPAD];

    const int qt = blockIdx.x, bh = blockIdx.y, split = blockIdx.z;
    const int BH = g.B * g.Hkv;
    const int b = bh / g.Hkv, h = bh % g.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, l32 = lane & 31;

    // this lane's query row (column of S^T)
    const int r = qt * kRowsPerBlock + wave * kRowsPerWave + l32;
    const bool row_ok = r < g.R;
    const int qi = r / g.G;
    bf16x8 qf[D / 16];
    {
        const uint16_t* qrow =
            q + (((size_t)b * g.Hq + (size_t)h * g.G + (r % g.G)) * g.S + qi) * D;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (row_ok) v = *(const u32x4*)(qrow + ks * 16 + half * 8);
            qf[ks] = as_bf16x8(v);
        }
    }

    const TileRange tr = tile_range(g, qt);
    const int t_begin = (int)((long)split * tr.total / nsplit);
    const int t_end = (int)((long)(split + 1) * tr.total / nsplit);

    const uint16_t* kc_bh = kc + (size_t)bh * g.C * D;
    const uint16_t* vc_bh = vc + (size_t)bh * g.C * D;
    const uint16_t* kn_bh = kn + (size_t)bh * g.S * D;
    const uint16_t* vn_bh = vn + (size_t)bh * g.S * D;

    float m_ref = -INFINITY;   // reference max (base 2), shared by both halves
    float l_acc = 0.f;         // this lane's partial row sum
    f32x16 o_acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) o_acc[db][v] = 0.f;

    for (int t = t_begin; t < t_end; ++t) {
        const bool chunk = t >= tr.n_ct;
        const int key0 = chunk ? (t - tr.n_ct) * KT : t * KT;
        const int lim = chunk ? g.S : g.n;
        __syncthreads();
        load_k_tile<D>(Ks, chunk ? kn_bh : kc_bh, key0, lim, tid);
        load_vt_tile<D>(Vt, chunk ? vn_bh : vc_bh, key0, lim, tid);
        __syncthreads();

        // S^T block: 32 keys x 32 rows per key block
        f32x16 s[KT / 32];
#pragma unroll
        for (int kb = 0; kb < KT / 32; ++kb) {
#pragma unroll
            for (int v = 0; v < 16; ++v) s[kb][v] = 0.f;
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                const bf16x8 kf =
                    as_bf16x8(*(const u32x4*)&Ks[kb * 32 + l32][ks * 16 + half * 8]);
                s[kb] = mfma32x32x16(kf, qf[ks], s[kb]);
            }
        }

        // scale, mask, tile max
        const bool full = !chunk && (key0 + KT <= g.n);
        float mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KT / 32; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int key = key0 + kb * 32 + acc_row(v, half);
                const bool ok = full || (key < lim && (!chunk || key <= qi));
                const float u = ok ? s[kb][v] * g.c : -INFINITY;
                s[kb][v] = u;
                mt = fmaxf(mt, u);
            }
        mt = fmaxf(mt, xor32(mt));

        // move the reference max only when it grows by more than 2^8, so
        // P = 2^(u - m_ref) stays <= 256 and rescaling is rare
        if (__any(mt > m_ref + 8.f)) {
            const float m_new = fmaxf(m_ref, mt);
            const float m_safe = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = fast_exp2(m_ref - m_safe);
            l_acc *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) o_acc[db][v] *= alpha;
            m_ref = m_new;
        }
        const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;

#pragma unroll
        for (int kb = 0; kb < KT / 32; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float p = fast_exp2(s[kb][v] - m_use);
                l_acc += p;
                s[kb][v] = p;
            }

        // O^T += V^T P^T; k-step (kb, hs) covers keys kb*32 + 16*hs + [0, 16)
        // in the order lane-half h supplies: 8*gg + 4*h + e, gg, e in 0..1, 0..3
#pragma unroll
        for (int kb = 0; kb < KT / 32; ++kb)
#pragma unroll
            for (int hs = 0; hs < 2; ++hs) {
                bf16x8 pf;
#pragma unroll
                for (int gg = 0; gg < 2; ++gg)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        pf[4 * gg + e] = (__bf16)s[kb][4 * (2 * hs + gg) + e];
                const int kcol = kb * 32 + 16 * hs + 4 * half;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const u32x2 lo = *(const u32x2*)&Vt[db * 32 + l32][kcol];
                    const u32x2 hi = *(const u32x2*)&Vt[db * 32 + l32][kcol + 8];
                    const u32x4 vv = {lo[0], lo[1], hi[0], hi[1]};
                    o_acc[db] = mfma32x32x16(as_bf16x8(vv), pf, o_acc[db]);
                }
            }
    }

    l_acc += xor32(l_acc);
    if (row_ok) {
        const size_t prow = ((size_t)split * BH + bh) * g.rows_pad + r;
        if (half == 0) {
            ml_part[prow * 2 + 0] = m_ref;
            ml_part[prow * 2 + 1] = l_acc;
        }
        float* orow = o_part + prow * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const f32x4 v4 = {o_acc[db][4 * gq + 0], o_acc[db][4 * gq + 1],
                                  o_acc[db][4 * gq + 2], o_acc[db][4 * gq + 3]};
                *(f32x4*)(orow + db * 32 + 8 * gq + 4 * half) = v4;
            }
    }
}

// ---------------------------------------------------------------------------
// combine the key splits: O (normalised), natural LSE, base-2 L for pass 2
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(
    const AttnGeom g, const int nsplit, const float* __restrict__ o_part,
    const float* __restrict__ ml_part, float* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ l2) {
    constexpr int CH = D / 4;
    const int BH = g.B * g.Hkv;
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long total = (long)BH * g.rows_pad * CH;
    if (idx >= total) return;
    const int dc = (int)(idx % CH);
    const long rr = idx / CH;
    const int r = (int)(rr % g.rows_pad);
    const int bh = (int)(rr / g.rows_pad);
    if (r >= g.R) {   // padding rows: weight 0 in pass 2
        if (dc == 0) l2[(size_t)bh * g.rows_pad + r] = INFINITY;
        return;
    }
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s)
        M = fmaxf(M, ml_part[(((size_t)s * BH + bh) * g.rows_pad + r) * 2]);
    float L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < nsplit; ++s) {
        const size_t prow = ((size_t)s * BH + bh) * g.rows_pad + r;
        const float w = fast_exp2(ml_part[prow * 2] - M);
        L += w * ml_part[prow * 2 + 1];
        const f32x4 o = *(const f32x4*)(o_part + prow * D + dc * 4);
        acc += w * o;
    }
    const float inv = 1.0f / L;
    const int b = bh / g.Hkv, h = bh % g.Hkv;
    const int i = r / g.G, a = h * g.G + r % g.G;
    const size_t orow = ((size_t)b * g.Hq + a) * g.S + i;
    *(f32x4*)(out + orow * D + dc * 4) = acc * inv;
    if (dc == 0) {
        const float L2 = M + fast_log2(L);
        l2[(size_t)bh * g.rows_pad + r] = L2;
        if (lse) lse[orow] = L2 * kLn2;
    }
}

// ---------------------------------------------------------------------------
// pass 2: column sums of P per row tile
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void attn_colsum_kernel(
    const AttnGeom g, const int nsplit, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ kn,
    const float* __restrict__ l2, float* __restrict__ wpart) {
    __shared__ __attribute__((aligned(16))) uint16_t Ks[KT][D + KPAD];
    __shared__ float colp[kWaves][KT];

    const int qt = blockIdx.x, bh = blockIdx.y, split = blockIdx.z;
    const int BH = g.B * g.Hkv;
    const int b = bh / g.Hkv, h = bh % g.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, l32 = lane & 31;
    const int W = g.C + g.S;

    const int rbase = qt * kRowsPerBlock + wave * kRowsPerWave;
    bf16x8 qf[D / 16];
    {
        const int r = rbase + l32;
        const bool row_ok = r < g.R;
        const uint16_t* qrow =
            q + (((size_t)b * g.Hq + (size_t)h * g.G + (r % g.G)) * g.S + r / g.G) * D;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (row_ok) v = *(const u32x4*)(qrow + ks * 16 + half * 8);
            qf[ks] = as_bf16x8(v);
        }
    }
    // rows held by this lane in the S accumulator, their base-2 LSE and query
    float l2v[16];
    int qiv[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int rr = rbase + acc_row(v, half);
        l2v[v] = l2[(size_t)bh * g.rows_pad + rr];
        qiv[v] = rr / g.G;
    }

    const TileRange tr = tile_range(g, qt);
    const int t_begin = (int)((long)split * tr.total / nsplit);
    const int t_end = (int)((long)(split + 1) * tr.total / nsplit);
    const uint16_t* kc_bh = kc + (size_t)bh * g.C * D;
    const uint16_t* kn_bh = kn + (size_t)bh * g.S * D;
    float* wrow = wpart + ((size_t)qt * BH + bh) * W;

    for (int t = t_begin; t < t_end; ++t) {
        const bool chunk = t >= tr.n_ct;
        const int key0 = chunk ? (t - tr.n_ct) * KT : t * KT;
        const int lim = chunk ? g.S : g.n;
        __syncthreads();
        load_k_tile<D>(Ks, chunk ? kn_bh : kc_bh, key0, lim, tid);
        __syncthreads();

#pragma unroll
        for (int kb = 0; kb < KT / 32; ++kb) {
            f32x16 s;
#pragma unroll
            for (int v = 0; v < 16; ++v) s[v] = 0.f;
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                const bf16x8 kf =
                    as_bf16x8(*(const u32x4*)&Ks[kb * 32 + l32][ks * 16 + half * 8]);
                s = mfma32x32x16(qf[ks], kf, s);
            }
            const int key = key0 + kb * 32 + l32;
            float col = 0.f;
            if (!chunk) {
#pragma unroll
                for (int v = 0; v < 16; ++v) col += fast_exp2(s[v] * g.c - l2v[v]);
                col = (key < lim) ? col : 0.f;
            } else {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const float p = fast_exp2(s[v] * g.c - l2v[v]);
                    col += (key < lim && key <= qiv[v]) ? p : 0.f;
                }
            }
            col += xor32(col);
            if (half == 0) colp[wave][kb * 32 + l32] = col;
        }
        __syncthreads();
        if (tid < KT) {
            const int key = key0 + tid;
            if (key < lim) {
                float tot = colp[0][tid];
#pragma unroll
                for (int w = 1; w < kWaves; ++w) tot += colp[w][tid];
                wrow[chunk ? g.C + key : key] = tot;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// sum the row-tile partials in tile order
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void wsum_reduce_kernel(
    const AttnGeom g, const float* __restrict__ wpart, float* __restrict__ wsum) {
    const int BH = g.B * g.Hkv;
    const int W = g.C + g.S;
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)BH * W) return;
    const int j = (int)(idx % W);
    const int bh = (int)(idx / W);
    float s = 0.f;
    if (j < g.n) {
        for (int qt = 0; qt < g.n_qt; ++qt) s += wpart[((size_t)qt * BH + bh) * W + j];
    } else if (j >= g.C) {
        const int t = j - g.C;
        for (int qt = 0; qt < g.n_qt; ++qt) {
            const int i_hi = (min((qt + 1) * kRowsPerBlock, g.R) - 1) / g.G;
            if (i_hi >= t) s += wpart[((size_t)qt * BH + bh) * W + j];
        }
    }
    wsum[idx] = s;
}

int pick_split(int base_blocks, int max_tiles) {
    const int target = 2 * 256;   // two workgroups per CU on 256 CUs
    int want = (target + base_blocks - 1) / base_blocks;
    int cap = max_tiles / 4;
    if (cap < 1) cap = 1;
    if (want > cap) want = cap;
    return want < 1 ? 1 : want;
}

template <int D>
hipError_t launch_attention_d(const AttnPlan& pl, const uint16_t* q,
                              const uint16_t* kc, const uint16_t* vc,
                              const uint16_t* kn, const uint16_t* vn, float* out,
                              float* lse, float* wsum, void* ws,
                              hipStream_t stream, bool sync_debug, hipEvent_t* ev) {
    const AttnGeom& g = pl.g;
    char* w = (char*)ws;
    float* o_part = (float*)(w + pl.off_o);
    float* ml_part = (float*)(w + pl.off_ml);
    float* l2 = (float*)(w + pl.off_l2);
    float* wpart = (float*)(w + pl.off_wp);
    const int BH = g.B * g.Hkv;
    hipError_t err;
#define H2O_CHECK()                                              \
    do {                                                         \
        err = hipGetLastError();                                 \
        if (err != hipSuccess) return err;                       \
        if (sync_debug) {                                        \
            err = hipStreamSynchronize(stream);                  \
            if (err != hipSuccess) return err;                   \
        }                                                        \
    } while (0)

    if (ev) hipEventRecord(ev[0], stream);
    hipLaunchKernelGGL(attn_fwd_kernel<D>, dim3(g.n_qt, BH, pl.split1), dim3(256), 0,
                       stream, g, pl.split1, q, kc, vc, kn, vn, o_part, ml_part);
    H2O_CHECK();
    if (ev) hipEventRecord(ev[1], stream);
    {
        const long total = (long)BH * g.rows_pad * (D / 4);
        hipLaunchKernelGGL(attn_combine_kernel<D>, dim3((unsigned)((total + 255) / 256)),
                           dim3(256), 0, stream, g, pl.split1, o_part, ml_part, out,
                           lse, l2);
        H2O_CHECK();
    }
    if (ev) hipEventRecord(ev[2], stream);
    hipLaunchKernelGGL(attn_colsum_kernel<D>, dim3(g.n_qt, BH, pl.split2), dim3(256), 0,
                       stream, g, pl.split2, q, kc, kn, l2, wpart);
    H2O_CHECK();
    if (ev) hipEventRecord(ev[3], stream);
    {
        const long total = (long)BH * (g.C + g.S);
        hipLaunchKernelGGL(wsum_reduce_kernel, dim3((unsigned)((total + 255) / 256)),
                           dim3(256), 0, stream, g, wpart, wsum);
        H2O_CHECK();
    }
    if (ev) hipEventRecord(ev[4], stream);
#undef H2O_CHECK
    return hipSuccess;
}

}  // namespace

bool make_attn_plan(int B, int Hq, int Hkv, int D, int C, int S, int n, float scale,
                    AttnPlan* pl) {
    AttnGeom& g = pl->g;
    g.B = B; g.Hq = Hq; g.Hkv = Hkv; g.G = Hq / Hkv; g.D = D;
    g.C = C; g.S = S; g.n = n;
    g.R = g.G * S;
    g.n_qt = (g.R + kRowsPerBlock - 1) / kRowsPerBlock;
    g.rows_pad = g.n_qt * kRowsPerBlock;
    const float tau = (scale > 0.f) ? scale : 1.0f / sqrtf((float)D);
    g.c = tau * kLog2e;
    const int BH = B * Hkv;
    const int max_tiles = (C + KT - 1) / KT + (S + KT - 1) / KT;
    pl->split1 = pick_split(g.n_qt * BH, max_tiles);
    pl->split2 = pick_split(g.n_qt * BH, max_tiles);
    auto align = [](size_t x) { return (x + 255) & ~(size_t)255; };
    size_t off = 0;
    pl->off_o = off;
    off = align(off + (size_t)pl->split1 * BH * g.rows_pad * D * sizeof(float));
    pl->off_ml = off;
    off = align(off + (size_t)pl->split1 * BH * g.rows_pad * 2 * sizeof(float));
    pl->off_l2 = off;
    off = align(off + (size_t)BH * g.rows_pad * sizeof(float));
    pl->off_wp = off;
    off = align(off + (size_t)g.n_qt * BH * (C + S) * sizeof(float));
    pl->bytes = off;
    return true;
}

hipError_t launch_attention(const AttnPlan& plan, const uint16_t* q, const uint16_t* kc,
                            const uint16_t* vc, const uint16_t* kn, const uint16_t* vn,
                            float* out, float* lse, float* wsum, void* ws,
                            hipStream_t stream, bool sync_debug, hipEvent_t* ev5) {
    if (plan.g.D == 64)
        return launch_attention_d<64>(plan, q, kc, vc, kn, vn, out, lse, wsum, ws, stream,
                                      sync_debug, ev5);
    return launch_attention_d<128>(plan, q, kc, vc, kn, vn, out, lse, wsum, ws, stream,
                                   sync_debug, ev5);
}

}  // namespace h2o
