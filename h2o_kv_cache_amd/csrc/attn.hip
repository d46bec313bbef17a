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
//   pass 2 (attn_colsum_kernel) S = Q K^T on the 16x16x32 MFMA (the other
//                               orientation: a lane owns one key and 8 query
//                               rows of a 16-key block), so the column sums
//                               of P = exp2(S*c - L2) reduce in-lane, then
//                               across the four 16-lane groups, then across
//                               the 8 waves through LDS in a fixed order.
//                               Writes one partial row of column sums per
//                               256-row tile.
//   wsum reduce                 sums the row-tile partials in tile order.
//
// Rows of a (b, kv head) pack the G query heads of its group: row r is query
// i = r / G of head h*G + r % G, so one K/V tile read serves the whole group.
// Every reduction has a fixed order, so results are bit-reproducible.
#include "h2o_device.h"
#include "h2o_launch.h"
#include "h2o_tiles.h"

#include <math.h>

namespace h2o {
namespace {

constexpr int KT = kKeyTile;
constexpr int RB = kRowBlocks;

// Row stride (floats) of the stored logits of the few-row path: C + S rounded
// up to a multiple of 4, so that a row starts on a 16-byte boundary.
__host__ __device__ inline int logit_stride(const AttnGeom& g) { return (g.C + g.S + 3) & ~3; }
constexpr int NT = kWaves * 64;   // threads per workgroup

// Key tiles seen by one row tile: cache tiles [0, n_ct), then the chunk tiles
// up to the last query of the row tile (causal).
struct TileRange {
    int n_ct, total;
};

template <int KTT = KT>
__device__ __forceinline__ TileRange tile_range(const AttnGeom& g, int qt) {
    TileRange t;
    t.n_ct = (g.n + KTT - 1) / KTT;
    const int r_last = min((qt + 1) * kRowsPerBlock, g.R) - 1;
    const int i_max = r_last / g.G;
    t.total = t.n_ct + i_max / KTT + 1;
    return t;
}

// First tile of key split `sp` of a row tile (sp = nsplit gives tr.total):
// the splits take contiguous ranges of equal estimated cost, a chunk tile
// counting 7/4 of a cache tile (the chunk tiles of a row tile take longer:
// per-workgroup timestamps of pass 1 show the split that holds them ending
// last by about 0.7 cache tiles per chunk tile).
__device__ __forceinline__ int split_tile(const TileRange& tr, int sp, int nsplit) {
    const long cache_cost = 4L * tr.n_ct;
    const long c = (long)sp * (cache_cost + 7L * (tr.total - tr.n_ct)) / nsplit;
    return c <= cache_cost ? (int)(c / 4) : tr.n_ct + (int)((c - cache_cost) / 7);
}

// Q fragments of this lane: row rbase + rb*32 + l32, dims 16*ks + 8*half + [0, 8).
// Serve as the B operand of S^T = K Q^T and the A operand of S = Q K^T.
template <int D>
__device__ __forceinline__ void load_q(bf16x8 (&qf)[RB][D / 16], const uint16_t* __restrict__ q,
                                       const AttnGeom& g, int b, int h, int rbase, int l32,
                                       int half) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int r = rbase + rb * 32 + l32;
        const bool ok = r < g.R;
        const uint16_t* qrow =
            q + (((size_t)b * g.Hq + (size_t)h * g.G + (r % g.G)) * g.S + r / g.G) * D;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (ok) v = *(const u32x4*)(qrow + ks * 16 + half * 8);
            qf[rb][ks] = as_bf16x8(v);
        }
    }
}

// Headroom (base 2) of the fixed per-row reference max in pass 1.
constexpr float kHeadroom = 64.f;
constexpr float kSumLimit = 0x1p64f;   // 2^kHeadroom

template <bool B>
struct TrackC {
    static constexpr bool value = B;
};
template <int N>
struct BufC {
    static constexpr int value = N;
};

// Per (b, kv head) state of the one-token step's tail (decode_tail_kernel,
// decode_scatter_kernel), 16 bytes in the workspace: the running minimum
// (score key << 32 | slot) over the tail's workgroups.  The streaming pass
// (its split-0 workgroup) resets it before the tail runs.
struct TailState {
    unsigned long long min_key;
    unsigned long long pad;
};

__device__ __forceinline__ void tail_state_init(TailState* ts, int bh) {
    if (ts) ts[bh].min_key = ~0ull;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

// One 32-key block (block kb of a KT-key tile) of pass 1 for one wave:
// S^T = K Q^T, online softmax in base 2, O^T += V^T P^T.  MASKED handles the
// last partial cache tile and the causal chunk tiles.  With a non-null
// `lg_row` the base-2 logits of this lane's row are also stored, at logits
// columns col0 + (key - key0).  The block's rows sit at block lkb of the LDS
// tiles (lkb = kb except for per-wave tiles).  KSC: the K tile holds int8
// codes, and logit j is multiplied by the key's scale ksc[lkb*32 + j].
// K8 / V8: K / V come straight from swizzled int8 tiles (k8, v8; V through
// the 8-bit transposed read) and are converted exactly; with V8 the V scale
// of key j (vsc[lkb*32 + j]) multiplies P before its bf16 rounding, and O is
// normalised by the exact row sum (lt_acc = l_acc).
template <int D, bool MASKED, bool KSC = false, bool K8 = false, bool V8 = false,
          bool TRACK = true>
__device__ __forceinline__ void fwd_block(const uint16_t* Ks, const uint16_t* Vs,
                                          const LdsOffsets<D>& off,
                                          const bf16x8 (&qf)[RB][D / 16],
                                          f32x16 (&o_acc)[RB][D / 32], float (&m_ref)[RB],
                                          float (&m_seen)[RB], bool& overflow,
                                          float (&l_acc)[RB], float (&lt_acc)[RB], float c,
                                          int kb, int key0, int lim, bool chunk, int G,
                                          int rbase, int lane, float* lg_row, int col0,
                                          int lkb, const float* ksc = nullptr,
                                          const uint8_t* k8 = nullptr,
                                          const uint8_t* v8 = nullptr,
                                          const float* vsc = nullptr,
                                          float* lg_stage = nullptr) {
    const int l32 = lane & 31, half = lane >> 5;
    {
        f32x16 s[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int v = 0; v < 16; ++v) s[rb][v] = 0.f;
        // K8: the K fragments come straight from a swizzled int8 tile (row
        // lkb*32 + l32, dims 16*ks + 8*half + [0, 8)), converted exactly
        const int krow = lkb * 32 + l32;
        const uint8_t* k8row = K8 ? k8 + krow * D + 8 * half : nullptr;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            bf16x8 kf;
            if constexpr (K8)
                kf = i8x8_to_bf16(*(const uint2*)(k8row + 16 * (ks ^ i8_swz<D>(krow))));
            else
                kf = as_bf16x8(lds_read16(Ks, off.k[ks] + lkb * 64 * D));
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) s[rb] = mfma32x32x16(kf, qf[rb][ks], s[rb]);
        }
        if (KSC) {   // element v is key lkb*32 + 8*(v/4) + 4*half + v%4 of the tile
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 k4 = *(const f32x4*)(ksc + lkb * 32 + 8 * g4 + 4 * half);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) s[rb][4 * g4 + e] *= k4[e];
            }
        }

        // mask (last partial cache tile, chunk tiles), then row max over raw
        // logits (c > 0)
        if (MASKED) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int r = rbase + rb * 32 + l32;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int key = key0 + kb * 32 + acc_row(v, half);
                    const bool ok = key < lim && (!chunk || key * G <= r);
                    s[rb][v] = ok ? s[rb][v] : -INFINITY;
                }
            }
        }
        if (!MASKED && lg_stage) {
            // base-2 logits of the block to the wave's LDS stage [row][32 keys]
            // (rows past R included; the caller copies the real rows out)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4)
                *(f32x4*)(lg_stage + l32 * 32 + 8 * g4 + 4 * half) =
                    f32x4{s[0][4 * g4] * c, s[0][4 * g4 + 1] * c, s[0][4 * g4 + 2] * c,
                          s[0][4 * g4 + 3] * c};
        }
        if (lg_row) {   // base-2 logits of the real keys (few-row path only)
            if constexpr (!MASKED) {
                // keys 8*g4 + 4*half + [0, 4) of the block are contiguous: one
                // 16-byte store each (col0 is a multiple of the tile length
                // and the row stride of the logits a multiple of 4 floats)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4)
                    *(f32x4*)(lg_row + col0 + kb * 32 + 8 * g4 + 4 * half) =
                        f32x4{s[0][4 * g4] * c, s[0][4 * g4 + 1] * c, s[0][4 * g4 + 2] * c,
                              s[0][4 * g4 + 3] * c};
            } else {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int kl = kb * 32 + acc_row(v, half);
                    if (key0 + kl < lim) lg_row[col0 + kl] = s[0][v] * c;
                }
            }
        }
        // TRACK: the reference max of a row is fixed by the first tile in
        // which the row sees a key (O and l are still 0 then, so nothing is
        // rescaled).  Later tiles may exceed it by up to kHeadroom (P <= 2^64,
        // far from fp32 overflow); beyond that the row is flagged and the
        // workgroup redoes its tiles with the exact row max in m_seen.
        // !TRACK: the caller has fixed every row's reference; no tile max is
        // formed (the caller checks the row sums instead).
        if constexpr (TRACK) {
            float mt[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                float mx = s[rb][0];
#pragma unroll
                for (int v = 1; v < 16; ++v) mx = fmaxf(mx, s[rb][v]);
                mx = fmaxf(mx, xor32(mx));
                mt[rb] = mx * c;
            }
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                m_seen[rb] = fmaxf(m_seen[rb], mt[rb]);
                m_ref[rb] = (m_ref[rb] == -INFINITY) ? mt[rb] : m_ref[rb];
                overflow |= mt[rb] > m_ref[rb] + kHeadroom;
            }
        }

        // P = 2^(s*c - m), row sums, P^T fragments in bf16: element v of the
        // accumulator is key 8*(v/4) + 4*half + v%4 of the block, i.e. entry
        // v%8 of k-step v/8.  l_acc sums P exactly (for the log-sum-exp);
        // lt_acc sums the bf16-rounded P that the PV MFMA sees, so that O is
        // normalised by the weights it was built from.
        bf16x8 pf[2][RB];
        float vs16[16];
        if (V8) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 v4 = *(const f32x4*)(vsc + lkb * 32 + 8 * g4 + 4 * half);
#pragma unroll
                for (int e = 0; e < 4; ++e) vs16[4 * g4 + e] = v4[e];
            }
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const float m_use = (!TRACK || m_ref[rb] != -INFINITY) ? m_ref[rb] : 0.f;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float p = fast_exp2(fmaf(s[rb][v], c, -m_use));
                l_acc[rb] += p;
                pf[v >> 3][rb][v & 7] = (__bf16)(V8 ? p * vs16[v] : p);
            }
            if (V8) {
                lt_acc[rb] = l_acc[rb];
            } else {
#pragma unroll
                for (int hs = 0; hs < 2; ++hs)
#pragma unroll
                    for (int e = 0; e < 8; e += 2) {
                        const bf16x2 pair = {pf[hs][rb][e], pf[hs][rb][e + 1]};
                        lt_acc[rb] =
                            __builtin_amdgcn_fdot2_f32_bf16(pair, kOnes2, lt_acc[rb], false);
                    }
            }
        }

        // k-step hs covers keys kb*32 + 16*hs + [0, 16) in the order lane-half
        // h supplies them: 8*gg + 4*h + e
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
            // keys kb*32 + 16*hs + 8*gg + 4*half + [0, 4): rows (kb*32 + 16*hs + 8*gg) below
            const uint32_t row_b = (uint32_t)(lkb * 32 + 16 * hs) * 2 * D;
            // V8: this lane points at key row lkb*32 + 16*hs + 4*half + r8 of
            // the int8 tile (r8 = {0,1,2,3,8,9,10,11}[(lane % 16) / 2]),
            // columns 32*db + 16*((lane / 16) % 2) + 8*(lane % 2) + [0, 8)
            const int j16 = lane & 15, b8 = j16 >> 1;
            const int vrow = lkb * 32 + 16 * hs + 4 * half + (b8 & 3) + 8 * (b8 >> 2);
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                bf16x8 vf;
                if constexpr (V8) {
                    const int c16 = 2 * db + ((lane >> 4) & 1);
                    vf = i8x8_to_bf16(lds_read_tr8(
                        v8 + vrow * D + 16 * (c16 ^ i8_swz_v<D>(vrow)) + 8 * (j16 & 1)));
                } else {
                    const u32x2 lo = lds_read_tr(Vs, off.v[db] + row_b);
                    const u32x2 hi = lds_read_tr(Vs, off.v[db] + row_b + 8 * 2 * D);
                    vf = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
                }
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    o_acc[rb][db] = mfma32x32x16(vf, pf[hs][rb], o_acc[rb][db]);
            }
        }
    }
}

// One KT-key tile of pass 1 for one wave: its 32-key blocks in order.
template <int D, bool MASKED, bool KSC = false, bool TRACK = true>
__device__ __forceinline__ void fwd_tile(const uint16_t* Ks, const uint16_t* Vs,
                                         const LdsOffsets<D>& off,
                                         const bf16x8 (&qf)[RB][D / 16],
                                         f32x16 (&o_acc)[RB][D / 32], float (&m_ref)[RB],
                                         float (&m_seen)[RB], bool& overflow,
                                         float (&l_acc)[RB], float (&lt_acc)[RB], float c,
                                         int key0, int lim, bool chunk, int G, int rbase,
                                         int lane, const float* ksc = nullptr) {
#pragma unroll
    for (int kb = 0; kb < KT / 32; ++kb)
        fwd_block<D, MASKED, KSC, false, false, TRACK>(Ks, Vs, off, qf, o_acc, m_ref, m_seen,
                                                      overflow, l_acc, lt_acc, c, kb, key0, lim,
                                                      chunk, G, rbase, lane, nullptr, 0, kb,
                                                      ksc);
}

// ---------------------------------------------------------------------------
// pass 1: partial (O, m, l) per key split
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(NT, 1) void attn_fwd_kernel(
    const AttnGeom g, const int nsplit, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn,
    float* __restrict__ o_part, float* __restrict__ ml_part) {
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][KT * D];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[2][KT * D];

    int qt, bh, split;
    decode_block(g.n_qt, nsplit, qt, bh, split);
    const int BH = g.B * g.Hkv;
    const int b = bh / g.Hkv, h = bh % g.Hkv;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const int half = lane >> 5, l32 = lane & 31;
    const int rbase = qt * kRowsPerBlock + wave * kRowsPerWave;
    // row blocks of this wave that hold any real row (uniform per wave)
    const int live = min(RB, max(0, (g.R - rbase + 31) / 32));

    bf16x8 qf[RB][D / 16];
    load_q<D>(qf, q, g, b, h, rbase, l32, half);
    const LdsOffsets<D> off(lane);

    const TileRange tr = tile_range(g, qt);
    const int t_begin = split_tile(tr, split, nsplit);
    const int t_end = split_tile(tr, split + 1, nsplit);
    const uint16_t* kc_bh = kc + (size_t)bh * g.C * D;
    const uint16_t* vc_bh = vc + (size_t)bh * g.C * D;
    const uint16_t* kn_bh = kn + (size_t)bh * g.S * D;
    const uint16_t* vn_bh = vn + (size_t)bh * g.S * D;

    float m_ref[RB], m_seen[RB], l_acc[RB], lt_acc[RB];
    f32x16 o_acc[RB][D / 32];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) m_seen[rb] = -INFINITY;

    // tiles whose rows all exist (the full cache tiles) are copied with the
    // scalar-base form and fixed lane offsets; the others clamp their rows
    const TileCopy<D, false> kcopy(wave, lane);
    const TileCopy<D, true> vcopy(wave, lane);
    const int n_full_tiles = g.n / KT;
    auto issue = [&](int t, int buf) {
        if (t < n_full_tiles) {
            kcopy.issue(Ks[buf], kc_bh + (size_t)t * KT * D, wave);
            vcopy.issue(Vs[buf], vc_bh + (size_t)t * KT * D, wave);
            return;
        }
        const bool chunk = t >= tr.n_ct;
        const int key0 = chunk ? (t - tr.n_ct) * KT : t * KT;
        const int lim = chunk ? g.S : g.n;
        issue_tile<D, false>(Ks[buf], chunk ? kn_bh : kc_bh, key0, lim, wave, lane);
        issue_tile<D, true>(Vs[buf], chunk ? vn_bh : vc_bh, key0, lim, wave, lane);
    };

    // Main sweep.  The reference of row r (query i = r / G) is its own
    // base-2 logit against chunk key i, which every row sees: P = 2^(s*c -
    // ref) needs no per-tile max.  A row whose logits in this split exceed
    // the reference by more than kHeadroom makes its sum of P exceed
    // 2^kHeadroom (P >= 0), which sends the workgroup to the tracked sweeps
    // below.  Logits far below the reference underflow to P = 0: their weight
    // relative to the row's own key is below fp32 resolution.
    {
        bool overflow = false;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int r = rbase + rb * 32 + l32;
            const bool ok = r < g.R;
            const uint16_t* kself = kn_bh + (size_t)(ok ? r / g.G : 0) * D + 8 * half;
            float dot = 0.f;
#pragma unroll
            for (int k16 = 0; k16 < D / 16; ++k16) {
                const bf16x8 kv = as_bf16x8(*(const u32x4*)(kself + 16 * k16));
#pragma unroll
                for (int e = 0; e < 8; ++e) dot = fmaf((float)qf[rb][k16][e], (float)kv[e], dot);
            }
            dot += xor32(dot);
            m_ref[rb] = ok ? dot * g.c : 0.f;
            l_acc[rb] = 0.f;
            lt_acc[rb] = 0.f;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) o_acc[rb][db][v] = 0.f;
        }
        if (t_begin < t_end) issue(t_begin, 0);
        wait_tiles();
        __syncthreads();
        const int n_full = g.n / KT;
        const int t_mid = max(t_begin, min(t_end, n_full));
        // unrolled by the two buffers, so that the LDS tile addresses are
        // constants folded into the reads' offsets
        auto full_tile = [&](auto BUFC, int t) {
            constexpr int BUF = decltype(BUFC)::value;
            if (t + 1 < t_end) issue(t + 1, BUF ^ 1);
            if (live > 0)
                fwd_tile<D, false, false, false>(Ks[BUF], Vs[BUF], off, qf, o_acc, m_ref, m_seen,
                                                 overflow, l_acc, lt_acc, g.c, 0, 0, false, 0,
                                                 rbase, lane);
            wait_tiles();
            __syncthreads();
        };
        for (int t = t_begin; t < t_mid; t += 2) {
            full_tile(BufC<0>{}, t);
            if (t + 1 < t_mid) full_tile(BufC<1>{}, t + 1);
        }
        // the rest: the partial cache tile and the chunk tiles; a chunk tile
        // whose keys all exist and precede this wave's first query (query
        // rbase / G) needs no mask, only the tiles on the diagonal do
        const int wave_q0 = rbase / g.G;
        for (int t = t_mid; t < t_end; ++t) {
            const int buf = (t - t_begin) & 1;
            const bool chunk = t >= tr.n_ct;
            const int key0 = chunk ? (t - tr.n_ct) * KT : t * KT;
            const int lim = chunk ? g.S : g.n;
            if (t + 1 < t_end) issue(t + 1, buf ^ 1);
            if (live > 0) {
                if (chunk && key0 + KT <= g.S && key0 + KT - 1 <= wave_q0)
                    fwd_tile<D, false, false, false>(Ks[buf], Vs[buf], off, qf, o_acc, m_ref,
                                                     m_seen, overflow, l_acc, lt_acc, g.c, 0, 0,
                                                     false, 0, rbase, lane);
                else
                    fwd_tile<D, true, false, false>(Ks[buf], Vs[buf], off, qf, o_acc, m_ref,
                                                    m_seen, overflow, l_acc, lt_acc, g.c, key0,
                                                    lim, chunk, g.G, rbase, lane);
            }
            wait_tiles();
            __syncthreads();
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) overflow |= !(l_acc[rb] <= kSumLimit);
        if (!__syncthreads_or(overflow)) goto store;
    }

    // Tracked sweeps (rare): the first fixes each row's reference max at its
    // first visible tile and records every tile max in m_seen; if a row's
    // logits still overshoot that reference by more than kHeadroom, the
    // second reruns the tiles with the exact row max
    for (int sweep = 0; sweep < 2; ++sweep) {
        bool overflow = false;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            m_ref[rb] = (sweep == 0) ? -INFINITY : m_seen[rb];
            l_acc[rb] = 0.f;
            lt_acc[rb] = 0.f;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) o_acc[rb][db][v] = 0.f;
        }
        if (t_begin < t_end) issue(t_begin, 0);
        wait_tiles();
        __syncthreads();

        // full cache tiles first (no mask), then the partial and chunk tiles
        const int n_full = g.n / KT;
        const int t_mid = max(t_begin, min(t_end, n_full));
        for (int t = t_begin; t < t_mid; ++t) {
            const int buf = (t - t_begin) & 1;
            if (t + 1 < t_end) issue(t + 1, buf ^ 1);   // next tile lands while this one is used
            if (live > 0)
                fwd_tile<D, false>(Ks[buf], Vs[buf], off, qf, o_acc, m_ref, m_seen, overflow, l_acc,
                                   lt_acc, g.c, 0, 0, false, 0, rbase, lane);
            wait_tiles();
            __syncthreads();
        }
        for (int t = t_mid; t < t_end; ++t) {
            const int buf = (t - t_begin) & 1;
            const bool chunk = t >= tr.n_ct;
            const int key0 = chunk ? (t - tr.n_ct) * KT : t * KT;
            const int lim = chunk ? g.S : g.n;
            if (t + 1 < t_end) issue(t + 1, buf ^ 1);
            if (live > 0)
                fwd_tile<D, true>(Ks[buf], Vs[buf], off, qf, o_acc, m_ref, m_seen, overflow, l_acc,
                                  lt_acc, g.c, key0, lim, chunk, g.G, rbase, lane);
            wait_tiles();
            __syncthreads();
        }
        if (!__syncthreads_or(overflow)) break;
    }

store:
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const float l = l_acc[rb] + xor32(l_acc[rb]);
        const float lt = lt_acc[rb] + xor32(lt_acc[rb]);
        const int r = rbase + rb * 32 + l32;
        if (r >= g.R) continue;
        const size_t prow = ((size_t)split * BH + bh) * g.rows_pad + r;
        if (half == 0) *(f32x4*)(ml_part + prow * 4) = f32x4{m_ref[rb], l, lt, 0.f};
        float* orow = o_part + prow * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const f32x4 v4 = {o_acc[rb][db][4 * gq + 0], o_acc[rb][db][4 * gq + 1],
                                  o_acc[rb][db][4 * gq + 2], o_acc[rb][db][4 * gq + 3]};
                *(f32x4*)(orow + db * 32 + 8 * gq + 4 * half) = v4;
            }
    }
}

// ---------------------------------------------------------------------------
// pass 1, few rows (G * S <= 32, e.g. one decode token per sequence): a
// single 32-row block per (b, kv head), so the waves of a workgroup take
// different 32-key blocks of each KT-key tile, keep their own softmax state,
// and merge it through LDS at the end.  The base-2 logits of the real rows
// are also written out (16 B per key for 4 rows, against 256 B of K), so the
// summed weights need no second read of K.
// ---------------------------------------------------------------------------
constexpr int NW_S = KT / 32;          // waves per workgroup (one key block each)
constexpr int NT_S = NW_S * 64;
constexpr int STAGES_S = 4;            // LDS tile buffers: 3 tiles in flight

// s_waitcnt with vmcnt(n) (n < 64) and no wait on the other counters.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int D>
__global__ __launch_bounds__(NT_S, 1) void attn_fwd_small_kernel(
    const AttnGeom g, const int nsplit, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn,
    float* __restrict__ o_part, float* __restrict__ ml_part, float* __restrict__ logits,
    TailState* __restrict__ ts) {
    // stage b: K tile in KV[b], V tile in KV[STAGES_S + b]; reused for the final merge
    __shared__ __attribute__((aligned(16))) uint16_t KV[2 * STAGES_S][KT * D];
    // per wave: the base-2 logits of its key blocks of up to LGS_ROWS / R
    // consecutive full tiles, [tile][row][key], written out together
    constexpr int LGS_ROWS = 64;
    __shared__ __attribute__((aligned(16))) float lgs[NW_S][LGS_ROWS * 32];
    uint16_t (*Ks)[KT * D] = KV;
    uint16_t (*Vs)[KT * D] = KV + STAGES_S;
    // this wave's copy instructions per tile (K and V)
    constexpr int PER_TILE = 2 * KT * (D / 8) / NT_S;

    int qt, bh, split;
    decode_block(1, nsplit, qt, bh, split);
    const int BH = g.B * g.Hkv;
    const int b = bh / g.Hkv, h = bh % g.Hkv;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    if (split == 0 && tid == 0) tail_state_init(ts, bh);   // for a tail that follows
    const int l32 = lane & 31, half = lane >> 5;

    const TileRange tr = tile_range(g, 0);
    const int t_begin = (int)((long)split * tr.total / nsplit);
    const int t_end = (int)((long)(split + 1) * tr.total / nsplit);
    const uint16_t* kc_bh = kc + (size_t)bh * g.C * D;
    const uint16_t* vc_bh = vc + (size_t)bh * g.C * D;
    const uint16_t* kn_bh = kn + (size_t)bh * g.S * D;
    const uint16_t* vn_bh = vn + (size_t)bh * g.S * D;

    float m_ref[RB], m_seen[RB], l_acc[RB], lt_acc[RB];
    f32x16 o_acc[RB][D / 32];
    m_seen[0] = -INFINITY;
    // Each wave copies the 32 K and V rows of its own key block of a tile and
    // reads only those, so the waves share no tile data: a wave waits for
    // its own copies (loads complete in issue order) and needs no barrier
    // per tile.  A stage is rewritten by the wave that read it, after its
    // reads of it have returned.
    const TileCopy<D, false, 1, 32, true> kcopy(0, lane);   // rows read once
    const TileCopy<D, true, 1, 32, true> vcopy(0, lane);
    const int n_full_tiles = g.n / KT;
    auto issue = [&](int t, int buf) {
        if (t < n_full_tiles) {   // every row exists: scalar base, fixed lane offsets
            const size_t row0 = (size_t)t * KT + wave * 32;
            kcopy.issue(Ks[buf] + wave * 32 * D, kc_bh + row0 * D, 0);
            vcopy.issue(Vs[buf] + wave * 32 * D, vc_bh + row0 * D, 0);
            return;
        }
        const bool chunk = t >= tr.n_ct;
        const int key0 = chunk ? (t - tr.n_ct) * KT : t * KT;
        const int lim = chunk ? g.S : g.n;
        issue_tile<D, false, 1, 32>(Ks[buf] + wave * 32 * D, chunk ? kn_bh : kc_bh,
                                    key0 + wave * 32, lim, 0, lane);
        issue_tile<D, true, 1, 32>(Vs[buf] + wave * 32 * D, chunk ? vn_bh : vc_bh,
                                   key0 + wave * 32, lim, 0, lane);
    };
    // tiles t_begin .. t_begin+2 in flight
    auto prologue = [&]() {
        for (int i = 0; i < STAGES_S - 1 && t_begin + i < t_end; ++i) issue(t_begin + i, i);
    };
    // The main sweep's first copies go out before the query and diagonal-key
    // loads below, so that their latency is not paid twice before the first
    // tile can be used.
    prologue();

    bf16x8 qf[RB][D / 16];
    load_q<D>(qf, q, g, b, h, 0, l32, half);
    const LdsOffsets<D> off(lane);
    float* lg_row = (l32 < g.R) ? logits + ((size_t)bh * g.R + l32) * logit_stride(g) : nullptr;

    float* const logits_bh = logits + (size_t)bh * g.R * logit_stride(g);
    // write_logits (wave-uniform): the main sweep stores the logits; the
    // tracked sweeps do not (the logits do not depend on the reference).
    // issued: the prologue's copies are already in flight.
    auto sweep_tiles = [&](auto TRC, bool& overflow, bool write_logits, bool issued) {
        constexpr bool TRACK = decltype(TRC)::value;
        float* const lg = write_logits ? lg_row : nullptr;
        // logits of full tiles batched in the LDS stage: nb tiles from key
        // b_key0 on; flushed when the stage is full, before a masked tile,
        // and at the end, so the stores of a batch go out back to back
        const int tf = LGS_ROWS / g.R;
        int nb = 0, b_key0 = 0;
        auto flush = [&]() {
            const int per = g.R * 8;   // 16-byte pieces per tile
            for (int cix = lane; cix < nb * per; cix += 64) {
                const int slot = cix / per, rem = cix - slot * per;
                const int row = rem >> 3, k4 = rem & 7;
                const f32x4 v = *(const f32x4*)&lgs[wave][(slot * g.R + row) * 32 + 4 * k4];
                *(f32x4*)(logits_bh + (size_t)row * logit_stride(g) + b_key0 + slot * KT +
                          wave * 32 + 4 * k4) = v;
            }
            nb = 0;
        };
        if (!issued) prologue();
        // wait for the first tile
        {
            const int later = min(STAGES_S - 2, t_end - 1 - t_begin);
            if (later >= 2)
                wait_vm<2 * PER_TILE>();
            else if (later == 1)
                wait_vm<PER_TILE>();
            else
                wait_tiles();
        }
        for (int t = t_begin; t < t_end; ++t) {
            const int buf = (t - t_begin) % STAGES_S;
            const bool chunk = t >= tr.n_ct;
            const int key0 = chunk ? (t - tr.n_ct) * KT : t * KT;
            const int lim = chunk ? g.S : g.n;
            const int col0 = chunk ? g.C + key0 : key0;
            // the stage of tile t+3 was last read, by this wave, for tile t-1
            if (t + STAGES_S - 1 < t_end) issue(t + STAGES_S - 1, (buf + STAGES_S - 1) % STAGES_S);
            if (!chunk && key0 + KT <= g.n) {
                // full tile: the logits of the real rows go to the LDS stage
                if (nb == 0) b_key0 = key0;
                float* const stage =
                    (write_logits && l32 < g.R) ? &lgs[wave][nb * g.R * 32] : nullptr;
                fwd_block<D, false, false, false, false, TRACK>(
                    Ks[buf], Vs[buf], off, qf, o_acc, m_ref, m_seen, overflow, l_acc, lt_acc, g.c,
                    wave, key0, lim, false, 0, 0, lane, nullptr, col0, wave, nullptr, nullptr,
                    nullptr, nullptr, stage);
                if (write_logits && ++nb == tf) flush();
            } else {
                if (nb > 0) flush();
                fwd_block<D, true, false, false, false, TRACK>(
                    Ks[buf], Vs[buf], off, qf, o_acc, m_ref, m_seen, overflow, l_acc, lt_acc, g.c,
                    wave, key0, lim, chunk, g.G, 0, lane, lg, col0, wave);
            }
            // this wave's copies of tile t+1 must have landed; tiles issued
            // after it may stay in flight
            const int later = min(STAGES_S - 2, t_end - 1 - (t + 1));
            if (later >= 2)
                wait_vm<2 * PER_TILE>();
            else if (later == 1)
                wait_vm<PER_TILE>();
            else
                wait_tiles();
        }
        if (nb > 0) flush();
    };
    auto zero_state = [&]() {
        l_acc[0] = 0.f;
        lt_acc[0] = 0.f;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) o_acc[0][db][v] = 0.f;
    };

    // Main sweep: each row's reference is its own base-2 logit against its
    // diagonal chunk key, as in attn_fwd_kernel (no per-tile max); row sums
    // above 2^kHeadroom send the workgroup to the tracked sweeps.  The
    // logits are written here only (they do not depend on the reference).
    {
        bool overflow = false;
        const int r = l32;
        const bool ok = r < g.R;
        const uint16_t* kself = kn_bh + (size_t)(ok ? r / g.G : 0) * D + 8 * half;
        float dot = 0.f;
#pragma unroll
        for (int k16 = 0; k16 < D / 16; ++k16) {
            const bf16x8 kv = as_bf16x8(*(const u32x4*)(kself + 16 * k16));
#pragma unroll
            for (int e = 0; e < 8; ++e) dot = fmaf((float)qf[0][k16][e], (float)kv[e], dot);
        }
        dot += xor32(dot);
        m_ref[0] = ok ? dot * g.c : 0.f;
        zero_state();
        sweep_tiles(TrackC<false>{}, overflow, true, true);
        overflow |= !(l_acc[0] <= kSumLimit);
        if (!__syncthreads_or(overflow)) goto merge;
    }
    // tracked sweeps (rare): first-tile reference with every tile max
    // recorded, then, if still overshot, the exact row max
    for (int sweep = 0; sweep < 2; ++sweep) {
        bool overflow = false;
        m_ref[0] = (sweep == 0) ? -INFINITY : m_seen[0];
        zero_state();
        sweep_tiles(TrackC<true>{}, overflow, false, false);
        if (!__syncthreads_or(overflow)) break;
    }

merge:
    // merge the waves' (m, l, lt, O) through LDS (the tiles are free now)
    const float l = l_acc[0] + xor32(l_acc[0]);
    const float lt = lt_acc[0] + xor32(lt_acc[0]);
    constexpr int XS = D / 2 + 4;               // [NW_S][64 lanes][XS] floats
    static_assert(NW_S * 64 * XS * 4 <= (int)sizeof(KV), "merge area exceeds the tiles");
    float* xch = (float*)&KV[0][0];
    float* mine = xch + ((size_t)wave * 64 + lane) * XS;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) mine[db * 16 + v] = o_acc[0][db][v];
    mine[D / 2 + 0] = m_ref[0];
    mine[D / 2 + 1] = l;
    mine[D / 2 + 2] = lt;
    __syncthreads();
    if (wave != 0) return;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW_S; ++w) M = fmaxf(M, xch[((size_t)w * 64 + lane) * XS + D / 2]);
    float wt[NW_S], L = 0.f, Lt = 0.f;
#pragma unroll
    for (int w = 0; w < NW_S; ++w) {
        const float* o = xch + ((size_t)w * 64 + lane) * XS;
        wt[w] = (M == -INFINITY) ? 0.f : fast_exp2(o[D / 2] - M);
        L += wt[w] * o[D / 2 + 1];
        Lt += wt[w] * o[D / 2 + 2];
    }
    const int r = l32;
    if (r >= g.R) return;
    const size_t prow = ((size_t)split * BH + bh) * g.rows_pad + r;
    if (half == 0) *(f32x4*)(ml_part + prow * 4) = f32x4{M, L, Lt, 0.f};
    float* orow = o_part + prow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < NW_S; ++w) {
                const float* o = xch + ((size_t)w * 64 + lane) * XS + db * 16 + 4 * gq;
                acc += wt[w] * f32x4{o[0], o[1], o[2], o[3]};
            }
            *(f32x4*)(orow + db * 32 + 8 * gq + 4 * half) = acc;
        }
}

// ---------------------------------------------------------------------------
// pass 1 for at most 16 rows (decode: the G <= 16 query heads of a group and
// one token): the few-row kernel's structure on the 16x16x32 MFMA.
//
// S^T = K Q^T takes 16 keys x 16 rows per instruction, so the unused rows
// cost a quarter of what they do on the 32x32 shape: lane l owns row l%16
// and keys 4*(l/16) + [0, 4) of each 16-key half of the wave's 32-key block,
// i.e. 8 logits per block to exponentiate instead of 16.  The PV product sums
// the block's 32 keys in the order the lanes hold them: MFMA k-index
// 8*(l/16) + e is key 4*(l/16) + e for e < 4 and 16 + 4*(l/16) + e - 4 for
// e >= 4, so the bf16 P^T fragment of a lane is its own 8 weights (no
// exchange between lanes) and V^T comes from two transposed LDS reads, one
// per 4-key run.
// ---------------------------------------------------------------------------
constexpr int kFewRows = 16;

// One 16x16x32 bf16 MFMA, fp32 accumulate.  Operand layout:
//   A (16 x 32): lane l holds row l%16, k-values 8*(l/16) + [0, 8);
//   B (32 x 16): lane l holds column l%16, k-values 8*(l/16) + [0, 8);
//   C (16 x 16): lane l holds column l%16, rows 4*(l/16) + [0, 4).
__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8 a, const bf16x8 b, const f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float xor16(float x) { return __shfl_xor(x, 16, 64); }

// Per-lane LDS byte offsets of the 16-row path inside a tile, for key block 0
// and 16-key half 0 (the block adds lkb*32 rows, the half 16 rows: constants
// that fold into the instructions' immediate offsets, since the swizzles
// depend only on key mod 16 and key mod 4).
//   k[ks]: K fragment, key l%16, dims 32*ks + 8*(l/16) + [0, 8);
//   v[db]: transposed V read of dims 16*db + [0, 16) over keys
//          4*(l/16) + [0, 4): input lane j of a 16-lane group reads dims
//          16*db + 4*(j%4) + [0, 4) of key 4*(l/16) + j/4, and the hardware
//          hands output lane i dim 16*db + i of those 4 keys.
template <int D>
struct LdsOffsets16 {
    uint32_t k[D / 32];
    uint32_t v[D / 16];
    __device__ __forceinline__ explicit LdsOffsets16(int lane) {
        const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
            k[ks] = 2u * (uint32_t)tile_off<D, false>(l16, 4 * ks + g);
        const int key = 4 * g + (l16 >> 2);
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
            const int d = 16 * db + 4 * (l16 & 3);
            v[db] = 2u * (uint32_t)(tile_off<D, true>(key, d >> 3) + (d & 7));
        }
    }
};

// One 32-key block of the 16-row pass 1 for one wave; the block's rows sit at
// block lkb of the (per-wave) LDS tiles.  Same contract as fwd_block, with
// one 16-row block per wave: MASKED handles the last partial cache tile and
// the chunk tiles; lg_stage (full tiles) receives the block's base-2 logits
// as [row][32 keys]; lg_row (masked tiles) receives them at logits columns
// col0 + (key - key0) for the real keys.
template <int D, bool MASKED, bool TRACK>
__device__ __forceinline__ void fwd_block16(const uint16_t* Ks, const uint16_t* Vs,
                                            const LdsOffsets16<D>& off,
                                            const bf16x8 (&qf)[D / 32], f32x4 (&o_acc)[D / 16],
                                            float& m_ref, float& m_seen, bool& overflow,
                                            float& l_acc, float& lt_acc, float c, int kb,
                                            int key0, int lim, bool chunk, int G, int lane,
                                            float* lg_row, int col0, int lkb, float* lg_stage) {
    const int l16 = lane & 15, g = lane >> 4;
    const uint32_t blk = (uint32_t)lkb * 32 * D * 2;   // bytes to this block's rows
    constexpr uint32_t HALF = 16 * D * 2;               // bytes to the second 16 keys
    // S^T of the two 16-key halves; each sums its k-steps in two chains (even
    // and odd k-steps), so that no MFMA waits for the one just issued
    f32x4 s[2];
    {
        f32x4 acc[2][2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int p = 0; p < 2; ++p) acc[h][p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const bf16x8 kf = as_bf16x8(lds_read16(Ks, off.k[ks] + blk + h * HALF));
                acc[h][ks & 1] = mfma16x16x32(kf, qf[ks], acc[h][ks & 1]);
            }
#pragma unroll
        for (int h = 0; h < 2; ++h) s[h] = acc[h][0] + acc[h][1];
    }
    // element e of s[h] is key kb*32 + 16*h + 4*g + e of the tile, row l16
    if (MASKED) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int key = key0 + kb * 32 + 16 * h + 4 * g + e;
                const bool ok = key < lim && (!chunk || key * G <= l16);
                s[h][e] = ok ? s[h][e] : -INFINITY;
            }
        if (lg_row) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int kl = kb * 32 + 16 * h + 4 * g + e;
                    if (key0 + kl < lim) lg_row[col0 + kl] = s[h][e] * c;
                }
        }
    } else if (lg_stage) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
            *(f32x4*)(lg_stage + l16 * 32 + 16 * h + 4 * g) = s[h] * c;
    }
    if constexpr (TRACK) {   // as in fwd_block: first-tile reference, every tile max kept
        float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                         fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
        mx = fmaxf(mx, xor16(mx));
        mx = fmaxf(mx, xor32(mx));   // the row's 4 lanes
        const float mt = mx * c;
        m_seen = fmaxf(m_seen, mt);
        m_ref = (m_ref == -INFINITY) ? mt : m_ref;
        overflow |= mt > m_ref + kHeadroom;
    }
    // P = 2^(s*c - m) and the row sums (l exact, lt over the bf16 weights)
    const float m_use = (!TRACK || m_ref != -INFINITY) ? m_ref : 0.f;
    bf16x8 pf;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float p = fast_exp2(fmaf(s[h][e], c, -m_use));
            l_acc += p;
            pf[4 * h + e] = (__bf16)p;
        }
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        const bf16x2 pair = {pf[e], pf[e + 1]};
        lt_acc = __builtin_amdgcn_fdot2_f32_bf16(pair, kOnes2, lt_acc, false);
    }
    // O^T += V^T P^T over the block's 32 keys, in the lanes' key order
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
        const u32x2 lo = lds_read_tr(Vs, off.v[db] + blk);
        const u32x2 hi = lds_read_tr(Vs, off.v[db] + blk + HALF);
        const bf16x8 vf = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
        o_acc[db] = mfma16x16x32(vf, pf, o_acc[db]);
    }
}

// LDS stages of the 16-row kernel: 2 tiles in flight while one is read (the
// fourth stage's LDS goes to the logits stage instead)
constexpr int STAGES_F = 3;

template <int D>
__global__ __launch_bounds__(NT_S, 1) void attn_fwd_few_kernel(
    const AttnGeom g, const int nsplit, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn,
    float* __restrict__ o_part, float* __restrict__ ml_part, float* __restrict__ logits,
    TailState* __restrict__ ts) {
    // stage b: K tile in KV[b], V tile in KV[STAGES_F + b]; reused for the final merge
    __shared__ __attribute__((aligned(16))) uint16_t KV[2 * STAGES_F][KT * D];
    // per wave: the base-2 logits of its key blocks of up to LGS_ROWS / R
    // consecutive full tiles, [tile][row][key], written out together (for a
    // one-token step, R <= 4, the whole split's logits go out in one burst at
    // its end)
    constexpr int LGS_ROWS = 128;
    __shared__ __attribute__((aligned(16))) float lgs[NW_S][LGS_ROWS * 32];
    uint16_t (*Ks)[KT * D] = KV;
    uint16_t (*Vs)[KT * D] = KV + STAGES_F;
    constexpr int PER_TILE = 2 * KT * (D / 8) / NT_S;   // this wave's copies per tile

    int qt, bh, split;
    decode_block(1, nsplit, qt, bh, split);
    const int BH = g.B * g.Hkv;
    const int b = bh / g.Hkv, h = bh % g.Hkv;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    if (split == 0 && tid == 0) tail_state_init(ts, bh);   // for a tail that follows
    const int l16 = lane & 15, grp = lane >> 4;

    const TileRange tr = tile_range(g, 0);
    const int t_begin = (int)((long)split * tr.total / nsplit);
    const int t_end = (int)((long)(split + 1) * tr.total / nsplit);
    const uint16_t* kc_bh = kc + (size_t)bh * g.C * D;
    const uint16_t* vc_bh = vc + (size_t)bh * g.C * D;
    const uint16_t* kn_bh = kn + (size_t)bh * g.S * D;
    const uint16_t* vn_bh = vn + (size_t)bh * g.S * D;

    // As in attn_fwd_small_kernel: each wave copies and reads only the 32 K
    // and V rows of its own key block of a tile, so it waits for its own
    // copies and needs no barrier per tile.
    const TileCopy<D, false, 1, 32, true> kcopy(0, lane);   // rows read once
    const TileCopy<D, true, 1, 32, true> vcopy(0, lane);
    const int n_full_tiles = g.n / KT;
    auto issue = [&](int t, int buf) {
        if (t < n_full_tiles) {
            const size_t row0 = (size_t)t * KT + wave * 32;
            kcopy.issue(Ks[buf] + wave * 32 * D, kc_bh + row0 * D, 0);
            vcopy.issue(Vs[buf] + wave * 32 * D, vc_bh + row0 * D, 0);
            return;
        }
        const bool chunk = t >= tr.n_ct;
        const int key0 = chunk ? (t - tr.n_ct) * KT : t * KT;
        const int lim = chunk ? g.S : g.n;
        issue_tile<D, false, 1, 32>(Ks[buf] + wave * 32 * D, chunk ? kn_bh : kc_bh,
                                    key0 + wave * 32, lim, 0, lane);
        issue_tile<D, true, 1, 32>(Vs[buf] + wave * 32 * D, chunk ? vn_bh : vc_bh,
                                   key0 + wave * 32, lim, 0, lane);
    };
    auto prologue = [&]() {
        for (int i = 0; i < STAGES_F - 1 && t_begin + i < t_end; ++i) issue(t_begin + i, i);
    };
    // the main sweep's first copies go out before the query loads
    prologue();

    // Q fragments (B operand of S^T = K Q^T): row l16, dims 32*ks + 8*grp + [0, 8)
    const bool row_ok = l16 < g.R;
    bf16x8 qf[D / 32];
    {
        const uint16_t* qrow =
            q + (((size_t)b * g.Hq + (size_t)h * g.G + (l16 % g.G)) * g.S + l16 / g.G) * D +
            8 * grp;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (row_ok) v = *(const u32x4*)(qrow + 32 * ks);
            qf[ks] = as_bf16x8(v);
        }
    }
    const LdsOffsets16<D> off(lane);
    float* lg_row = row_ok ? logits + ((size_t)bh * g.R + l16) * logit_stride(g) : nullptr;
    float* const logits_bh = logits + (size_t)bh * g.R * logit_stride(g);

    float m_ref = 0.f, m_seen = -INFINITY, l_acc = 0.f, lt_acc = 0.f;
    f32x4 o_acc[D / 16];
    auto zero_state = [&]() {
        l_acc = 0.f;
        lt_acc = 0.f;
#pragma unroll
        for (int db = 0; db < D / 16; ++db) o_acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    // write_logits (wave-uniform): the main sweep stores the logits, the
    // tracked sweeps do not; issued: the prologue's copies are in flight
    auto sweep_tiles = [&](auto TRC, bool& overflow, bool write_logits, bool issued) {
        constexpr bool TRACK = decltype(TRC)::value;
        float* const lg = write_logits ? lg_row : nullptr;
        const int tf = LGS_ROWS / g.R;
        int nb = 0, b_key0 = 0;
        auto flush = [&]() {
            const int per = g.R * 8;   // 16-byte pieces per tile
            for (int cix = lane; cix < nb * per; cix += 64) {
                const int slot = cix / per, rem = cix - slot * per;
                const int row = rem >> 3, k4 = rem & 7;
                const f32x4 v = *(const f32x4*)&lgs[wave][(slot * g.R + row) * 32 + 4 * k4];
                *(f32x4*)(logits_bh + (size_t)row * logit_stride(g) + b_key0 + slot * KT +
                          wave * 32 + 4 * k4) = v;
            }
            nb = 0;
        };
        if (!issued) prologue();
        {
            const int later = min(STAGES_F - 2, t_end - 1 - t_begin);
            if (later >= 2)
                wait_vm<2 * PER_TILE>();
            else if (later == 1)
                wait_vm<PER_TILE>();
            else
                wait_tiles();
        }
        for (int t = t_begin; t < t_end; ++t) {
            const int buf = (t - t_begin) % STAGES_F;
            const bool chunk = t >= tr.n_ct;
            const int key0 = chunk ? (t - tr.n_ct) * KT : t * KT;
            const int lim = chunk ? g.S : g.n;
            const int col0 = chunk ? g.C + key0 : key0;
            // the stage of tile t+2 was last read, by this wave, for tile t-1
            if (t + STAGES_F - 1 < t_end) issue(t + STAGES_F - 1, (buf + STAGES_F - 1) % STAGES_F);
            if (!chunk && key0 + KT <= g.n) {
                if (nb == 0) b_key0 = key0;
                float* const stage =
                    (write_logits && row_ok) ? &lgs[wave][nb * g.R * 32] : nullptr;
                fwd_block16<D, false, TRACK>(Ks[buf], Vs[buf], off, qf, o_acc, m_ref, m_seen,
                                             overflow, l_acc, lt_acc, g.c, wave, key0, lim,
                                             false, 0, lane, nullptr, col0, wave, stage);
                if (write_logits && ++nb == tf) flush();
            } else {
                if (nb > 0) flush();
                fwd_block16<D, true, TRACK>(Ks[buf], Vs[buf], off, qf, o_acc, m_ref, m_seen,
                                            overflow, l_acc, lt_acc, g.c, wave, key0, lim, chunk,
                                            g.G, lane, lg, col0, wave, nullptr);
            }
            const int later = min(STAGES_F - 2, t_end - 1 - (t + 1));
            if (later >= 2)
                wait_vm<2 * PER_TILE>();
            else if (later == 1)
                wait_vm<PER_TILE>();
            else
                wait_tiles();
        }
        if (nb > 0) flush();
    };
    // the row sum of a lane's row: its 4 lanes (l16 + 16*grp)
    auto row_sum = [&](float x) {
        x += xor16(x);
        return x + xor32(x);
    };

    // Main sweep with each row's reference at its own logit against its
    // diagonal chunk key (no per-tile max); row sums above 2^kHeadroom send
    // the workgroup to the tracked sweeps.
    {
        bool overflow = false;
        const uint16_t* kself = kn_bh + (size_t)(row_ok ? l16 / g.G : 0) * D + 8 * grp;
        float dot = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            const bf16x8 kv = as_bf16x8(*(const u32x4*)(kself + 32 * ks));
#pragma unroll
            for (int e = 0; e < 8; ++e) dot = fmaf((float)qf[ks][e], (float)kv[e], dot);
        }
        dot = row_sum(dot);
        m_ref = row_ok ? dot * g.c : 0.f;
        zero_state();
        sweep_tiles(TrackC<false>{}, overflow, true, true);
        overflow |= !(row_sum(l_acc) <= kSumLimit);
        if (!__syncthreads_or(overflow)) goto merge;
    }
    // tracked sweeps (rare): first-tile reference with every tile max
    // recorded, then, if still overshot, the exact row max
    for (int sweep = 0; sweep < 2; ++sweep) {
        bool overflow = false;
        m_ref = (sweep == 0) ? -INFINITY : m_seen;
        zero_state();
        sweep_tiles(TrackC<true>{}, overflow, false, false);
        if (!__syncthreads_or(overflow)) break;
    }

merge:
    // merge the waves' (m, l, lt, O) through LDS (the tiles are free now)
    {
        const float l = row_sum(l_acc);
        const float lt = row_sum(lt_acc);
        constexpr int XS = D / 4 + 4;   // [NW_S][64 lanes][XS] floats
        static_assert(NW_S * 64 * XS * 4 <= (int)sizeof(KV), "merge area exceeds the tiles");
        float* xch = (float*)&KV[0][0];
        float* mine = xch + ((size_t)wave * 64 + lane) * XS;
#pragma unroll
        for (int db = 0; db < D / 16; ++db) *(f32x4*)(mine + 4 * db) = o_acc[db];
        mine[D / 4 + 0] = m_ref;
        mine[D / 4 + 1] = l;
        mine[D / 4 + 2] = lt;
        __syncthreads();
        if (wave != 0) return;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW_S; ++w) M = fmaxf(M, xch[((size_t)w * 64 + lane) * XS + D / 4]);
        float wt[NW_S], L = 0.f, Lt = 0.f;
#pragma unroll
        for (int w = 0; w < NW_S; ++w) {
            const float* o = xch + ((size_t)w * 64 + lane) * XS;
            wt[w] = (M == -INFINITY) ? 0.f : fast_exp2(o[D / 4] - M);
            L += wt[w] * o[D / 4 + 1];
            Lt += wt[w] * o[D / 4 + 2];
        }
        if (!row_ok) return;
        const size_t prow = ((size_t)split * BH + bh) * g.rows_pad + l16;
        if (grp == 0) *(f32x4*)(ml_part + prow * 4) = f32x4{M, L, Lt, 0.f};
        float* orow = o_part + prow * D;
        // lane holds dims 16*db + 4*grp + [0, 4) of its row
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < NW_S; ++w)
                acc += wt[w] * *(const f32x4*)(xch + ((size_t)w * 64 + lane) * XS + 4 * db);
            *(f32x4*)(orow + 16 * db + 4 * grp) = acc;
        }
    }
}

// Summed weights of columns j0 .. j0+3 of one (b, kv head) straight from the
// stored logits (few-row path): column j sums 2^(u_rj - L2_r) over the rows
// that see it, in row order, one 16-byte load per row (the logit rows are
// padded to a multiple of 4 floats, so the quad stays inside the row).
// `lg` points at column j0 of row 0; `lb` at the rows' base-2 LSE.
__device__ __forceinline__ void logit_quad_sums(const AttnGeom& g, const float* __restrict__ lg,
                                                const float* lb, int j0, float (&s)[4]) {
    const int W = g.C + g.S;
    const int WL = logit_stride(g);
    // column j0 + e is a valid cache slot or a chunk token, seen by rows
    // r >= r_lo[e] (row r sees chunk token t iff t*G <= r)
    bool col[4];
    int r_lo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int jj = j0 + e;
        col[e] = jj < W && (jj < g.n || jj >= g.C);
        r_lo[e] = jj < g.C ? 0 : (jj - g.C) * g.G;
        s[e] = 0.f;
    }
    // rows in order; the logits of 8 rows are loaded before they are summed
    for (int r0 = 0; r0 < g.R; r0 += 8) {
        f32x4 x[8];
        float lr[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int r = min(r0 + u, g.R - 1);
            x[u] = *(const f32x4*)(lg + (size_t)r * WL);
            lr[u] = lb[r];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (r0 + u < g.R && col[e] && r0 + u >= r_lo[e]) s[e] += fast_exp2(x[u][e] - lr[u]);
    }
}

// Summed weights straight from the stored logits (few-row path): a thread
// takes four consecutive columns.
// With non-null `scores` the kernel also accumulates: scores[j] += wsum[j]
// (j < n), new_scores[t] = wsum[C + t].
__global__ __launch_bounds__(256) void wsum_from_logits_kernel(
    const AttnGeom g, const float* __restrict__ logits, const float* __restrict__ l2,
    float* __restrict__ wsum, float* __restrict__ scores, float* __restrict__ new_scores) {
    const int W = g.C + g.S;
    const int nq = (W + 3) / 4;   // column quads per (b, kv head)
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)g.B * g.Hkv * nq) return;
    const int j0 = (int)(idx % nq) * 4;
    const int bh = (int)(idx / nq);
    float s[4];
    logit_quad_sums(g, logits + (size_t)bh * g.R * logit_stride(g) + j0,
                    l2 + (size_t)bh * g.rows_pad, j0, s);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int j = j0 + e;
        if (j >= W) continue;
        wsum[(size_t)bh * W + j] = s[e];
        if (scores) {
            if (j < g.n)
                scores[(size_t)bh * g.C + j] += s[e];
            else if (j >= g.C)
                new_scores[(size_t)bh * g.S + (j - g.C)] = s[e];
        }
    }
}

// ---------------------------------------------------------------------------
// combine the key splits: O (normalised), natural LSE, base-2 L for pass 2
// ---------------------------------------------------------------------------
// Merge of the key splits of row r (dims 4*dc .. 4*dc+3): the largest split
// reference M, the exact and the bf16-weight row sums L and Lt against M, and
// the O sums.  Splits are combined in order; the loads of CB splits are
// issued before any of them is used.
template <int D>
__device__ __forceinline__ void merge_splits(const AttnGeom& g, int nsplit,
                                             const float* __restrict__ o_part,
                                             const float* __restrict__ ml_part, int bh, int r,
                                             int dc, float& M, float& L, float& Lt, f32x4& acc) {
    const int BH = g.B * g.Hkv;
    constexpr int CB = 8;
    M = -INFINITY;
    L = 0.f;
    Lt = 0.f;
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
    if (nsplit <= 4) {   // few splits: one pass, all loads first
        f32x4 ml[4], o[4];
#pragma unroll
        for (int sp = 0; sp < 4; ++sp) {
            const size_t prow = ((size_t)sp * BH + bh) * g.rows_pad + r;
            ml[sp] = sp < nsplit ? *(const f32x4*)(ml_part + prow * 4)
                                 : f32x4{-INFINITY, 0.f, 0.f, 0.f};
            o[sp] = sp < nsplit ? *(const f32x4*)(o_part + prow * D + dc * 4)
                                : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int sp = 0; sp < 4; ++sp) M = fmaxf(M, ml[sp][0]);
#pragma unroll
        for (int sp = 0; sp < 4; ++sp) {
            if (sp < nsplit) {
                const float w = fast_exp2(ml[sp][0] - M);
                L += w * ml[sp][1];
                Lt += w * ml[sp][2];
                acc += w * o[sp];
            }
        }
        return;
    }
    for (int s0 = 0; s0 < nsplit; s0 += CB) {
        float m[CB];
#pragma unroll
        for (int u = 0; u < CB; ++u) {
            const int sp = s0 + u;
            m[u] = sp < nsplit ? ml_part[(((size_t)sp * BH + bh) * g.rows_pad + r) * 4]
                               : -INFINITY;
        }
#pragma unroll
        for (int u = 0; u < CB; ++u) M = fmaxf(M, m[u]);
    }
    for (int s0 = 0; s0 < nsplit; s0 += CB) {
        f32x4 ml[CB], o[CB];
#pragma unroll
        for (int u = 0; u < CB; ++u) {
            const int sp = s0 + u;
            const size_t prow = ((size_t)sp * BH + bh) * g.rows_pad + r;
            ml[u] = sp < nsplit ? *(const f32x4*)(ml_part + prow * 4) : f32x4{0.f, 0.f, 0.f, 0.f};
            o[u] = sp < nsplit ? *(const f32x4*)(o_part + prow * D + dc * 4)
                               : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < CB; ++u) {
            if (s0 + u < nsplit) {
                const float w = fast_exp2(ml[u][0] - M);
                L += w * ml[u][1];
                Lt += w * ml[u][2];
                acc += w * o[u];
            }
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
    float M, L, Lt;
    f32x4 acc;
    merge_splits<D>(g, nsplit, o_part, ml_part, bh, r, dc, M, L, Lt, acc);
    const float inv = 1.0f / Lt;
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
// One-token chunks on the few-row path: everything after the streaming pass
// in one workgroup per (b, kv head) -- the split merge (O, LSE), the summed
// weights from the stored logits, the score accumulation, the lexicographic
// minimum of (score, slot) (or the first empty slot while the cache fills)
// and the scatter of the token into that slot.  Each part does exactly the
// arithmetic of its own kernel (combine, logits-to-weights, accumulation,
// choice, scatter), so the results are those of the separate calls.
// ---------------------------------------------------------------------------
// The tail of a one-token step, in two kernels.  decode_tail_kernel splits
// each (b, kv head) over TAIL_P workgroups of TAIL_T threads by cache
// columns, so that it fills the chip: split merge, summed weights, score
// update and the running minimum (a device-scope atomic on the TailState).
// decode_scatter_kernel then makes the choice and writes the token into the
// chosen slot; the kernel boundary orders its score write after the
// columns' (a workgroup of the first kernel may have written that slot's
// score from another XCD's L2).
constexpr int TAIL_T = 256;
constexpr int TAIL_NQ = 4;   // column quads per thread in flight
constexpr int TAIL_P = 4;    // workgroups per (b, kv head)

template <int D>
__global__ __launch_bounds__(TAIL_T) void decode_tail_kernel(
    const AttnGeom g, const int nsplit, const float* __restrict__ o_part,
    const float* __restrict__ ml_part, const float* __restrict__ logits,
    TailState* __restrict__ ts, float* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ wsum, float* __restrict__ scores, float* __restrict__ new_scores) {
    constexpr int CH = D / 4;
    __shared__ float sh_l2[32];
    __shared__ float sh_pc[32];   // part 0: weight of the token's own column, per row
    __shared__ unsigned long long sh_min;
    const int bh = blockIdx.x / TAIL_P, part = blockIdx.x % TAIL_P;
    const int tid = threadIdx.x;
    const int W = g.C + 1;
    const float* lg = logits + (size_t)bh * g.R * logit_stride(g);
    const int WL = logit_stride(g);
    float* sc = scores + (size_t)bh * g.C;
    float* wrow = wsum + (size_t)bh * W;
    // this part's column quads [q_lo, q_hi); a thread takes quads TAIL_T apart
    const int nq = (g.C + 3) / 4;
    const int qp = (nq + TAIL_P - 1) / TAIL_P;
    const int q_lo = part * qp, q_hi = min(nq, q_lo + qp);
    constexpr int QSTEP = TAIL_T * TAIL_NQ;

    // The logits do not depend on the rows' final log-sum-exp: the first pass
    // of this thread's column quads (rows 0..3) is loaded before the merge,
    // so that both share one memory round trip.
    f32x4 x[TAIL_NQ][4];
    float old[TAIL_NQ][4];
#define H2O_TAIL_LOAD_ROWS(q0, r0)                                              \
    _Pragma("unroll") for (int u = 0; u < 4; ++u) {                             \
        const int r = min((r0) + u, g.R - 1);                                   \
        _Pragma("unroll") for (int k = 0; k < TAIL_NQ; ++k) {                   \
            const int q = (q0) + TAIL_T * k;                                    \
            x[k][u] = q < q_hi ? *(const f32x4*)(lg + (size_t)r * WL + 4 * q)   \
                               : f32x4{0.f, 0.f, 0.f, 0.f};                     \
        }                                                                       \
    }
    H2O_TAIL_LOAD_ROWS(q_lo + tid, 0)

    // the rows' base-2 log-sum-exp from the key splits (thread r < R); part 0
    // instead merges all of O (threads (r, dc)) and takes the weight of the
    // token's own column (column C, summed over the rows in order)
    if (part == 0) {
        for (int idx = tid; idx < g.R * CH; idx += TAIL_T) {
            const int r = idx / CH, dc = idx % CH;
            const float xc = dc == 0 ? lg[(size_t)r * WL + g.C] : 0.f;
            float M, L, Lt;
            f32x4 acc;
            merge_splits<D>(g, nsplit, o_part, ml_part, bh, r, dc, M, L, Lt, acc);
            const float inv = 1.0f / Lt;
            const int b = bh / g.Hkv, h = bh % g.Hkv;
            const size_t orow = (size_t)b * g.Hq + h * g.G + r;   // S = 1: row r is head h*G + r
            *(f32x4*)(out + orow * D + dc * 4) = acc * inv;
            if (dc == 0) {
                const float L2 = M + fast_log2(L);
                sh_l2[r] = L2;
                sh_pc[r] = fast_exp2(xc - L2);
                if (lse) lse[orow] = L2 * kLn2;
            }
        }
    } else if (tid < g.R) {
        float M, L, Lt;
        f32x4 acc;
        merge_splits<D>(g, nsplit, o_part, ml_part, bh, tid, 0, M, L, Lt, acc);
        sh_l2[tid] = M + fast_log2(L);
    }
    if (tid == 0) sh_min = ~0ull;
    __syncthreads();
    if (part == 0 && tid == 0) {
        float s_new = 0.f;   // rows in order
        for (int r = 0; r < g.R; ++r) s_new += sh_pc[r];
        wrow[g.C] = s_new;
        new_scores[bh] = s_new;
    }
    // summed weights of the cache columns, accumulated scores and the running
    // minimum; per column the rows are summed in row order as in
    // logit_quad_sums
    unsigned long long best = ~0ull;
    for (int q0 = q_lo + tid; q0 < q_hi; q0 += QSTEP) {
#pragma unroll
        for (int k = 0; k < TAIL_NQ; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 4 * (q0 + TAIL_T * k) + e;
                old[k][e] = j < g.n ? sc[j] : 0.f;
            }
        if (q0 != q_lo + tid) {
            H2O_TAIL_LOAD_ROWS(q0, 0)
        }
        float s[TAIL_NQ][4];
#pragma unroll
        for (int k = 0; k < TAIL_NQ; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) s[k][e] = 0.f;
        for (int r0 = 0; r0 < g.R; r0 += 4) {
            if (r0 > 0) {
                H2O_TAIL_LOAD_ROWS(q0, r0)
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (r0 + u >= g.R) break;
                const float lr = sh_l2[r0 + u];
#pragma unroll
                for (int k = 0; k < TAIL_NQ; ++k)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int j = 4 * (q0 + TAIL_T * k) + e;
                        if (j < g.n) s[k][e] += fast_exp2(x[k][u][e] - lr);
                    }
            }
        }
#pragma unroll
        for (int k = 0; k < TAIL_NQ; ++k) {
            if (q0 + TAIL_T * k >= q_hi) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 4 * (q0 + TAIL_T * k) + e;
                if (j >= g.C) continue;
                wrow[j] = s[k][e];
                if (j < g.n) {
                    const float acc = old[k][e] + s[k][e];
                    sc[j] = acc;
                    const unsigned long long kj =
                        ((unsigned long long)score_key(acc) << 32) | (unsigned)j;
                    best = kj < best ? kj : best;
                }
            }
        }
    }
#undef H2O_TAIL_LOAD_ROWS
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const unsigned long long o = __shfl_xor(best, off, 64);
        best = o < best ? o : best;
    }
    if ((tid & 63) == 0) atomicMin(&sh_min, best);
    __syncthreads();
    if (tid == 0) atomicMin(&ts[bh].min_key, sh_min);
}

// The choice and the scatter of a one-token step, one workgroup per (b, kv
// head): the first empty slot while the cache fills, else the lexicographic
// minimum the tail kernel left in the TailState; the token's K/V row, score
// and position go into that slot.
template <int D>
__global__ __launch_bounds__(64) void decode_scatter_kernel(
    const AttnGeom g, const TailState* __restrict__ ts, float* __restrict__ scores,
    const float* __restrict__ new_scores, int32_t* __restrict__ evict,
    uint16_t* __restrict__ kc, uint16_t* __restrict__ vc, int64_t* __restrict__ pos,
    const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn, int64_t p0) {
    constexpr int TPR = D / 8;   // threads per row (16 bytes each)
    const int bh = blockIdx.x, tid = threadIdx.x;
    const int slot = g.n < g.C ? g.n : (int)(ts[bh].min_key & 0xFFFFFFFFull);
    if (tid < 2 * TPR) {
        const u32x4 v = *(const u32x4*)((tid < TPR ? kn : vn) + (size_t)bh * D + (tid % TPR) * 8);
        *(u32x4*)((tid < TPR ? kc : vc) + ((size_t)bh * g.C + slot) * D + (tid % TPR) * 8) = v;
    }
    if (tid == 0) {
        evict[bh] = slot;
        scores[(size_t)bh * g.C + slot] = new_scores[bh];
        if (pos) pos[(size_t)bh * g.C + slot] = p0;
    }
}

// One KT-key tile of pass 2 for one wave: S = Q K^T per 32-key block, then
// the column sums of P = 2^(S*c - L2) over this wave's rows into colp.
// MASKED handles the last partial cache tile (G == 0) and chunk tiles (G > 0:
// row r sees chunk key t iff t*G <= r).
template <int D, bool MASKED, bool KSC = false, int KTT = KT>
__device__ __forceinline__ void colsum_tile(const uint16_t* Ks, const LdsOffsets<D>& off,
                                            float* colp,
                                            const bf16x8 (&qf)[RB][D / 16],
                                            const float (&l2v)[RB][16], float c, int key0,
                                            int lim, int G, int rbase, int l32, int half,
                                            const float* ksc = nullptr) {
    float col[KTT / 32];
#pragma unroll
    for (int kb = 0; kb < KTT / 32; ++kb) {
        f32x16 s[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int v = 0; v < 16; ++v) s[rb][v] = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            const bf16x8 kf = as_bf16x8(lds_read16(Ks, off.k[ks] + kb * 64 * D));
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) s[rb] = mfma32x32x16(qf[rb][ks], kf, s[rb]);
        }
        const int key = key0 + kb * 32 + l32;
        // KSC: the lane's key scale folds into the logit scale
        const float ck = KSC ? c * ksc[kb * 32 + l32] : c;
        // P in place of S, then a pairwise sum: the 16 exponentials of a row
        // block are independent, and the sum is a tree of depth 4 instead of
        // a chain of 16 dependent adds
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float p = fast_exp2(fmaf(s[rb][v], ck, -l2v[rb][v]));
                if (MASKED) {
                    const int r = rbase + rb * 32 + acc_row(v, half);
                    s[rb][v] = (key < lim && key * G <= r) ? p : 0.f;
                } else {
                    s[rb][v] = p;
                }
            }
#pragma unroll
        for (int rb = 1; rb < RB; ++rb)
#pragma unroll
            for (int v = 0; v < 16; ++v) s[0][v] += s[rb][v];
#pragma unroll
        for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
            for (int v = 0; v < w; ++v) s[0][v] += s[0][v + w];
        const float cs = s[0][0];
        col[kb] = cs + xor32(cs);
    }
    // both halves hold the sums; the lower half stores them (one divergent
    // region per tile, so the key blocks above schedule as one stretch)
    if (half == 0) {
#pragma unroll
        for (int kb = 0; kb < KTT / 32; ++kb) colp[kb * 32 + l32] = col[kb];
    }
}

// Pass 2 on the 16x16x32 MFMA.  S = Q K^T per 16-key block: a lane holds key
// l%16 of the block and rows 4*(l/16) + [0, 4) of each of the wave's two
// 16-row blocks, so a block needs 8 accumulator registers and the products
// of the next block are issued before this block's exponentials (the two
// streams of one wave overlap on the SIMD).  Each lane sums its 8 rows per
// block; the four 16-lane groups are then reduced in a reduce-scatter, so
// that lane l ends with the totals of NB/4 blocks.
//   qf[rb][ks]: row rbase + 16*rb + l%16, dims 32*ks + 8*(l/16) + [0, 8)
//   l2v[rb][e]: base-2 LSE of row rbase + 16*rb + 4*(l/16) + e
//   koff[ks]:   K fragment of key l%16, dims 32*ks + 8*(l/16) + [0, 8)
template <int D>
__device__ __forceinline__ void load_q16(bf16x8 (&qf)[2][D / 32], const uint16_t* __restrict__ q,
                                         const AttnGeom& g, int b, int h, int rbase, int l16,
                                         int grp) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int r = rbase + rb * 16 + l16;
        const bool ok = r < g.R;
        const uint16_t* qrow =
            q + (((size_t)b * g.Hq + (size_t)h * g.G + (r % g.G)) * g.S + r / g.G) * D;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (ok) v = *(const u32x4*)(qrow + ks * 32 + grp * 8);
            qf[rb][ks] = as_bf16x8(v);
        }
    }
}

template <int D, bool MASKED, int KTT>
__device__ __forceinline__ void colsum_tile16(const uint16_t* Ks, const uint32_t (&koff)[D / 32],
                                              float* colp, const bf16x8 (&qf)[2][D / 32],
                                              const float (&l2v)[2][4], float c, int key0,
                                              int lim, int G, int rbase, int lane) {
    constexpr int NB = KTT / 16;
    static_assert(NB % 4 == 0, "tile of 64-key multiples");
    const int l16 = lane & 15, grp = lane >> 4;
    // software pipeline, one stage per 16-key block: the K fragments of
    // block i+1 are read and its products issued while the weights of block
    // i are formed; the scheduling fence between stages keeps the compiler
    // from hoisting every read of the tile (register pressure)
    auto read_k = [&](int blk, bf16x8 (&kf)[D / 32]) {
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
            kf[ks] = as_bf16x8(lds_read16(Ks, koff[ks] + blk * 16 * D * 2));
    };
    auto products = [&](const bf16x8 (&kf)[D / 32], f32x4 (&s)[2]) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) s[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) s[rb] = mfma16x16x32(qf[rb][ks], kf[ks], s[rb]);
    };
    auto weights = [&](int blk, const f32x4 (&s)[2]) {
        float p[8];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float x = fast_exp2(fmaf(s[rb][e], c, -l2v[rb][e]));
                if (MASKED) {
                    const int key = key0 + blk * 16 + l16;
                    const int r = rbase + rb * 16 + 4 * grp + e;
                    x = (key < lim && key * G <= r) ? x : 0.f;
                }
                p[rb * 4 + e] = x;
            }
        return ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    };
    float part[NB];
    f32x4 sv[2][2];
    {
        bf16x8 kf[D / 32];
        read_k(0, kf);
        products(kf, sv[0]);
    }
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
        __builtin_amdgcn_sched_barrier(0);
        if (blk + 1 < NB) {
            bf16x8 kf[D / 32];
            read_k(blk + 1, kf);
            products(kf, sv[(blk + 1) & 1]);
        }
        part[blk] = weights(blk, sv[blk & 1]);
        // pinned here: the sums are used only after the loop, and would
        // otherwise sink below the later stages' products
        asm volatile("" : "+v"(part[blk]));
    }
    // reduce-scatter over the four 16-lane groups: groups 0,1 keep the first
    // half of the blocks and 2,3 the second, then 0,2 the first quarter of
    // their half and 1,3 the second
    const bool up2 = (grp & 2) != 0, up1 = (grp & 1) != 0;
    float h2[NB / 2];
#pragma unroll
    for (int i = 0; i < NB / 2; ++i) {
        const float keep = up2 ? part[i + NB / 2] : part[i];
        const float send = up2 ? part[i] : part[i + NB / 2];
        h2[i] = keep + xor32(send);
    }
#pragma unroll
    for (int i = 0; i < NB / 4; ++i) {
        const float keep = up1 ? h2[i + NB / 4] : h2[i];
        const float send = up1 ? h2[i] : h2[i + NB / 4];
        const float tot = keep + xor16(send);
        const int blk = (up2 ? NB / 2 : 0) + (up1 ? NB / 4 : 0) + i;
        colp[blk * 16 + l16] = tot;
    }
}

// ---------------------------------------------------------------------------
// pass 2: column sums of P per row tile
// ---------------------------------------------------------------------------
// Pass 2 reads only K, so its tiles can be twice as long as pass 1's at the
// same LDS budget (two workgroups per CU): half the barriers per key.
constexpr int KT2 = 2 * KT;

template <int D>
__global__ __launch_bounds__(NT, 4) void attn_colsum_kernel(
    const AttnGeom g, const int nsplit, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ kn,
    const float* __restrict__ l2, float* __restrict__ wpart) {
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][KT2 * D];
    __shared__ float colp[2][kWaves][KT2];

    int qt, bh, split;
    decode_block(g.n_qt, nsplit, qt, bh, split);
    const int BH = g.B * g.Hkv;
    const int b = bh / g.Hkv, h = bh % g.Hkv;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const int half = lane >> 5, l32 = lane & 31;
    const int W = g.C + g.S;
    const int rbase = qt * kRowsPerBlock + wave * kRowsPerWave;
    const int live = min(RB, max(0, (g.R - rbase + 31) / 32));
    const int l16 = lane & 15, grp = lane >> 4;

    bf16x8 qf[2][D / 32];
    load_q16<D>(qf, q, g, b, h, rbase, l16, grp);
    uint32_t koff[D / 32];
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
        koff[ks] = 2u * (uint32_t)tile_off<D, false>(l16, 4 * ks + grp);
    // base-2 LSE of the rows this lane holds in the S accumulators
    // (padding rows carry +inf, so their weights are 0)
    float l2v[2][4];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            l2v[rb][e] = l2[(size_t)bh * g.rows_pad + rbase + rb * 16 + 4 * grp + e];

    const TileRange tr = tile_range<KT2>(g, qt);
    const int t_begin = (int)((long)split * tr.total / nsplit);
    const int t_end = (int)((long)(split + 1) * tr.total / nsplit);
    const uint16_t* kc_bh = kc + (size_t)bh * g.C * D;
    const uint16_t* kn_bh = kn + (size_t)bh * g.S * D;
    float* wrow = wpart + ((size_t)qt * BH + bh) * W;

    // column sums of tile t are written to wpart after the barrier that ends it
    auto flush = [&](int t, int buf) {
        if (tid < KT2) {
            const bool chunk = t >= tr.n_ct;
            const int key = (chunk ? (t - tr.n_ct) * KT2 : t * KT2) + tid;
            if (key < (chunk ? g.S : g.n)) {
                float tot = colp[buf][0][tid];
#pragma unroll
                for (int w = 1; w < kWaves; ++w) tot += colp[buf][w][tid];
                wrow[chunk ? g.C + key : key] = tot;
            }
        }
    };
    // full cache tiles: scalar-base copies with fixed lane offsets
    const TileCopy<D, false, kWaves, KT2> kcopy(wave, lane);
    const int n_full_tiles = g.n / KT2;
    auto issue = [&](int t, int buf) {
        if (t < n_full_tiles) {
            kcopy.issue(Ks[buf], kc_bh + (size_t)t * KT2 * D, wave);
            return;
        }
        const bool chunk = t >= tr.n_ct;
        const int key0 = chunk ? (t - tr.n_ct) * KT2 : t * KT2;
        issue_tile<D, false, kWaves, KT2>(Ks[buf], chunk ? kn_bh : kc_bh, key0,
                                          chunk ? g.S : g.n, wave, lane);
    };
    if (t_begin < t_end) issue(t_begin, 0);
    wait_tiles();
    __syncthreads();

    // unrolled by the two buffers, so that the LDS tile addresses are
    // constants folded into the reads' offsets
    auto step = [&](auto BUFC, int t) {
        constexpr int buf = decltype(BUFC)::value;
        const bool chunk = t >= tr.n_ct;
        const int key0 = chunk ? (t - tr.n_ct) * KT2 : t * KT2;
        const int lim = chunk ? g.S : g.n;
        if (t + 1 < t_end) issue(t + 1, buf ^ 1);
        if (t > t_begin) flush(t - 1, buf ^ 1);
        if (live == 0) {
            if (half == 0) {
#pragma unroll
                for (int kb = 0; kb < KT2 / 32; ++kb) colp[buf][wave][kb * 32 + l32] = 0.f;
            }
        } else if (chunk ? key0 + KT2 <= g.S && key0 + KT2 - 1 <= rbase / g.G
                         : key0 + KT2 <= g.n) {
            // a full cache tile, or a chunk tile whose keys all exist and
            // precede this wave's first query: no mask
            colsum_tile16<D, false, KT2>(Ks[buf], koff, colp[buf][wave], qf, l2v, g.c, 0, 0, 0,
                                         rbase, lane);
        } else {
            colsum_tile16<D, true, KT2>(Ks[buf], koff, colp[buf][wave], qf, l2v, g.c, key0, lim,
                                        chunk ? g.G : 0, rbase, lane);
        }
        wait_tiles();
        __syncthreads();
    };
    for (int t = t_begin; t < t_end; t += 2) {
        step(BufC<0>{}, t);
        if (t + 1 < t_end) step(BufC<1>{}, t + 1);
    }
    if (t_begin < t_end) flush(t_end - 1, (t_end - 1 - t_begin) & 1);
}

// ---------------------------------------------------------------------------
// 8-bit cache: the cache tiles arrive as int8 codes plus one float scale per
// row and are converted in LDS into the bf16 tiles the blocks above read --
// K codes exactly (integers of at most 7 bits; the K scale multiplies the
// logit), V codes times their scale, rounded to bf16.  Chunk tiles are bf16
// already and are only copied.  Conversion of tile t+1 runs after the MFMA
// work of tile t, so a tile costs one barrier, as in the bf16 kernels.
// ---------------------------------------------------------------------------
struct Q8Cache {
    const int8_t* kc;
    const float* ks;
    const int8_t* vc;
    const float* vs;
};

// Staging area of one tile: K then V, each KT rows of D bf16 (chunk tiles,
// already swizzled for the MFMA reads) or of D int8 codes (cache tiles).
template <int D>
constexpr int stage_bytes() { return 2 * KT * D * 2; }

// Copy (chunk tile) or convert (cache tile) one staged tile into the bf16
// tiles kt / vt, and its K scales into kscale (1 for chunk tiles).  Called by
// all NT_ threads of the workgroup.
template <int D, int NT_>
__device__ __forceinline__ void convert_stage(const uint8_t* stg, const float* sks,
                                              const float* svs, uint16_t* kt, uint16_t* vt,
                                              float* kscale, bool chunk, int tid) {
    if (chunk) {
        constexpr int U = KT * D / 8;   // 16-byte pieces per tensor, layout kept
#pragma unroll
        for (int u0 = 0; u0 < 2 * U; u0 += NT_) {
            const int u = u0 + tid;
            if (u < 2 * U) {
                const bool isv = u >= U;
                const int uu = isv ? u - U : u;
                const u32x4 x = *(const u32x4*)(stg + (isv ? KT * D * 2 : 0) + uu * 16);
                *(u32x4*)((isv ? vt : kt) + uu * 8) = x;
            }
        }
        if (tid < KT) kscale[tid] = 1.f;
    } else {
        constexpr int CPR = D / 16;     // 16 codes per piece
        constexpr int U = KT * CPR;
#pragma unroll
        for (int u0 = 0; u0 < 2 * U; u0 += NT_) {
            const int u = u0 + tid;
            if (u < 2 * U) {
                const bool isv = u >= U;
                const int uu = isv ? u - U : u;
                const int key = uu / CPR, c = uu % CPR;
                const u32x4 x = *(const u32x4*)(stg + (isv ? KT * D : 0) + key * D + c * 16);
                u32x4 lo, hi;
                if (isv) {
                    i8x16_to_bf16_scaled(x, svs[key], lo, hi);
                    *(u32x4*)(vt + tile_off<D, true>(key, 2 * c)) = lo;
                    *(u32x4*)(vt + tile_off<D, true>(key, 2 * c + 1)) = hi;
                } else {
                    i8x16_to_bf16(x, lo, hi);
                    *(u32x4*)(kt + tile_off<D, false>(key, 2 * c)) = lo;
                    *(u32x4*)(kt + tile_off<D, false>(key, 2 * c + 1)) = hi;
                }
            }
        }
        if (tid < KT) kscale[tid] = sks[tid];
    }
}

// DMA of one tile into a staging area: int8 rows + scales for cache tiles,
// swizzled bf16 rows for chunk tiles.
template <int D, int NW>
__device__ __forceinline__ void issue_stage(uint8_t* stg, float* sks, float* svs,
                                            const Q8Cache& qc, const uint16_t* kn_bh,
                                            const uint16_t* vn_bh, size_t cache_row0,
                                            bool chunk, int key0, int lim, int wave, int lane) {
    if (chunk) {
        issue_tile<D, false, NW>((uint16_t*)stg, kn_bh, key0, lim, wave, lane);
        issue_tile<D, true, NW>((uint16_t*)(stg + KT * D * 2), vn_bh, key0, lim, wave, lane);
    } else {
        issue_tile_i8<D, NW>(stg, qc.kc + cache_row0 * D, key0, lim, wave, lane);
        issue_tile_i8<D, NW>(stg + KT * D, qc.vc + cache_row0 * D, key0, lim, wave, lane);
        issue_scales<0, NW - 1>(sks, svs, qc.ks + cache_row0, qc.vs + cache_row0, key0, lim,
                                wave, lane);
    }
}

// pass 1 over an 8-bit cache
template <int D>
__global__ __launch_bounds__(NT, 1) void attn_fwd_q8_kernel(
    const AttnGeom g, const int nsplit, const uint16_t* __restrict__ q, const Q8Cache qc,
    const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn,
    float* __restrict__ o_part, float* __restrict__ ml_part) {
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][KT * D];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[2][KT * D];
    __shared__ __attribute__((aligned(16))) uint8_t stg[2][stage_bytes<D>()];
    __shared__ __attribute__((aligned(16))) float ssc[2][2][KT];
    __shared__ __attribute__((aligned(16))) float ksc[2][KT];

    int qt, bh, split;
    decode_block(g.n_qt, nsplit, qt, bh, split);
    const int BH = g.B * g.Hkv;
    const int b = bh / g.Hkv, h = bh % g.Hkv;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, l32 = lane & 31;
    const int rbase = qt * kRowsPerBlock + wave * kRowsPerWave;
    const int live = min(RB, max(0, (g.R - rbase + 31) / 32));

    bf16x8 qf[RB][D / 16];
    load_q<D>(qf, q, g, b, h, rbase, l32, half);
    const LdsOffsets<D> off(lane);

    const TileRange tr = tile_range(g, qt);
    const int t_begin = (int)((long)split * tr.total / nsplit);
    const int t_end = (int)((long)(split + 1) * tr.total / nsplit);
    const uint16_t* kn_bh = kn + (size_t)bh * g.S * D;
    const uint16_t* vn_bh = vn + (size_t)bh * g.S * D;

    float m_ref[RB], m_seen[RB], l_acc[RB], lt_acc[RB];
    f32x16 o_acc[RB][D / 32];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) m_seen[rb] = -INFINITY;

    auto issue = [&](int t, int sb) {
        const bool chunk = t >= tr.n_ct;
        const int key0 = chunk ? (t - tr.n_ct) * KT : t * KT;
        issue_stage<D, kWaves>(stg[sb], ssc[sb][0], ssc[sb][1], qc, kn_bh, vn_bh,
                               (size_t)bh * g.C, chunk, key0, chunk ? g.S : g.n, wave, lane);
    };
    auto convert = [&](int t, int sb) {
        convert_stage<D, NT>(stg[sb], ssc[sb][0], ssc[sb][1], Ks[sb], Vs[sb], ksc[sb],
                             t >= tr.n_ct, tid);
    };

    // One sweep over this split's tiles (TRACK: with the tile max, as in
    // the tracked sweeps of attn_fwd_kernel).
    auto sweep_tiles = [&](auto TRC, bool& overflow) {
        constexpr bool TRACK = decltype(TRC)::value;
        // prologue: tile t_begin converted, tile t_begin+1 staged
        if (t_begin < t_end) {
            issue(t_begin, 0);
            wait_tiles();
            __syncthreads();
            convert(t_begin, 0);
        }
        if (t_begin + 1 < t_end) issue(t_begin + 1, 1);
        wait_tiles();
        __syncthreads();

        const int n_full = g.n / KT;
        const int t_mid = max(t_begin, min(t_end, n_full));
        // buffer b holds tile t (converted) and, until this iteration's
        // issue, the staging of tile t that was converted last iteration
        for (int t = t_begin; t < t_mid; ++t) {
            const int bb = (t - t_begin) & 1;
            if (t + 2 < t_end) issue(t + 2, bb);
            if (live > 0)
                fwd_tile<D, false, true, TRACK>(Ks[bb], Vs[bb], off, qf, o_acc, m_ref, m_seen,
                                                overflow, l_acc, lt_acc, g.c, 0, 0, false, 0,
                                                rbase, lane, ksc[bb]);
            if (t + 1 < t_end) convert(t + 1, bb ^ 1);
            wait_tiles();
            __syncthreads();
        }
        for (int t = t_mid; t < t_end; ++t) {
            const int bb = (t - t_begin) & 1;
            const bool chunk = t >= tr.n_ct;
            const int key0 = chunk ? (t - tr.n_ct) * KT : t * KT;
            const int lim = chunk ? g.S : g.n;
            if (t + 2 < t_end) issue(t + 2, bb);
            if (live > 0)
                fwd_tile<D, true, true, TRACK>(Ks[bb], Vs[bb], off, qf, o_acc, m_ref, m_seen,
                                               overflow, l_acc, lt_acc, g.c, key0, lim, chunk,
                                               g.G, rbase, lane, ksc[bb]);
            if (t + 1 < t_end) convert(t + 1, bb ^ 1);
            wait_tiles();
            __syncthreads();
        }
    };
    auto zero_state = [&]() {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            l_acc[rb] = 0.f;
            lt_acc[rb] = 0.f;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) o_acc[rb][db][v] = 0.f;
        }
    };

    // Main sweep: each row's reference is its own base-2 logit against its
    // chunk key (bf16 in both caches), as in attn_fwd_kernel; row sums above
    // 2^kHeadroom send the workgroup to the tracked sweeps.
    {
        bool overflow = false;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int r = rbase + rb * 32 + l32;
            const bool ok = r < g.R;
            const uint16_t* kself = kn_bh + (size_t)(ok ? r / g.G : 0) * D + 8 * half;
            float dot = 0.f;
#pragma unroll
            for (int k16 = 0; k16 < D / 16; ++k16) {
                const bf16x8 kv = as_bf16x8(*(const u32x4*)(kself + 16 * k16));
#pragma unroll
                for (int e = 0; e < 8; ++e) dot = fmaf((float)qf[rb][k16][e], (float)kv[e], dot);
            }
            dot += xor32(dot);
            m_ref[rb] = ok ? dot * g.c : 0.f;
        }
        zero_state();
        sweep_tiles(TrackC<false>{}, overflow);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) overflow |= !(l_acc[rb] <= kSumLimit);
        if (!__syncthreads_or(overflow)) goto store;
    }
    // tracked sweeps (rare): first-tile reference with every tile max
    // recorded, then, if still overshot, the exact row max
    for (int sweep = 0; sweep < 2; ++sweep) {
        bool overflow = false;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) m_ref[rb] = (sweep == 0) ? -INFINITY : m_seen[rb];
        zero_state();
        sweep_tiles(TrackC<true>{}, overflow);
        if (!__syncthreads_or(overflow)) break;
    }

store:
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const float l = l_acc[rb] + xor32(l_acc[rb]);
        const float lt = lt_acc[rb] + xor32(lt_acc[rb]);
        const int r = rbase + rb * 32 + l32;
        if (r >= g.R) continue;
        const size_t prow = ((size_t)split * BH + bh) * g.rows_pad + r;
        if (half == 0) *(f32x4*)(ml_part + prow * 4) = f32x4{m_ref[rb], l, lt, 0.f};
        float* orow = o_part + prow * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const f32x4 v4 = {o_acc[rb][db][4 * gq + 0], o_acc[rb][db][4 * gq + 1],
                                  o_acc[rb][db][4 * gq + 2], o_acc[rb][db][4 * gq + 3]};
                *(f32x4*)(orow + db * 32 + 8 * gq + 4 * half) = v4;
            }
    }
}

// pass 2 over an 8-bit cache (K only)
template <int D>
__global__ __launch_bounds__(NT, 2) void attn_colsum_q8_kernel(
    const AttnGeom g, const int nsplit, const uint16_t* __restrict__ q, const Q8Cache qc,
    const uint16_t* __restrict__ kn, const float* __restrict__ l2, float* __restrict__ wpart) {
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][KT * D];
    __shared__ __attribute__((aligned(16))) uint8_t stg[2][KT * D * 2];
    __shared__ __attribute__((aligned(16))) float ssc[2][KT];
    __shared__ __attribute__((aligned(16))) float ksc[2][KT];
    __shared__ float colp[2][kWaves][KT];

    int qt, bh, split;
    decode_block(g.n_qt, nsplit, qt, bh, split);
    const int BH = g.B * g.Hkv;
    const int b = bh / g.Hkv, h = bh % g.Hkv;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, l32 = lane & 31;
    const int W = g.C + g.S;
    const int rbase = qt * kRowsPerBlock + wave * kRowsPerWave;
    const int live = min(RB, max(0, (g.R - rbase + 31) / 32));

    bf16x8 qf[RB][D / 16];
    load_q<D>(qf, q, g, b, h, rbase, l32, half);
    const LdsOffsets<D> off(lane);
    float l2v[RB][16];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
            l2v[rb][v] = l2[(size_t)bh * g.rows_pad + rbase + rb * 32 + acc_row(v, half)];

    const TileRange tr = tile_range(g, qt);
    const int t_begin = (int)((long)split * tr.total / nsplit);
    const int t_end = (int)((long)(split + 1) * tr.total / nsplit);
    const uint16_t* kn_bh = kn + (size_t)bh * g.S * D;
    const size_t row0 = (size_t)bh * g.C;
    float* wrow = wpart + ((size_t)qt * BH + bh) * W;

    auto flush = [&](int t, int buf) {
        if (tid < KT) {
            const bool chunk = t >= tr.n_ct;
            const int key = (chunk ? (t - tr.n_ct) * KT : t * KT) + tid;
            if (key < (chunk ? g.S : g.n)) {
                float tot = colp[buf][0][tid];
#pragma unroll
                for (int w = 1; w < kWaves; ++w) tot += colp[buf][w][tid];
                wrow[chunk ? g.C + key : key] = tot;
            }
        }
    };
    auto issue = [&](int t, int sb) {
        const bool chunk = t >= tr.n_ct;
        const int key0 = chunk ? (t - tr.n_ct) * KT : t * KT;
        if (chunk) {
            issue_tile<D, false>((uint16_t*)stg[sb], kn_bh, key0, g.S, wave, lane);
        } else {
            issue_tile_i8<D, kWaves>(stg[sb], qc.kc + row0 * D, key0, g.n, wave, lane);
            issue_scales<0, -1>(ssc[sb], nullptr, qc.ks + row0, nullptr, key0, g.n, wave, lane);
        }
    };
    // K only: the V half of convert_stage is skipped by converting a
    // K-sized "tile pair" whose V part is never read
    auto convert = [&](int t, int sb) {
        const bool chunk = t >= tr.n_ct;
        if (chunk) {
            constexpr int U = KT * D / 8;
#pragma unroll
            for (int u0 = 0; u0 < U; u0 += NT) {
                const int u = u0 + tid;
                if (u < U) *(u32x4*)(Ks[sb] + u * 8) = *(const u32x4*)(stg[sb] + u * 16);
            }
            if (tid < KT) ksc[sb][tid] = 1.f;
        } else {
            constexpr int CPR = D / 16;
            constexpr int U = KT * CPR;
#pragma unroll
            for (int u0 = 0; u0 < U; u0 += NT) {
                const int u = u0 + tid;
                if (u < U) {
                    const int key = u / CPR, c = u % CPR;
                    u32x4 lo, hi;
                    i8x16_to_bf16(*(const u32x4*)(stg[sb] + key * D + c * 16), lo, hi);
                    *(u32x4*)(Ks[sb] + tile_off<D, false>(key, 2 * c)) = lo;
                    *(u32x4*)(Ks[sb] + tile_off<D, false>(key, 2 * c + 1)) = hi;
                }
            }
            if (tid < KT) ksc[sb][tid] = ssc[sb][tid];
        }
    };

    if (t_begin < t_end) {
        issue(t_begin, 0);
        wait_tiles();
        __syncthreads();
        convert(t_begin, 0);
    }
    if (t_begin + 1 < t_end) issue(t_begin + 1, 1);
    wait_tiles();
    __syncthreads();

    for (int t = t_begin; t < t_end; ++t) {
        const int bb = (t - t_begin) & 1;
        const bool chunk = t >= tr.n_ct;
        const int key0 = chunk ? (t - tr.n_ct) * KT : t * KT;
        const int lim = chunk ? g.S : g.n;
        if (t + 2 < t_end) issue(t + 2, bb);
        if (t > t_begin) flush(t - 1, bb ^ 1);
        if (live == 0) {
            if (half == 0) {
                colp[bb][wave][l32] = 0.f;
                colp[bb][wave][32 + l32] = 0.f;
            }
        } else if (!chunk && key0 + KT <= g.n) {
            colsum_tile<D, false, true>(Ks[bb], off, colp[bb][wave], qf, l2v, g.c, 0, 0, 0,
                                        rbase, l32, half, ksc[bb]);
        } else {
            colsum_tile<D, true, true>(Ks[bb], off, colp[bb][wave], qf, l2v, g.c, key0, lim,
                                       chunk ? g.G : 0, rbase, l32, half, ksc[bb]);
        }
        if (t + 1 < t_end) convert(t + 1, bb ^ 1);
        wait_tiles();
        __syncthreads();
    }
    if (t_begin < t_end) flush(t_end - 1, (t_end - 1 - t_begin) & 1);
}

// few-row pass 1 over an 8-bit cache.  The waves take different 32-key
// blocks of each tile.  Both K and V are read straight from the staged int8
// tiles (K as row fragments, V through the 8-bit transposed read; each with
// its own chunk swizzle) and converted exactly in registers; the K scale
// multiplies the logit and the V scale multiplies P.  Without bf16 copies the
// workgroup needs only its staging buffers, so three fit on a CU.  Every block
// runs the masked variant, so no branch separates accumulator updates.
constexpr int STQ = 3;                 // staging buffers: 2 cache tiles in flight

template <int PT>
__device__ __forceinline__ void wait_later(int later) {
    if (later >= 3)
        wait_vm<3 * PT>();
    else if (later == 2)
        wait_vm<2 * PT>();
    else if (later == 1)
        wait_vm<PT>();
    else
        wait_tiles();
}

// One wave per SIMD is what the kernel holds: at D = 128 its registers with
// the accumulators exceed 256 (a higher occupancy target only made the
// compiler spill at D = 64).
template <int D>
__global__ __launch_bounds__(NT_S, 1) void attn_fwd_small_q8_kernel(
    const AttnGeom g, const int nsplit, const uint16_t* __restrict__ q, const Q8Cache qc,
    const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn,
    float* __restrict__ o_part, float* __restrict__ ml_part, float* __restrict__ logits) {
    __shared__ __attribute__((aligned(16))) uint8_t stg[STQ][2 * KT * D];
    // per stage and wave: the K scales then the V scales of its 32 keys
    __shared__ __attribute__((aligned(16))) float ssc[STQ][NW_S][64];
    // per wave: the base-2 logits of its key blocks of up to Q8_LGS_ROWS / R
    // consecutive full tiles, [tile][row][key] (R <= Q8_LGS_ROWS)
    constexpr int Q8_LGS_ROWS = 8;
    __shared__ __attribute__((aligned(16))) float lgs[NW_S][Q8_LGS_ROWS * 32];
    // this wave's copy instructions per cache tile: K and V codes of its 32
    // rows, one 4-byte copy of its 64 scales
    constexpr int PER_TILE = 2 * (32 * D / 16 / 64) + 1;
    static_assert(STQ - 2 <= 3, "wait_later covers up to three later tiles");
    static_assert(STQ * 2 * KT * D >= 2 * KT * D * 2, "the bf16 chunk tile fits the staging");

    int qt, bh, split;
    decode_block(1, nsplit, qt, bh, split);
    const int BH = g.B * g.Hkv;
    const int b = bh / g.Hkv, h = bh % g.Hkv;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, half = lane >> 5;

    bf16x8 qf[RB][D / 16];
    load_q<D>(qf, q, g, b, h, 0, l32, half);
    const LdsOffsets<D> off(lane);
    const int WL = logit_stride(g);
    float* lg_row = (l32 < g.R) ? logits + ((size_t)bh * g.R + l32) * WL : nullptr;
    float* const logits_bh = logits + (size_t)bh * g.R * WL;

    const TileRange tr = tile_range(g, 0);
    const int t_begin = (int)((long)split * tr.total / nsplit);
    const int t_end = (int)((long)(split + 1) * tr.total / nsplit);
    const int c_end = min(t_end, tr.n_ct);       // cache tiles of this split: [t_begin, c_end)
    const size_t row0 = (size_t)bh * g.C;
    const uint16_t* kn_bh = kn + (size_t)bh * g.S * D;
    const uint16_t* vn_bh = vn + (size_t)bh * g.S * D;

    float m_ref[RB], m_seen[RB], l_acc[RB], lt_acc[RB];
    f32x16 o_acc[RB][D / 32];
    m_seen[0] = -INFINITY;
    // Each wave copies the codes of the 32 rows of its own key block of a
    // tile, and their K and V scales, and reads only those: the waves share
    // no tile data and need no barrier per tile.  A stage is rewritten by the
    // wave that read it, after its reads of it have returned.
    auto issue = [&](int t, int sb) {
        const int k0 = t * KT + wave * 32;
        // rows read once: non-temporal copies
        issue_tile_i8<D, 1, 32, 1, true>(stg[sb] + wave * 32 * D, qc.kc + row0 * D, k0, g.n, 0,
                                         lane);
        issue_tile_i8<D, 1, 32, 2, true>(stg[sb] + KT * D + wave * 32 * D, qc.vc + row0 * D, k0,
                                         g.n, 0, lane);
        const int gkey = min(k0 + l32, g.n - 1);
        dma4((half ? qc.vs : qc.ks) + row0 + gkey,
             __builtin_amdgcn_readfirstlane(lds_addr(&ssc[sb][wave][0])));
    };
    // scale pointers as fwd_block indexes them: element lkb*32 + j, lkb = wave
    auto kscale = [&](int sb) { return &ssc[sb][0][0] + wave * 32; };
    auto vscale = [&](int sb) { return &ssc[sb][0][0] + wave * 32 + 32; };

    // write_logits (wave-uniform): the main sweep stores the logits
    auto sweep_tiles = [&](auto TRC, bool& overflow, bool write_logits) {
        constexpr bool TRACK = decltype(TRC)::value;
        float* const lg = write_logits ? lg_row : nullptr;
        const bool staged = write_logits && g.R <= Q8_LGS_ROWS;
        const int tf = staged ? Q8_LGS_ROWS / g.R : 1;
        int nb = 0, b_key0 = 0;
        auto flush = [&]() {
            const int per = g.R * 8;   // 16-byte pieces per tile
            for (int cix = lane; cix < nb * per; cix += 64) {
                const int slot = cix / per, rem = cix - slot * per;
                const int row = rem >> 3, k4 = rem & 7;
                const f32x4 v = *(const f32x4*)&lgs[wave][(slot * g.R + row) * 32 + 4 * k4];
                *(f32x4*)(logits_bh + (size_t)row * WL + b_key0 + slot * KT + wave * 32 +
                          4 * k4) = v;
            }
            nb = 0;
        };
        for (int i = 0; i < STQ - 1 && t_begin + i < c_end; ++i) issue(t_begin + i, i);
        wait_later<PER_TILE>(min(STQ - 2, c_end - 1 - t_begin));
        for (int t = t_begin; t < c_end; ++t) {
            const int sb = (t - t_begin) % STQ;
            const int key0 = t * KT;
            // the stage of tile t+2 was last read, by this wave, for tile t-1
            if (t + STQ - 1 < c_end) issue(t + STQ - 1, (sb + STQ - 1) % STQ);
            if (key0 + KT <= g.n) {
                if (nb == 0) b_key0 = key0;
                float* const stage =
                    (staged && l32 < g.R) ? &lgs[wave][nb * g.R * 32] : nullptr;
                fwd_block<D, false, true, true, true, TRACK>(
                    nullptr, nullptr, off, qf, o_acc, m_ref, m_seen, overflow, l_acc, lt_acc, g.c,
                    wave, key0, g.n, false, g.G, 0, lane, staged ? nullptr : lg, key0, wave,
                    kscale(sb), stg[sb], stg[sb] + KT * D, vscale(sb), stage);
                if (staged && ++nb == tf) flush();
            } else {
                if (nb > 0) flush();
                fwd_block<D, true, true, true, true, TRACK>(
                    nullptr, nullptr, off, qf, o_acc, m_ref, m_seen, overflow, l_acc, lt_acc, g.c,
                    wave, key0, g.n, false, g.G, 0, lane, lg, key0, wave, kscale(sb), stg[sb],
                    stg[sb] + KT * D, vscale(sb));
            }
            // this wave's copies of tile t+1 must have landed; a tile issued
            // after it may stay in flight
            wait_later<PER_TILE>(min(STQ - 2, c_end - 1 - (t + 1)));
        }
        if (nb > 0) flush();
        if (t_end > tr.n_ct) {   // the chunk tile (S <= 32 here: a single tile)
            const int key0 = (t_end - 1 - tr.n_ct) * KT;
            // bf16 K and V tiles in the staging area (K in the space of
            // buffer 0, V in that of buffer 1); each wave writes its own 32
            // rows straight from the chunk, after every wave is done with the
            // cache tiles there; K scales 1
            __syncthreads();
            uint16_t* mk = (uint16_t*)stg[0];
            uint16_t* mv = (uint16_t*)stg[1];
            constexpr int CPR = D / 8;
#pragma unroll
            for (int u0 = 0; u0 < 32 * CPR; u0 += 64) {
                const int u = u0 + lane;
                const int r = wave * 32 + u / CPR, cc = u % CPR;
                const int key = min(key0 + r, g.S - 1);
                *(u32x4*)(mk + tile_off<D, false>(r, cc)) =
                    *(const u32x4*)(kn_bh + (size_t)key * D + cc * 8);
                *(u32x4*)(mv + tile_off<D, true>(r, cc)) =
                    *(const u32x4*)(vn_bh + (size_t)key * D + cc * 8);
            }
            if (lane < 32) ssc[0][wave][lane] = 1.f;
            fwd_block<D, true, true, false, false, TRACK>(
                mk, mv, off, qf, o_acc, m_ref, m_seen, overflow, l_acc, lt_acc, g.c, wave, key0,
                g.S, true, g.G, 0, lane, lg, g.C + key0, wave, kscale(0));
            // the cache blocks set lt = l; this bf16 block adds its rounded weights
        }
    };
    auto zero_state = [&]() {
        l_acc[0] = 0.f;
        lt_acc[0] = 0.f;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) o_acc[0][db][v] = 0.f;
    };

    // Main sweep: each row's reference is its own base-2 logit against its
    // diagonal chunk key (bf16), as in attn_fwd_kernel; row sums above
    // 2^kHeadroom send the workgroup to the tracked sweeps.
    {
        bool overflow = false;
        const int r = l32;
        const bool ok = r < g.R;
        const uint16_t* kself = kn_bh + (size_t)(ok ? r / g.G : 0) * D + 8 * half;
        float dot = 0.f;
#pragma unroll
        for (int k16 = 0; k16 < D / 16; ++k16) {
            const bf16x8 kv = as_bf16x8(*(const u32x4*)(kself + 16 * k16));
#pragma unroll
            for (int e = 0; e < 8; ++e) dot = fmaf((float)qf[0][k16][e], (float)kv[e], dot);
        }
        dot += xor32(dot);
        m_ref[0] = ok ? dot * g.c : 0.f;
        zero_state();
        sweep_tiles(TrackC<false>{}, overflow, true);
        overflow |= !(l_acc[0] <= kSumLimit);
        if (!__syncthreads_or(overflow)) goto merge;
    }
    // tracked sweeps (rare): first-tile reference with every tile max
    // recorded, then, if still overshot, the exact row max
    for (int sweep = 0; sweep < 2; ++sweep) {
        bool overflow = false;
        m_ref[0] = (sweep == 0) ? -INFINITY : m_seen[0];
        zero_state();
        sweep_tiles(TrackC<true>{}, overflow, false);
        if (!__syncthreads_or(overflow)) break;
    }

merge:
    // merge the waves' (m, l, lt, O) through LDS (the staging buffers are free)
    const float l = l_acc[0] + xor32(l_acc[0]);
    const float lt = lt_acc[0] + xor32(lt_acc[0]);
    constexpr int XS = D / 2 + 4;
    static_assert(NW_S * 64 * XS * 4 <= (int)sizeof(stg), "merge area exceeds the staging");
    float* xch = (float*)&stg[0][0];
    float* mine = xch + ((size_t)wave * 64 + lane) * XS;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) mine[db * 16 + v] = o_acc[0][db][v];
    mine[D / 2 + 0] = m_ref[0];
    mine[D / 2 + 1] = l;
    mine[D / 2 + 2] = lt;
    __syncthreads();
    if (wave != 0) return;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW_S; ++w) M = fmaxf(M, xch[((size_t)w * 64 + lane) * XS + D / 2]);
    float wt[NW_S], L = 0.f, Lt = 0.f;
#pragma unroll
    for (int w = 0; w < NW_S; ++w) {
        const float* o = xch + ((size_t)w * 64 + lane) * XS;
        wt[w] = (M == -INFINITY) ? 0.f : fast_exp2(o[D / 2] - M);
        L += wt[w] * o[D / 2 + 1];
        Lt += wt[w] * o[D / 2 + 2];
    }
    const int r = l32;
    if (r >= g.R) return;
    const size_t prow = ((size_t)split * BH + bh) * g.rows_pad + r;
    if (half == 0) *(f32x4*)(ml_part + prow * 4) = f32x4{M, L, Lt, 0.f};
    float* orow = o_part + prow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < NW_S; ++w) {
                const float* o = xch + ((size_t)w * 64 + lane) * XS + db * 16 + 4 * gq;
                acc += wt[w] * f32x4{o[0], o[1], o[2], o[3]};
            }
            *(f32x4*)(orow + db * 32 + 8 * gq + 4 * half) = acc;
        }
}

// ---------------------------------------------------------------------------
// pass 1 over the 8-bit cache with at most 16 rows (e.g. one decode token per
// sequence): the 16-row pass of attn_fwd_few_kernel with the codes read
// straight from LDS and converted in registers.
// ---------------------------------------------------------------------------
// One 32-key block of a cache tile for one wave.  kt / vt hold the K / V
// codes of the wave's 32 rows (swizzled by i8_swz_k16 / i8_swz_v16), ksc /
// vsc their scales.  As fwd_block16, with the K fragments converted exactly
// from the codes and each logit multiplied by its key's scale; P times the
// key's V scale is rounded to bf16 for the PV product (V^T from the 8-bit
// transposed read, in the lanes' key order), and O is normalised by the exact
// row sum (lt = l), as in the 32-row 8-bit pass.  MASKED: the last partial
// cache tile.
template <int D, bool MASKED, bool TRACK>
__device__ __forceinline__ void fwd_block16_q8(const uint8_t* kt, const uint8_t* vt,
                                               const float* ksc, const float* vsc,
                                               const bf16x8 (&qf)[D / 32],
                                               f32x4 (&o_acc)[D / 16], float& m_ref,
                                               float& m_seen, bool& overflow, float& l_acc,
                                               float& lt_acc, float c, int kb, int key0, int lim,
                                               int lane, float* lg_row, int col0,
                                               float* lg_stage) {
    const int l16 = lane & 15, g = lane >> 4;
    // S^T of the two 16-key halves (key 16*h + l16 of the block is the A row),
    // each over two chains of k-steps
    f32x4 s[2];
    {
        f32x4 acc[2][2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int p = 0; p < 2; ++p) acc[h][p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int key = 16 * h + l16;
                const int ch = 2 * ks + (g >> 1);   // dims 32*ks + 8*g + [0, 8)
                const bf16x8 kf = i8x8_to_bf16(*(const uint2*)(
                    kt + key * D + 16 * (ch ^ i8_swz_k16<D>(key)) + 8 * (g & 1)));
                acc[h][ks & 1] = mfma16x16x32(kf, qf[ks], acc[h][ks & 1]);
            }
#pragma unroll
        for (int h = 0; h < 2; ++h) s[h] = acc[h][0] + acc[h][1];
    }
    // element e of s[h] is key 16*h + 4*g + e of the block: its K scale
    // multiplies the logit, its V scale the weight
    f32x4 vs4[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        s[h] = s[h] * *(const f32x4*)(ksc + 16 * h + 4 * g);
        vs4[h] = *(const f32x4*)(vsc + 16 * h + 4 * g);
    }
    if (MASKED) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int key = key0 + kb * 32 + 16 * h + 4 * g + e;
                s[h][e] = key < lim ? s[h][e] : -INFINITY;
            }
        if (lg_row) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int kl = kb * 32 + 16 * h + 4 * g + e;
                    if (key0 + kl < lim) lg_row[col0 + kl] = s[h][e] * c;
                }
        }
    } else if (lg_stage) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
            *(f32x4*)(lg_stage + l16 * 32 + 16 * h + 4 * g) = s[h] * c;
    }
    if constexpr (TRACK) {   // as in fwd_block16
        float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                         fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
        mx = fmaxf(mx, xor16(mx));
        mx = fmaxf(mx, xor32(mx));
        const float mt = mx * c;
        m_seen = fmaxf(m_seen, mt);
        m_ref = (m_ref == -INFINITY) ? mt : m_ref;
        overflow |= mt > m_ref + kHeadroom;
    }
    const float m_use = (!TRACK || m_ref != -INFINITY) ? m_ref : 0.f;
    bf16x8 pf;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float p = fast_exp2(fmaf(s[h][e], c, -m_use));
            l_acc += p;
            pf[4 * h + e] = (__bf16)(p * vs4[h][e]);
        }
    lt_acc = l_acc;
    // O^T += V^T P^T: input lane j of a 16-lane group points at row vkey
    // (b = j / 2: 4*g + b, or 16 + 4*g + b - 4) and half j % 2 of chunk db;
    // output lane i then holds dims 16*db + i of those 8 rows as its k-values
    const int b8 = l16 >> 1;
    const int vkey = b8 < 4 ? 4 * g + b8 : 16 + 4 * g + b8 - 4;
    const uint8_t* vrow = vt + vkey * D + 8 * (l16 & 1);
    const int vsw = i8_swz_v16<D>(vkey);
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
        const bf16x8 vf = i8x8_to_bf16(lds_read_tr8(vrow + 16 * (db ^ vsw)));
        o_acc[db] = mfma16x16x32(vf, pf, o_acc[db]);
    }
}

// Per-wave stages of the 16-row 8-bit pass (three tiles in flight while one
// is read; a stage of one wave is 8 KiB at D = 128, so two workgroups fit a CU)
constexpr int STAGES_FQ = 4;

template <int D>
__global__ __launch_bounds__(NT_S, 1) void attn_fwd_few_q8_kernel(
    const AttnGeom g, const int nsplit, const uint16_t* __restrict__ q, const Q8Cache qc,
    const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn,
    float* __restrict__ o_part, float* __restrict__ ml_part, float* __restrict__ logits) {
    // per wave and stage: the K codes then the V codes of its 32 rows; the
    // first two stages of a wave take its bf16 chunk tile at the end
    __shared__ __attribute__((aligned(16))) uint8_t stg[NW_S][STAGES_FQ][2 * 32 * D];
    // per wave and stage: the K scales then the V scales of its 32 rows
    __shared__ __attribute__((aligned(16))) float ssc[NW_S][STAGES_FQ][64];
    // per wave: the base-2 logits of its key blocks of up to LGS_ROWS / R
    // consecutive full tiles, [tile][row][key], written out together
    constexpr int LGS_ROWS = 32;
    __shared__ __attribute__((aligned(16))) float lgs[NW_S][LGS_ROWS * 32];
    constexpr int PER_TILE = 2 * (32 * D / 16 / 64) + 1;   // this wave's copies per tile
    static_assert(STAGES_FQ >= 2 && STAGES_FQ - 2 <= 3, "waits cover up to three later tiles");

    int qt, bh, split;
    decode_block(1, nsplit, qt, bh, split);
    const int BH = g.B * g.Hkv;
    const int b = bh / g.Hkv, h = bh % g.Hkv;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const int l16 = lane & 15, grp = lane >> 4;

    const TileRange tr = tile_range(g, 0);
    const int t_begin = (int)((long)split * tr.total / nsplit);
    const int t_end = (int)((long)(split + 1) * tr.total / nsplit);
    const int c_end = min(t_end, tr.n_ct);   // cache tiles of this split: [t_begin, c_end)
    const size_t row0 = (size_t)bh * g.C;
    const uint16_t* kn_bh = kn + (size_t)bh * g.S * D;
    const uint16_t* vn_bh = vn + (size_t)bh * g.S * D;

    // Each wave copies the codes and scales of the 32 rows of its own key
    // block of a tile and reads only those (no barrier per tile); rows past
    // n re-read row n - 1 and are masked.  Rows read once: non-temporal.
    auto issue = [&](int t, int sb) {
        const int k0 = t * KT + wave * 32;
        uint8_t* st = stg[wave][sb];
        issue_tile_i8<D, 1, 32, 3, true>(st, qc.kc + row0 * D, k0, g.n, 0, lane);
        issue_tile_i8<D, 1, 32, 4, true>(st + 32 * D, qc.vc + row0 * D, k0, g.n, 0, lane);
        const int gkey = min(k0 + (lane & 31), g.n - 1);
        dma4((lane >= 32 ? qc.vs : qc.ks) + row0 + gkey,
             __builtin_amdgcn_readfirstlane(lds_addr(&ssc[wave][sb][0])));
    };
    auto prologue = [&]() {
        for (int i = 0; i < STAGES_FQ - 1 && t_begin + i < c_end; ++i) issue(t_begin + i, i);
    };
    // waits until the copies of all but the `later` tiles issued last landed
    auto wait_later_q = [&](int later) {
        if (later >= 3)
            wait_vm<3 * PER_TILE>();
        else if (later == 2)
            wait_vm<2 * PER_TILE>();
        else if (later == 1)
            wait_vm<PER_TILE>();
        else
            wait_tiles();
    };
    // the main sweep's first copies go out before the query loads
    prologue();

    // Q fragments (B operand of S^T = K Q^T): row l16, dims 32*ks + 8*grp + [0, 8)
    const bool row_ok = l16 < g.R;
    bf16x8 qf[D / 32];
    {
        const uint16_t* qrow =
            q + (((size_t)b * g.Hq + (size_t)h * g.G + (l16 % g.G)) * g.S + l16 / g.G) * D +
            8 * grp;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (row_ok) v = *(const u32x4*)(qrow + 32 * ks);
            qf[ks] = as_bf16x8(v);
        }
    }
    const LdsOffsets16<D> off(lane);   // the bf16 chunk tile
    float* lg_row = row_ok ? logits + ((size_t)bh * g.R + l16) * logit_stride(g) : nullptr;
    float* const logits_bh = logits + (size_t)bh * g.R * logit_stride(g);

    float m_ref = 0.f, m_seen = -INFINITY, l_acc = 0.f, lt_acc = 0.f;
    f32x4 o_acc[D / 16];
    auto zero_state = [&]() {
        l_acc = 0.f;
        lt_acc = 0.f;
#pragma unroll
        for (int db = 0; db < D / 16; ++db) o_acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    // write_logits (wave-uniform): the main sweep stores the logits, the
    // tracked sweeps do not; issued: the prologue's copies are in flight
    auto sweep_tiles = [&](auto TRC, bool& overflow, bool write_logits, bool issued) {
        constexpr bool TRACK = decltype(TRC)::value;
        float* const lg = write_logits ? lg_row : nullptr;
        const int tf = LGS_ROWS / g.R;
        int nb = 0, b_key0 = 0;
        auto flush = [&]() {
            const int per = g.R * 8;   // 16-byte pieces per tile
            for (int cix = lane; cix < nb * per; cix += 64) {
                const int slot = cix / per, rem = cix - slot * per;
                const int row = rem >> 3, k4 = rem & 7;
                const f32x4 v = *(const f32x4*)&lgs[wave][(slot * g.R + row) * 32 + 4 * k4];
                *(f32x4*)(logits_bh + (size_t)row * logit_stride(g) + b_key0 + slot * KT +
                          wave * 32 + 4 * k4) = v;
            }
            nb = 0;
        };
        if (!issued) prologue();
        wait_later_q(min(STAGES_FQ - 2, c_end - 1 - t_begin));
        for (int t = t_begin; t < c_end; ++t) {
            const int sb = (t - t_begin) % STAGES_FQ;
            const int key0 = t * KT;
            // the stage of tile t + STAGES_FQ - 1 was last read, by this
            // wave, for tile t - 1
            if (t + STAGES_FQ - 1 < c_end)
                issue(t + STAGES_FQ - 1, (sb + STAGES_FQ - 1) % STAGES_FQ);
            const uint8_t* st = stg[wave][sb];
            const float* sc = &ssc[wave][sb][0];
            if (key0 + KT <= g.n) {
                if (nb == 0) b_key0 = key0;
                float* const stage =
                    (write_logits && row_ok) ? &lgs[wave][nb * g.R * 32] : nullptr;
                fwd_block16_q8<D, false, TRACK>(st, st + 32 * D, sc, sc + 32, qf, o_acc, m_ref,
                                                m_seen, overflow, l_acc, lt_acc, g.c, wave, key0,
                                                g.n, lane, nullptr, key0, stage);
                if (write_logits && ++nb == tf) flush();
            } else {
                if (nb > 0) flush();
                fwd_block16_q8<D, true, TRACK>(st, st + 32 * D, sc, sc + 32, qf, o_acc, m_ref,
                                               m_seen, overflow, l_acc, lt_acc, g.c, wave, key0,
                                               g.n, lane, lg, key0, nullptr);
            }
            // this wave's copies of tile t+1 must have landed; tiles issued
            // after it may stay in flight
            wait_later_q(min(STAGES_FQ - 2, c_end - 1 - (t + 1)));
        }
        if (nb > 0) flush();
        if (t_end > tr.n_ct) {   // the chunk tile (S <= 16 here: a single tile)
            const int key0 = (t_end - 1 - tr.n_ct) * KT;
            // bf16 K and V rows of this wave's key block in its first two
            // stages (every copy of this wave has landed; no other wave
            // touches them); the chunk's K has no scale
            wait_tiles();
            uint16_t* mk = (uint16_t*)stg[wave][0];
            uint16_t* mv = mk + 32 * D;
            constexpr int CPR = D / 8;
#pragma unroll
            for (int u0 = 0; u0 < 32 * CPR; u0 += 64) {
                const int u = u0 + lane;
                const int r = u / CPR, cc = u % CPR;
                const int key = min(key0 + wave * 32 + r, g.S - 1);
                *(u32x4*)(mk + tile_off<D, false>(r, cc)) =
                    *(const u32x4*)(kn_bh + (size_t)key * D + cc * 8);
                *(u32x4*)(mv + tile_off<D, true>(r, cc)) =
                    *(const u32x4*)(vn_bh + (size_t)key * D + cc * 8);
            }
            // the cache blocks set lt = l; this bf16 block adds its rounded weights
            fwd_block16<D, true, TRACK>(mk, mv, off, qf, o_acc, m_ref, m_seen, overflow, l_acc,
                                        lt_acc, g.c, wave, key0, g.S, true, g.G, lane, lg,
                                        g.C + key0, 0, nullptr);
        }
    };
    // the row sum of a lane's row: its 4 lanes (l16 + 16*grp)
    auto row_sum = [&](float x) {
        x += xor16(x);
        return x + xor32(x);
    };

    // Main sweep: each row's reference is its own base-2 logit against its
    // diagonal chunk key (bf16); row sums above 2^kHeadroom send the
    // workgroup to the tracked sweeps.
    {
        bool overflow = false;
        const uint16_t* kself = kn_bh + (size_t)(row_ok ? l16 / g.G : 0) * D + 8 * grp;
        float dot = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            const bf16x8 kv = as_bf16x8(*(const u32x4*)(kself + 32 * ks));
#pragma unroll
            for (int e = 0; e < 8; ++e) dot = fmaf((float)qf[ks][e], (float)kv[e], dot);
        }
        dot = row_sum(dot);
        m_ref = row_ok ? dot * g.c : 0.f;
        zero_state();
        sweep_tiles(TrackC<false>{}, overflow, true, true);
        overflow |= !(row_sum(l_acc) <= kSumLimit);
        if (!__syncthreads_or(overflow)) goto merge;
    }
    // tracked sweeps (rare): first-tile reference with every tile max
    // recorded, then, if still overshot, the exact row max
    for (int sweep = 0; sweep < 2; ++sweep) {
        bool overflow = false;
        m_ref = (sweep == 0) ? -INFINITY : m_seen;
        zero_state();
        sweep_tiles(TrackC<true>{}, overflow, false, false);
        if (!__syncthreads_or(overflow)) break;
    }

merge:
    // merge the waves' (m, l, lt, O) through LDS (the stages are free now)
    {
        const float l = row_sum(l_acc);
        const float lt = row_sum(lt_acc);
        constexpr int XS = D / 4 + 4;   // [NW_S][64 lanes][XS] floats
        static_assert(NW_S * 64 * XS * 4 <= (int)sizeof(stg), "merge area exceeds the stages");
        float* xch = (float*)&stg[0][0][0];
        float* mine = xch + ((size_t)wave * 64 + lane) * XS;
#pragma unroll
        for (int db = 0; db < D / 16; ++db) *(f32x4*)(mine + 4 * db) = o_acc[db];
        mine[D / 4 + 0] = m_ref;
        mine[D / 4 + 1] = l;
        mine[D / 4 + 2] = lt;
        __syncthreads();
        if (wave != 0) return;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW_S; ++w) M = fmaxf(M, xch[((size_t)w * 64 + lane) * XS + D / 4]);
        float wt[NW_S], L = 0.f, Lt = 0.f;
#pragma unroll
        for (int w = 0; w < NW_S; ++w) {
            const float* o = xch + ((size_t)w * 64 + lane) * XS;
            wt[w] = (M == -INFINITY) ? 0.f : fast_exp2(o[D / 4] - M);
            L += wt[w] * o[D / 4 + 1];
            Lt += wt[w] * o[D / 4 + 2];
        }
        if (!row_ok) return;
        const size_t prow = ((size_t)split * BH + bh) * g.rows_pad + l16;
        if (grp == 0) *(f32x4*)(ml_part + prow * 4) = f32x4{M, L, Lt, 0.f};
        float* orow = o_part + prow * D;
        // lane holds dims 16*db + 4*grp + [0, 4) of its row
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < NW_S; ++w)
                acc += wt[w] * *(const f32x4*)(xch + ((size_t)w * 64 + lane) * XS + 4 * db);
            *(f32x4*)(orow + 16 * db + 4 * grp) = acc;
        }
    }
}

// ---------------------------------------------------------------------------
// sum the row-tile partials in tile order
// ---------------------------------------------------------------------------
// With non-null `scores` the kernel also accumulates, as wsum_from_logits_kernel.
__global__ __launch_bounds__(256) void wsum_reduce_kernel(
    const AttnGeom g, const float* __restrict__ wpart, float* __restrict__ wsum,
    float* __restrict__ scores, float* __restrict__ new_scores) {
    const int BH = g.B * g.Hkv;
    const int W = g.C + g.S;
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)BH * W) return;
    const int j = (int)(idx % W);
    const int bh = (int)(idx / W);
    // row tiles in order; the loads of 8 tiles are issued before their sums
    // (the partials are >= 0, so the +0.0 of a skipped tile changes nothing)
    float s = 0.f;
    if (j < g.n || j >= g.C) {
        const int t = j - g.C;   // chunk token (chunk columns only)
        for (int q0 = 0; q0 < g.n_qt; q0 += 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int qt = q0 + u;
                const int i_hi = (min((qt + 1) * kRowsPerBlock, g.R) - 1) / g.G;
                const bool use = qt < g.n_qt && (j < g.n || i_hi >= t);
                v[u] = use ? wpart[((size_t)qt * BH + bh) * W + j] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) s += v[u];
        }
    }
    wsum[idx] = s;
    if (scores) {
        if (j < g.n)
            scores[(size_t)bh * g.C + j] += s;
        else if (j >= g.C)
            new_scores[(size_t)bh * g.S + (j - g.C)] = s;
    }
}

int pick_split(int base_blocks, int max_tiles, int target) {
    int want = (target + base_blocks - 1) / base_blocks;
    int cap = max_tiles / 4;
    if (cap < 1) cap = 1;
    if (want > cap) want = cap;
    return want < 1 ? 1 : want;
}


// Q8: the cache is int8 codes + scales (qc); otherwise bf16 (kc, vc).
template <int D, bool Q8>
hipError_t launch_attention_d(const AttnPlan& pl, const uint16_t* q,
                              const uint16_t* kc, const uint16_t* vc, const Q8Cache& qc,
                              const uint16_t* kn, const uint16_t* vn, float* out,
                              float* lse, float* wsum, void* ws,
                              hipStream_t stream, bool sync_debug, hipEvent_t* ev,
                              float* scores = nullptr, float* new_scores = nullptr) {
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
#define H2O_EVENT(i)                                                               \
    do {                                                                           \
        if (ev && (err = hipEventRecord(ev[i], stream)) != hipSuccess) return err; \
    } while (0)

    H2O_EVENT(0);
    if constexpr (Q8) {
        if (pl.small && g.R <= kFewRows)
            hipLaunchKernelGGL(attn_fwd_few_q8_kernel<D>, dim3(BH * pl.split1), dim3(NT_S), 0,
                               stream, g, pl.split1, q, qc, kn, vn, o_part, ml_part, wpart);
        else if (pl.small)
            hipLaunchKernelGGL(attn_fwd_small_q8_kernel<D>, dim3(BH * pl.split1), dim3(NT_S), 0,
                               stream, g, pl.split1, q, qc, kn, vn, o_part, ml_part, wpart);
        else
            hipLaunchKernelGGL(attn_fwd_q8_kernel<D>, dim3(g.n_qt * BH * pl.split1), dim3(NT),
                               0, stream, g, pl.split1, q, qc, kn, vn, o_part, ml_part);
    } else {
        if (pl.small && g.R <= kFewRows)
            hipLaunchKernelGGL(attn_fwd_few_kernel<D>, dim3(BH * pl.split1), dim3(NT_S), 0,
                               stream, g, pl.split1, q, kc, vc, kn, vn, o_part, ml_part, wpart,
                               nullptr);
        else if (pl.small)
            hipLaunchKernelGGL(attn_fwd_small_kernel<D>, dim3(BH * pl.split1), dim3(NT_S), 0,
                               stream, g, pl.split1, q, kc, vc, kn, vn, o_part, ml_part, wpart,
                               nullptr);
        else
            hipLaunchKernelGGL(attn_fwd_kernel<D>, dim3(g.n_qt * BH * pl.split1), dim3(NT), 0,
                               stream, g, pl.split1, q, kc, vc, kn, vn, o_part, ml_part);
    }
    H2O_CHECK();
    H2O_EVENT(1);
    {
        const long total = (long)BH * g.rows_pad * (D / 4);
        hipLaunchKernelGGL(attn_combine_kernel<D>, dim3((unsigned)((total + 255) / 256)),
                           dim3(256), 0, stream, g, pl.split1, o_part, ml_part, out,
                           lse, l2);
        H2O_CHECK();
    }
    H2O_EVENT(2);
    const long wtotal = (long)BH * (g.C + g.S);
    if (pl.small) {
        const long qtotal = (long)BH * ((g.C + g.S + 3) / 4);
        hipLaunchKernelGGL(wsum_from_logits_kernel, dim3((unsigned)((qtotal + 255) / 256)),
                           dim3(256), 0, stream, g, wpart, l2, wsum, scores, new_scores);
        H2O_CHECK();
        H2O_EVENT(3);
    } else {
        if constexpr (Q8)
            hipLaunchKernelGGL(attn_colsum_q8_kernel<D>, dim3(g.n_qt * BH * pl.split2), dim3(NT),
                               0, stream, g, pl.split2, q, qc, kn, l2, wpart);
        else
            hipLaunchKernelGGL(attn_colsum_kernel<D>, dim3(g.n_qt * BH * pl.split2), dim3(NT),
                               0, stream, g, pl.split2, q, kc, kn, l2, wpart);
        H2O_CHECK();
        H2O_EVENT(3);
        hipLaunchKernelGGL(wsum_reduce_kernel, dim3((unsigned)((wtotal + 255) / 256)),
                           dim3(256), 0, stream, g, wpart, wsum, scores, new_scores);
        H2O_CHECK();
    }
    H2O_EVENT(4);
#undef H2O_CHECK
#undef H2O_EVENT
    return hipSuccess;
}

}  // namespace

bool make_attn_plan(int B, int Hq, int Hkv, int D, int C, int S, int n, float scale,
                    AttnPlan* pl) {
    AttnGeom& g = pl->g;
    g.B = B; g.Hq = Hq; g.Hkv = Hkv; g.G = Hq / Hkv; g.D = D;
    g.C = C; g.S = S; g.n = n;
    g.R = g.G * S;
    pl->small = g.R <= 32;
    g.n_qt = pl->small ? 1 : (g.R + kRowsPerBlock - 1) / kRowsPerBlock;
    g.rows_pad = pl->small ? 32 : g.n_qt * kRowsPerBlock;
    const float tau = (scale > 0.f) ? scale : 1.0f / sqrtf((float)D);
    g.c = tau * kLog2e;
    const int BH = B * Hkv;
    const int max_tiles = (C + KT - 1) / KT + (S + KT - 1) / KT;
    // pass 1 holds one workgroup per CU (few-row path: two), pass 2 two
    pl->split1 = pick_split(g.n_qt * BH, max_tiles, pl->small ? 1024 : 256);
    const int max_tiles2 = (C + KT2 - 1) / KT2 + (S + KT2 - 1) / KT2;
    pl->split2 = pl->small ? 1 : pick_split(g.n_qt * BH, max_tiles2, 512);
    auto align = [](size_t x) { return (x + 255) & ~(size_t)255; };
    size_t off = 0;
    pl->off_o = off;
    off = align(off + (size_t)pl->split1 * BH * g.rows_pad * D * sizeof(float));
    pl->off_ml = off;
    off = align(off + (size_t)pl->split1 * BH * g.rows_pad * 4 * sizeof(float));
    pl->off_l2 = off;
    off = align(off + (size_t)BH * g.rows_pad * sizeof(float));
    pl->off_wp = off;   // row-tile partial sums, or the logits of the few-row path
    off = align(off + (size_t)(pl->small ? g.R * logit_stride(g) : g.n_qt * (C + S)) * BH *
                          sizeof(float));
    pl->off_tail = off;
    off = align(off + (size_t)BH * 16);
    pl->bytes = off;
    return true;
}

hipError_t launch_attention(const AttnPlan& plan, const uint16_t* q, const uint16_t* kc,
                            const uint16_t* vc, const uint16_t* kn, const uint16_t* vn,
                            float* out, float* lse, float* wsum, void* ws,
                            hipStream_t stream, bool sync_debug, hipEvent_t* ev5,
                            float* scores, float* new_scores) {
    const Q8Cache none{nullptr, nullptr, nullptr, nullptr};
    if (plan.g.D == 64)
        return launch_attention_d<64, false>(plan, q, kc, vc, none, kn, vn, out, lse, wsum, ws,
                                             stream, sync_debug, ev5, scores, new_scores);
    return launch_attention_d<128, false>(plan, q, kc, vc, none, kn, vn, out, lse, wsum, ws,
                                          stream, sync_debug, ev5, scores, new_scores);
}

// One-token step on the few-row path: the streaming pass, then the tail
// kernels (split merge, summed weights, accumulation and the running
// minimum; then the choice and the scatter).
template <int D>
hipError_t launch_decode_step_d(const AttnPlan& pl, const uint16_t* q, uint16_t* kc,
                                uint16_t* vc, const uint16_t* kn, const uint16_t* vn,
                                float* out, float* lse, float* wsum, float* scores,
                                float* new_scores, int32_t* evict, int64_t* pos, int64_t p0,
                                void* ws, hipStream_t stream, bool sync_debug, hipEvent_t* ev) {
    const AttnGeom& g = pl.g;
    char* w = (char*)ws;
    float* o_part = (float*)(w + pl.off_o);
    float* ml_part = (float*)(w + pl.off_ml);
    float* logits = (float*)(w + pl.off_wp);
    const int BH = g.B * g.Hkv;
    hipError_t err;
    auto check = [&]() {
        err = hipGetLastError();
        if (err == hipSuccess && sync_debug) err = hipStreamSynchronize(stream);
        return err;
    };
    auto event = [&](int i) { return ev ? hipEventRecord(ev[i], stream) : hipSuccess; };
    if ((err = event(0)) != hipSuccess) return err;
    TailState* tstate = (TailState*)(w + pl.off_tail);
    if (g.R <= kFewRows)
        hipLaunchKernelGGL(attn_fwd_few_kernel<D>, dim3(BH * pl.split1), dim3(NT_S), 0, stream,
                           g, pl.split1, q, kc, vc, kn, vn, o_part, ml_part, logits, tstate);
    else
        hipLaunchKernelGGL(attn_fwd_small_kernel<D>, dim3(BH * pl.split1), dim3(NT_S), 0,
                           stream, g, pl.split1, q, kc, vc, kn, vn, o_part, ml_part, logits,
                           tstate);
    if (check() != hipSuccess) return err;
    if ((err = event(1)) != hipSuccess) return err;
    hipLaunchKernelGGL(decode_tail_kernel<D>, dim3(BH * TAIL_P), dim3(TAIL_T), 0, stream, g,
                       pl.split1, o_part, ml_part, logits, tstate, out, lse, wsum, scores,
                       new_scores);
    if (check() != hipSuccess) return err;
    hipLaunchKernelGGL(decode_scatter_kernel<D>, dim3(BH), dim3(64), 0, stream, g, tstate,
                       scores, new_scores, evict, kc, vc, pos, kn, vn, p0);
    if (check() != hipSuccess) return err;
    for (int i = 2; i < 5; ++i)
        if ((err = event(i)) != hipSuccess) return err;
    return hipSuccess;
}

bool decode_tail_applies(const AttnPlan& pl) { return pl.small && pl.g.S == 1; }

hipError_t launch_decode_step(const AttnPlan& pl, const uint16_t* q, uint16_t* kc,
                              uint16_t* vc, const uint16_t* kn, const uint16_t* vn, float* out,
                              float* lse, float* wsum, float* scores, float* new_scores,
                              int32_t* evict, int64_t* pos, int64_t p0, void* ws,
                              hipStream_t stream, bool sync_debug, hipEvent_t* ev5) {
    if (pl.g.D == 64)
        return launch_decode_step_d<64>(pl, q, kc, vc, kn, vn, out, lse, wsum, scores,
                                        new_scores, evict, pos, p0, ws, stream, sync_debug, ev5);
    return launch_decode_step_d<128>(pl, q, kc, vc, kn, vn, out, lse, wsum, scores, new_scores,
                                     evict, pos, p0, ws, stream, sync_debug, ev5);
}

hipError_t launch_attention_q8(const AttnPlan& plan, const uint16_t* q, const int8_t* kc,
                               const float* ks, const int8_t* vc, const float* vs,
                               const uint16_t* kn, const uint16_t* vn, float* out, float* lse,
                               float* wsum, void* ws, hipStream_t stream, bool sync_debug,
                               hipEvent_t* ev5) {
    const Q8Cache qc{kc, ks, vc, vs};
    if (plan.g.D == 64)
        return launch_attention_d<64, true>(plan, q, nullptr, nullptr, qc, kn, vn, out, lse,
                                            wsum, ws, stream, sync_debug, ev5);
    return launch_attention_d<128, true>(plan, q, nullptr, nullptr, qc, kn, vn, out, lse, wsum,
                                         ws, stream, sync_debug, ev5);
}

}  // namespace h2o
