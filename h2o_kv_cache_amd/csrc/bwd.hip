// Backward of the chunk attention with the slot layout fixed, for gfx950.
//
// Method: "Learning how to Forget: Fine-tuning for Long-Context Sparse
// Attention" -- Chinese translation page, abstract and §1: the fine-tuning
// computes gradients through the sparse attention with the KV cache policy in
// place, with no approximation beyond the sparse attention.  The eviction
// decisions that produced the slot layout are discrete and not
// differentiated; gradients flow to Q, to the K/V rows of the valid cache
// slots, and to the chunk's K/V.
//
// With P = 2^(S*c - L2) the forward's normalised weights (c = scale*log2 e,
// L2 the row's base-2 log-sum-exp):
//   dP = dO V^T,  D_i = sum_j P_ij dP_ij = dO_i . O_i,  dS = P * (dP - D),
//   dQ = scale dS K,   dK = scale dS^T Q,   dV = P^T dO.
// Kernels:
//   bwd_prep_kernel       per packed row: L2 and D.
//   dkdv_pair_body        key-major, D = 128.  Two waves of one SIMD share a
//                         32-key block of one KV head: one keeps the K
//                         fragments and dV^T accumulators (S, P, dV), the
//                         other the V fragments and dK^T accumulators (dP,
//                         dS, dK), P passing between them through LDS.  They
//                         walk the rows of the G query heads in 32-row blocks
//                         (a lane owns a key and 16 rows); the contractions
//                         over rows read their row fragments transposed from
//                         LDS.
//   bwd_dkdv_kernel       key-major, D = 64: one wave owns two 32-key blocks
//                         with both sets of fragments and accumulators.
//   dq_body               row-major, shaped like the forward's pass 1:
//                         S^T = K Q^T and dP^T = V dO^T (a lane owns a row),
//                         then dQ^T += K^T dS^T (bwd_dq_kernel at D = 64).
//   bwd_dkdv_dq_kernel    D = 128: the dK/dV key tiles and the dQ row tiles
//                         in one grid, so that the dQ workgroups fill the
//                         last, partial round of key tiles.
// Rows are packed as in the forward: row r of a (b, kv head h) is query r / G
// of head h*G + r % G.  Every reduction has a fixed order.
#include "h2o_device.h"
#include "h2o_launch.h"
#include "h2o_tiles.h"

namespace h2o {
namespace {

// ---------------------------------------------------------------------------
// prep: L2 = lse * log2(e) and D = dO . O per packed row
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const BwdGeom g,
                                                      const float* __restrict__ out,
                                                      const float* __restrict__ lse,
                                                      const uint16_t* __restrict__ dout,
                                                      float* __restrict__ l2,
                                                      float* __restrict__ drow) {
    constexpr int LPR = D / 8;   // lanes per row, 8 elements each (consecutive lanes)
    const long row = ((long)blockIdx.x * 256 + threadIdx.x) / LPR;
    const int part = threadIdx.x % LPR;
    const long total = (long)g.B * g.Hkv * g.R;
    const bool ok = row < total;
    float acc = 0.f;
    size_t head_row = 0;
    if (ok) {
        const int bh = (int)(row / g.R), r = (int)(row % g.R);
        const int b = bh / g.Hkv, h = bh % g.Hkv;
        head_row = ((size_t)b * g.Hq + (size_t)h * g.G + r % g.G) * g.S + r / g.G;
        const float* o = out + head_row * D + part * 8;
        const f32x4 o0 = *(const f32x4*)o, o1 = *(const f32x4*)(o + 4);
        const bf16x8 d8 = as_bf16x8(*(const u32x4*)(dout + head_row * D + part * 8));
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = fmaf((float)d8[e], o0[e], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = fmaf((float)d8[4 + e], o1[e], acc);
    }
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) acc += __shfl_xor(acc, off, 64);
    if (ok && part == 0) {
        drow[row] = acc;
        l2[row] = lse[head_row] * kLog2e;
    }
}

// ---------------------------------------------------------------------------
// shared pieces of the two main kernels
// ---------------------------------------------------------------------------
constexpr int BR = 32;   // rows per row block / keys per key block

// Copy packed rows r0 .. r0+ROWS-1 of q or dO (base = the tensor at head
// h*G, query 0) into a ROWS x D LDS tile with swizzle VT.  The rows of one
// tile come from G different heads, so every 16-byte chunk computes its own
// source; rows past R re-read row R-1 (a valid row whose weights are masked).
template <int D, bool VT, int NW, int ROWS>
__device__ __forceinline__ void issue_rows(uint16_t* tile, const uint16_t* __restrict__ base,
                                           int r0, int R, int G, int S, int wave, int lane) {
    constexpr int CPR = D / 8;
    constexpr int ITER = ROWS * CPR / (NW * 64);
    static_assert(ITER * NW * 64 == ROWS * CPR, "tile must split into whole 1 KiB blocks");
    const uint32_t tb = __builtin_amdgcn_readfirstlane(lds_addr(tile));
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        const int blk = it * NW + wave;
        const int p = blk * 64 + lane;
        const int row = p / CPR;
        const int chunk = (p % CPR) ^ tile_swz<D, VT>(row);
        const int gr = min(r0 + row, R - 1);
        dma16(base + ((size_t)(gr % G) * S + gr / G) * D + chunk * 8, tb + blk * 1024);
    }
}

// K (or V) fragments of one key of this lane as the B operand of an MFMA
// whose k-dimension is the head dimension: dims 16*ks + 8*half + [0, 8) of
// `row` (zeros when the key does not exist).
template <int D>
__device__ __forceinline__ void load_key_frags(bf16x8 (&f)[D / 16], const uint16_t* row, bool ok,
                                               int half) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (ok) v = *(const u32x4*)(row + ks * 16 + half * 8);
        f[ks] = as_bf16x8(v);
    }
}

// ---------------------------------------------------------------------------
// dK, dV: key-major, one wave per SIMD (D = 64; D = 128 uses the pair kernel
// below)
// ---------------------------------------------------------------------------
constexpr int KV_WAVES = 4;                 // one wave per SIMD (up to 512 registers)
constexpr int KV_NT = KV_WAVES * 64;
// 32-key blocks per wave: each Q / dO fragment read feeds KB MFMAs (at D = 128
// the fragments and accumulators of two blocks would exceed 512 registers)
template <int D>
constexpr int kv_kb() { return D == 128 ? 1 : 2; }
template <int D>
constexpr int kv_keys() { return KV_WAVES * kv_kb<D>() * BR; }   // keys per workgroup

template <int D>
__global__ __launch_bounds__(KV_NT, 1) void bwd_dkdv_kernel(
    const BwdGeom g, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const uint16_t* __restrict__ kn,
    const uint16_t* __restrict__ vn, const uint16_t* __restrict__ dout,
    const float* __restrict__ l2, const float* __restrict__ drow, float* __restrict__ dkc,
    float* __restrict__ dvc, float* __restrict__ dkn, float* __restrict__ dvn) {
    constexpr int TILE = BR * D;            // elements of one row-block tile
    constexpr int KV_KB = kv_kb<D>();
    constexpr int KV_KEYS = kv_keys<D>();
    // per buffer: Q (row-fragment swizzle), Q (transposed-read swizzle),
    // dO (both swizzles), then L2 and D of the 32 rows
    __shared__ __attribute__((aligned(16))) uint16_t tiles[2][4][TILE];
    __shared__ __attribute__((aligned(16))) float stats[2][2 * BR];

    const int n_ct = (g.C + KV_KEYS - 1) / KV_KEYS;   // cache key tiles (all C slots)
    const int n_kt = n_ct + (g.S + KV_KEYS - 1) / KV_KEYS;
    const int bh = blockIdx.x / n_kt, kt = blockIdx.x % n_kt;
    const int b = bh / g.Hkv, h = bh % g.Hkv;
    const bool chunk = kt >= n_ct;
    const int key0 = (chunk ? kt - n_ct : kt) * KV_KEYS;   // first key of the tile
    const int lim = chunk ? g.S : g.n;                     // keys that exist
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, l32 = lane & 31;

    // this lane's keys: key0 + wave*64 + kb*32 + l32
    bf16x8 kf[KV_KB][D / 16], vf[KV_KB][D / 16];
    int key[KV_KB], vis_lo[KV_KB], vis_hi[KV_KB];
    bool kok[KV_KB];
#pragma unroll
    for (int kb = 0; kb < KV_KB; ++kb) {
        key[kb] = key0 + wave * (KV_KB * BR) + kb * BR + l32;
        kok[kb] = key[kb] < lim;
        // row r (query r / G) sees the key iff it exists, r < R, and for a chunk
        // key j, r / G >= j, i.e. r >= j * G
        vis_lo[kb] = chunk ? key[kb] * g.G : 0;
        vis_hi[kb] = kok[kb] ? g.R : 0;
        const size_t krow = chunk ? ((size_t)bh * g.S + key[kb]) * D : ((size_t)bh * g.C + key[kb]) * D;
        load_key_frags<D>(kf[kb], (chunk ? kn : kc) + krow, kok[kb], half);
        load_key_frags<D>(vf[kb], (chunk ? vn : vc) + krow, kok[kb], half);
    }
    f32x16 dk_acc[KV_KB][D / 32], dv_acc[KV_KB][D / 32];
#pragma unroll
    for (int kb = 0; kb < KV_KB; ++kb)
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) dk_acc[kb][db][v] = dv_acc[kb][db][v] = 0.f;

    // rows that can see a key of this tile: all for cache slots (if any slot
    // of the tile is valid), rows with query >= key0 for chunk keys
    const int nrb = (g.R + BR - 1) / BR;
    int rb0 = chunk ? (key0 * g.G) / BR : 0;
    if (key0 >= lim) rb0 = nrb;             // no valid key: gradients stay 0
    const uint16_t* q_h = q + ((size_t)b * g.Hq + (size_t)h * g.G) * g.S * D;
    const uint16_t* do_h = dout + ((size_t)b * g.Hq + (size_t)h * g.G) * g.S * D;
    const float* l2_bh = l2 + (size_t)bh * g.R;
    const float* dr_bh = drow + (size_t)bh * g.R;

    auto issue = [&](int rb, int buf) {
        const int r0 = rb * BR;
        issue_rows<D, false, KV_WAVES, BR>(tiles[buf][0], q_h, r0, g.R, g.G, g.S, wave, lane);
        issue_rows<D, true, KV_WAVES, BR>(tiles[buf][1], q_h, r0, g.R, g.G, g.S, wave, lane);
        issue_rows<D, false, KV_WAVES, BR>(tiles[buf][2], do_h, r0, g.R, g.G, g.S, wave, lane);
        issue_rows<D, true, KV_WAVES, BR>(tiles[buf][3], do_h, r0, g.R, g.G, g.S, wave, lane);
        if (wave == 0) {   // lanes 0-31: L2 of rows r0.., lanes 32-63: D
            const int gr = min(r0 + l32, g.R - 1);
            dma4((half ? dr_bh : l2_bh) + gr,
                 __builtin_amdgcn_readfirstlane(lds_addr(stats[buf])));
        }
    };

    const LdsOffsets<D> off(lane);
    const float c = g.c;
    if (rb0 < nrb) issue(rb0, 0);
    wait_tiles();
    __syncthreads();
    for (int rb = rb0; rb < nrb; ++rb) {
        const int buf = (rb - rb0) & 1;
        if (rb + 1 < nrb) issue(rb + 1, buf ^ 1);
        const uint16_t* Qk = tiles[buf][0];
        const uint16_t* Qv = tiles[buf][1];
        const uint16_t* Ok = tiles[buf][2];
        const uint16_t* Ov = tiles[buf][3];
        const int r0 = rb * BR;

        // S = Q K^T and dP = dO V^T for both key blocks: element v of a lane
        // is row r0 + 8*(v/4) + 4*half + v%4 against the lane's key
        f32x16 s[KV_KB], dp[KV_KB];
#pragma unroll
        for (int kb = 0; kb < KV_KB; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) s[kb][v] = dp[kb][v] = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            const bf16x8 qa = as_bf16x8(lds_read16(Qk, off.k[ks]));
            const bf16x8 oa = as_bf16x8(lds_read16(Ok, off.k[ks]));
#pragma unroll
            for (int kb = 0; kb < KV_KB; ++kb) {
                s[kb] = mfma32x32x16(qa, kf[kb][ks], s[kb]);
                dp[kb] = mfma32x32x16(oa, vf[kb][ks], dp[kb]);
            }
        }

        // P and dS (selects, so masked entries are exactly 0 whatever the
        // arithmetic gives), in bf16 as the B operands of the row contraction
        float l2v[16], drv[16];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 a = *(const f32x4*)&stats[buf][8 * g4 + 4 * half];
            const f32x4 d = *(const f32x4*)&stats[buf][BR + 8 * g4 + 4 * half];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                l2v[4 * g4 + e] = a[e];
                drv[4 * g4 + e] = d[e];
            }
        }
        bf16x8 pf[KV_KB][2], sf[KV_KB][2];
#pragma unroll
        for (int kb = 0; kb < KV_KB; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = r0 + acc_row(v, half);
                const bool vis = row >= vis_lo[kb] && row < vis_hi[kb];
                const float p = vis ? fast_exp2(fmaf(s[kb][v], c, -l2v[v])) : 0.f;
                const float ds = vis ? p * (dp[kb][v] - drv[v]) : 0.f;
                pf[kb][v >> 3][v & 7] = (__bf16)p;
                sf[kb][v >> 3][v & 7] = (__bf16)ds;
            }

        // dV^T += dO^T P and dK^T += Q^T dS: k-step hs covers rows
        // r0 + 16*hs + {4*half + [0,4), 8 + 4*half + [0,4)}, the rows the
        // accumulator elements 8*hs .. 8*hs+7 hold
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
            const uint32_t row_b = (uint32_t)(16 * hs) * 2 * D;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const u32x2 olo = lds_read_tr(Ov, off.v[db] + row_b);
                const u32x2 ohi = lds_read_tr(Ov, off.v[db] + row_b + 8 * 2 * D);
                const u32x2 qlo = lds_read_tr(Qv, off.v[db] + row_b);
                const u32x2 qhi = lds_read_tr(Qv, off.v[db] + row_b + 8 * 2 * D);
                const bf16x8 ot = as_bf16x8(u32x4{olo[0], olo[1], ohi[0], ohi[1]});
                const bf16x8 qt = as_bf16x8(u32x4{qlo[0], qlo[1], qhi[0], qhi[1]});
#pragma unroll
                for (int kb = 0; kb < KV_KB; ++kb) {
                    dv_acc[kb][db] = mfma32x32x16(ot, pf[kb][hs], dv_acc[kb][db]);
                    dk_acc[kb][db] = mfma32x32x16(qt, sf[kb][hs], dk_acc[kb][db]);
                }
            }
        }
        wait_tiles();
        __syncthreads();
    }

    // dK = scale * (dK^T)^T, dV = (dV^T)^T: lane holds its key's dims
    // 32*db + 8*gq + 4*half + [0, 4) in elements 4*gq .. 4*gq+3
#pragma unroll
    for (int kb = 0; kb < KV_KB; ++kb) {
        if (key[kb] >= (chunk ? g.S : g.C)) continue;
        const size_t row = chunk ? ((size_t)bh * g.S + key[kb]) * D : ((size_t)bh * g.C + key[kb]) * D;
        float* dk = (chunk ? dkn : dkc) + row;
        float* dv = (chunk ? dvn : dvc) + row;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int d = db * 32 + 8 * gq + 4 * half;
                *(f32x4*)(dk + d) = g.tau * f32x4{dk_acc[kb][db][4 * gq + 0], dk_acc[kb][db][4 * gq + 1],
                                                  dk_acc[kb][db][4 * gq + 2], dk_acc[kb][db][4 * gq + 3]};
                *(f32x4*)(dv + d) = f32x4{dv_acc[kb][db][4 * gq + 0], dv_acc[kb][db][4 * gq + 1],
                                          dv_acc[kb][db][4 * gq + 2], dv_acc[kb][db][4 * gq + 3]};
            }
    }
}

// ---------------------------------------------------------------------------
// dK, dV at D = 128 with two waves per SIMD.  Waves w and w + 4 (one SIMD)
// share a 32-key block: the P-wave (w < 4) computes S and P and accumulates
// dV^T += dO^T P; the dS-wave computes dP, takes P from the P-wave through
// LDS, forms dS and accumulates dK^T += Q^T dS.  Each wave keeps one set of
// K or V fragments and one set of accumulators (about half of the
// single-wave kernel's registers), so two fit per SIMD; the MFMA count per
// key block is unchanged, at the price of one more barrier per row block.
// The row-block loop is unrolled by the two tile buffers so that every LDS
// operand address is a per-lane register plus an immediate, and the mask is
// applied only to row blocks that are not wholly visible to the key block.
// ---------------------------------------------------------------------------
constexpr int PQ_WAVES = 8;
constexpr int PQ_NT = PQ_WAVES * 64;
constexpr int PQ_KEYS = (PQ_WAVES / 2) * BR;   // keys per workgroup

// Swizzle of bf16 tiles read both as row fragments and transposed, so that
// one copy serves both reads (64 banks of 4 bytes, 256 bytes per cycle):
//   D = 128: chunk ^ (4*(r mod 4) + (r/4) mod 4).  Row-fragment reads (16
//     lanes, one chunk of 16 consecutive rows) see a permutation of the 16
//     chunk positions; transposed reads (32 lanes, four chunks of rows
//     4a..4a+3) see the rows' 64-byte runs in four disjoint bank groups.
//   D = 64 (two rows per 256-byte bank line): chunk ^ (4*((r/2) mod 2) +
//     (r/4) mod 4): the 8 even (and the 8 odd) rows of 16 see distinct chunk
//     positions, and rows 4a, 4a+2 (4a+1, 4a+3) runs differ in chunk bit 2.
// Both depend on row bits 0..3 only: rows 16 apart share the swizzle.
template <int D>
__device__ __forceinline__ int pq_swz(int r) {
    static_assert(D == 64 || D == 128, "head dim");
    return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

template <int N>
struct IntC {
    static constexpr int value = N;
};

__device__ __forceinline__ u32x4 lds_ld16(uint32_t addr) {
    return *(const __attribute__((address_space(3))) u32x4*)(size_t)addr;
}
__device__ __forceinline__ u32x2 lds_ld_tr(uint32_t addr) {
    const i16x4 v =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(size_t)addr);
    return __builtin_bit_cast(u32x2, v);
}

// The body of one dK/dV workgroup (key tile `blk` of the (b, kv head)-major
// list), run by bwd_dkdv_dq_kernel.
template <int D>
__device__ __forceinline__ void dkdv_pair_body(
    const int blk, const BwdGeom& g, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn,
    const uint16_t* __restrict__ dout, const float* __restrict__ l2,
    const float* __restrict__ drow, float* __restrict__ dkc, float* __restrict__ dvc,
    float* __restrict__ dkn, float* __restrict__ dvn) {
    constexpr int TILE = BR * D;
    constexpr int NDB = D / 32;
    constexpr int CPR = D / 8;                       // 16-byte chunks per row
    constexpr uint32_t BUF_B = 2 * TILE * 2;         // bytes of one buffer's tiles
    // each lane copies one 16-byte chunk of each tile per row block
    static_assert(BR * CPR == PQ_NT, "one copy per lane per tile");
    static_assert(D == 128, "written for eight k-steps of 16");
    // per buffer: Q and dO of 32 rows, one copy each, read both as row
    // fragments and transposed (swizzle pq_swz)
    __shared__ __attribute__((aligned(16))) uint16_t tiles[2][2][TILE];
    __shared__ __attribute__((aligned(16))) float stats[2][2 * BR];
    // P of each pair: [pair][element group][lane][4]
    __shared__ __attribute__((aligned(16))) float xch[PQ_WAVES / 2][4][64][4];

    const int n_ct = (g.C + PQ_KEYS - 1) / PQ_KEYS;
    const int n_kt = n_ct + (g.S + PQ_KEYS - 1) / PQ_KEYS;
    const int bh = blk / n_kt, kt = blk % n_kt;
    const int b = bh / g.Hkv, h = bh % g.Hkv;
    const bool chunk = kt >= n_ct;
    const int key0 = (chunk ? kt - n_ct : kt) * PQ_KEYS;
    const int lim = chunk ? g.S : g.n;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pair = wave & 3;
    const bool dsw = wave >= 4;                 // the dS-wave of the pair
    const int half = lane >> 5, l32 = lane & 31;

    const int kp0 = key0 + pair * BR;           // the pair's key block
    const int key = kp0 + l32;
    const bool kok = key < lim;
    // row r (query r / G) sees the key iff it exists, r < R, and for a chunk
    // key j, r / G >= j, i.e. r >= j * G; a row block [r0, r0 + 32) sees the
    // whole key block iff r0 >= full_lo and r0 + 32 <= full_hi
    const int vis_lo = chunk ? key * g.G : 0, vis_hi = kok ? g.R : 0;
    const int full_lo = chunk ? (kp0 + BR - 1) * g.G : 0;
    const int full_hi = kp0 + BR - 1 < lim ? g.R : 0;
    bf16x8 kvf[D / 16];   // K fragments (P-wave) or V fragments (dS-wave)
    {
        const size_t krow = chunk ? ((size_t)bh * g.S + key) * D : ((size_t)bh * g.C + key) * D;
        const uint16_t* src = dsw ? (chunk ? vn : vc) : (chunk ? kn : kc);
        load_key_frags<D>(kvf, src + krow, kok, half);
    }
    f32x16 acc[NDB];      // dV^T (P-wave) or dK^T (dS-wave)
#pragma unroll
    for (int i = 0; i < NDB; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;

    const int nrb = (g.R + BR - 1) / BR;
    int rb0 = chunk ? (key0 * g.G) / BR : 0;
    if (key0 >= lim) rb0 = nrb;
    const uint16_t* q_h = q + ((size_t)b * g.Hq + (size_t)h * g.G) * g.S * D;
    const uint16_t* do_h = dout + ((size_t)b * g.Hq + (size_t)h * g.G) * g.S * D;
    const float* l2_bh = l2 + (size_t)bh * g.R;
    const float* dr_bh = drow + (size_t)bh * g.R;

    // Row-block copies: lane (wave, lane) copies chunk p % CPR of row p / CPR
    // (p = 64 * wave + lane) of each tile, stored at LDS slot p under the
    // tile's swizzle.  Packed row r is query r / G of head h*G + r % G; the
    // lane tracks (r % G, r / G) of its row from block to block, and rows past
    // R re-read row R - 1 (query S - 1 of head G - 1).
    const int cp = wave * 64 + lane;
    const int crow = cp / CPR;
    const int cu = (cp % CPR) ^ pq_swz<D>(crow);
    const int g_div = BR / g.G, g_mod = BR % g.G;
    int nx_r = rb0 * BR + crow;                 // this lane's row in the next block to copy
    int nx_a = nx_r % g.G, nx_i = nx_r / g.G;
    auto issue_next = [&](auto BUFC) {
        constexpr int BUF = decltype(BUFC)::value;
        const bool past = nx_r >= g.R;
        const int a = past ? g.G - 1 : nx_a, i = past ? g.S - 1 : nx_i;
        const size_t ro = ((size_t)a * g.S + i) * D;
        const uint32_t lb = __builtin_amdgcn_readfirstlane(lds_addr(tiles[BUF][0])) + wave * 1024;
        dma16(q_h + ro + cu * 8, lb);
        dma16(do_h + ro + cu * 8, lb + TILE * 2);
        if (wave == 0) {
            const int gr = min(nx_r - crow + l32, g.R - 1);
            dma4((half ? dr_bh : l2_bh) + gr,
                 __builtin_amdgcn_readfirstlane(lds_addr(stats[BUF])));
        }
        nx_r += BR;
        nx_a += g_mod;
        nx_i += g_div;
        if (nx_a >= g.G) {
            nx_a -= g.G;
            nx_i += 1;
        }
    };

    // per-lane LDS byte addresses, in buffer 0, of this wave's operands:
    //   ra[ks]: row-fragment read of S = Q K^T (P-wave) or dP = dO V^T
    //           (dS-wave): row l32, dims 16*ks + 8*half + [0, 8);
    //   ta[k][db]: transposed read of dO (P-wave) or Q (dS-wave) for rows
    //           8*k + 4*half + (lane%16)/4 (k = 0, 1; rows 16 further on share
    //           the swizzle and add an immediate), dims
    //           32*db + 16*((lane/16)%2) + 4*(lane%4) + [0, 4).
    uint32_t ra[D / 16], ta[2][NDB];
    {
        const uint32_t rbase = lds_addr(tiles[0][dsw ? 1 : 0]);
        const uint32_t tbase = lds_addr(tiles[0][dsw ? 0 : 1]);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            ra[ks] = rbase + 2u * (uint32_t)(l32 * D + (((2 * ks + half) ^ pq_swz<D>(l32)) << 3));
        const int j = lane & 15;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int r = 8 * k + 4 * half + (j >> 2);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const int d = db * 32 + (lane & 16) + 4 * (j & 3);
                ta[k][db] = tbase + 2u * (uint32_t)(r * D + (((d >> 3) ^ pq_swz<D>(r)) << 3) + (d & 7));
            }
        }
    }
    const float c = g.c;
    float* my_x = &xch[pair][0][lane][0];

    // P-wave: P = 2^(S c - L2) (masked entries exactly 0) to LDS and, in bf16,
    // to `bop`
    auto p_block = [&](auto BUFC, auto MASKC, int r0, const f32x16& sd, bf16x8 (&bop)[2]) {
        constexpr int BUF = decltype(BUFC)::value;
        constexpr bool MASK = decltype(MASKC)::value != 0;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 a = *(const f32x4*)&stats[BUF][8 * g4 + 4 * half];
            float p[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int v = 4 * g4 + e;
                p[e] = fast_exp2(fmaf(sd[v], c, -a[e]));
                if (MASK) {
                    const int row = r0 + acc_row(v, half);
                    p[e] = (row >= vis_lo && row < vis_hi) ? p[e] : 0.f;
                }
                bop[v >> 3][v & 7] = (__bf16)p[e];
            }
            *(f32x4*)(my_x + g4 * 64 * 4) = f32x4{p[0], p[1], p[2], p[3]};
        }
    };

    auto step = [&](auto BUFC, int rb) {
        constexpr int BUF = decltype(BUFC)::value;
        if (rb + 1 < nrb) issue_next(IntC<BUF ^ 1>{});
        const int r0 = rb * BR;

        // S = Q K^T (P-wave) or dP = dO V^T (dS-wave): element v of a lane is
        // row r0 + 8*(v/4) + 4*half + v%4 against the lane's key
        // all eight operand reads are issued before the first product (the
        // empty asm takes them together)
        u32x4 ar[D / 16];
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) ar[ks] = lds_ld16(ra[ks] + BUF * BUF_B);
        asm volatile("" : "+v"(ar[0]), "+v"(ar[1]), "+v"(ar[2]), "+v"(ar[3]), "+v"(ar[4]),
                     "+v"(ar[5]), "+v"(ar[6]), "+v"(ar[7]));
        // the transposed operand of the row contraction (dO for the P-wave, Q
        // for the dS-wave) does not depend on P, so its 16 reads are issued
        // here, under the products, and not after the barrier
        u32x2 trv[2][NDB][2];
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
            const uint32_t o = BUF * BUF_B + (uint32_t)(16 * hs) * 2 * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                trv[hs][db][0] = lds_ld_tr(ta[0][db] + o);
                trv[hs][db][1] = lds_ld_tr(ta[1][db] + o);
            }
        }
        f32x16 sd;
#pragma unroll
        for (int v = 0; v < 16; ++v) sd[v] = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) sd = mfma32x32x16(as_bf16x8(ar[ks]), kvf[ks], sd);

        bf16x8 bop[2];   // B operand of the row contraction: P or dS, in bf16
        if (!dsw) {
            if (r0 >= full_lo && r0 + BR <= full_hi)
                p_block(BUFC, IntC<0>{}, r0, sd, bop);
            else
                p_block(BUFC, IntC<1>{}, r0, sd, bop);
        }
        __syncthreads();
        // dS-wave: dS = P * (dP - D); P is exactly 0 where masked and dP - D is
        // finite (K, V of missing keys read as 0, rows past R re-read a valid
        // row), so dS needs no mask of its own
        if (dsw) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 pp = *(const f32x4*)(my_x + g4 * 64 * 4);
                const f32x4 d = *(const f32x4*)&stats[BUF][BR + 8 * g4 + 4 * half];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int v = 4 * g4 + e;
                    bop[v >> 3][v & 7] = (__bf16)(pp[e] * (sd[v] - d[e]));
                }
            }
        }

        // dV^T += dO^T P (P-wave) or dK^T += Q^T dS (dS-wave): k-step hs covers
        // rows r0 + 16*hs + {4*half + [0,4), 8 + 4*half + [0,4)}
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const u32x2 lo = trv[hs][db][0];
                const u32x2 hi = trv[hs][db][1];
                acc[db] = mfma32x32x16(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), bop[hs],
                                       acc[db]);
            }
        }
        wait_tiles();
        __syncthreads();
    };

    if (rb0 < nrb) issue_next(IntC<0>{});
    wait_tiles();
    __syncthreads();
    for (int rb = rb0; rb < nrb; rb += 2) {
        step(IntC<0>{}, rb);
        if (rb + 1 < nrb) step(IntC<1>{}, rb + 1);
    }

    if (key >= (chunk ? g.S : g.C)) return;
    const size_t row = chunk ? ((size_t)bh * g.S + key) * D : ((size_t)bh * g.C + key) * D;
    float* dst = (dsw ? (chunk ? dkn : dkc) : (chunk ? dvn : dvc)) + row;
    const float sc = dsw ? g.tau : 1.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const int d = db * 32 + 8 * gq + 4 * half;
            *(f32x4*)(dst + d) = sc * f32x4{acc[db][4 * gq + 0], acc[db][4 * gq + 1],
                                            acc[db][4 * gq + 2], acc[db][4 * gq + 3]};
        }
}


// ---------------------------------------------------------------------------
// dQ: row-major
// ---------------------------------------------------------------------------
constexpr int Q_WAVES = 8;
constexpr int Q_NT = Q_WAVES * 64;
constexpr int Q_ROWS = Q_WAVES * BR;        // rows per workgroup
constexpr int Q_KT = 64;                    // keys per tile

// The body of dQ workgroup `blk` of `nblk`, shared by bwd_dq_kernel and
// bwd_dkdv_dq_kernel.
template <int D>
__device__ __forceinline__ void dq_body(
    const int blk, const int nblk, const BwdGeom& g, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn,
    const uint16_t* __restrict__ dout, const float* __restrict__ l2,
    const float* __restrict__ drow, const int nsplit, float* __restrict__ dq,
    float* __restrict__ dq_part) {
    constexpr int TILE = Q_KT * D;
    constexpr int CPR = D / 8;
    constexpr int NDB = D / 32;
    constexpr uint32_t BUF_B = 2 * TILE * 2;         // bytes of one buffer's tiles
    // per buffer: K (read as row fragments and transposed) and V (row
    // fragments), both with swizzle pq_swz
    __shared__ __attribute__((aligned(16))) uint16_t tiles[2][2][TILE];

    const int n_rt = (g.R + Q_ROWS - 1) / Q_ROWS;
    int rt, bh, split;
    decode_block_at(blk, nblk, n_rt, nsplit, rt, bh, split);
    const int b = bh / g.Hkv, h = bh % g.Hkv;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, l32 = lane & 31;
    const int wr0 = rt * Q_ROWS + wave * BR;         // the wave's first packed row
    const int r = wr0 + l32;                         // this lane's packed row
    const bool rok = r < g.R;
    const int rr = rok ? r : g.R - 1;
    const int i = rr / g.G;                          // its query
    const size_t head_row = ((size_t)b * g.Hq + (size_t)h * g.G + rr % g.G) * g.S + i;
    // a key block [kk0, kk0 + 32) is wholly visible to the wave's rows iff
    // they all exist, the keys exist, and (chunk keys) kk0 + 31 <= the
    // smallest query of the rows
    const bool rows_all = wr0 + BR <= g.R;
    const int i_min = wr0 / g.G;

    // Q and dO fragments of the row: B operands of S^T = K Q^T and dP^T = V dO^T
    bf16x8 qf[D / 16], of[D / 16];
    load_key_frags<D>(qf, q + head_row * D, rok, half);
    load_key_frags<D>(of, dout + head_row * D, rok, half);
    const float l2r = l2[(size_t)bh * g.R + rr];
    const float drr = drow[(size_t)bh * g.R + rr];

    // key tiles: the n valid cache slots, then the chunk keys up to the last
    // query of this row tile
    const int n_ct = (g.n + Q_KT - 1) / Q_KT;
    const int r_last = min((rt + 1) * Q_ROWS, g.R) - 1;
    const int total = n_ct + (r_last / g.G) / Q_KT + 1;
    const int t_begin = (int)((long)split * total / nsplit);
    const int t_end = (int)((long)(split + 1) * total / nsplit);
    const uint16_t* kc_bh = kc + (size_t)bh * g.C * D;
    const uint16_t* vc_bh = vc + (size_t)bh * g.C * D;
    const uint16_t* kn_bh = kn + (size_t)bh * g.S * D;
    const uint16_t* vn_bh = vn + (size_t)bh * g.S * D;
    // lane byte offsets of the K and V copies inside a tile (both use pq_swz)
    constexpr int ITER = Q_KT * CPR / (Q_WAVES * 64);
    static_assert(ITER * Q_WAVES * 64 == Q_KT * CPR, "whole 1 KiB blocks");
    uint32_t coff[ITER];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        const int p = (it * Q_WAVES + wave) * 64 + lane;
        const int key = p / CPR;
        coff[it] = 2u * (uint32_t)(key * D + (((p % CPR) ^ pq_swz<D>(key)) << 3));
    }
    auto issue = [&](auto BUFC, int t) {
        constexpr int BUF = decltype(BUFC)::value;
        const bool ch = t >= n_ct;
        const int k0 = ch ? (t - n_ct) * Q_KT : t * Q_KT;
        const int lim = ch ? g.S : g.n;
        const uint16_t* ksrc = ch ? kn_bh : kc_bh;
        const uint16_t* vsrc = ch ? vn_bh : vc_bh;
        const uint32_t kb_lds = __builtin_amdgcn_readfirstlane(lds_addr(tiles[BUF][0]));
        if (!ch && k0 + Q_KT <= g.n) {
            // every row exists: scalar base (row k0) and the fixed lane offsets
            const uint16_t* kb = uniform_ptr(ksrc + (size_t)k0 * D);
            const uint16_t* vb = uniform_ptr(vsrc + (size_t)k0 * D);
#pragma unroll
            for (int it = 0; it < ITER; ++it) {
                dma16_s(kb, coff[it], kb_lds + (it * Q_WAVES + wave) * 1024);
                dma16_s(vb, coff[it], kb_lds + TILE * 2 + (it * Q_WAVES + wave) * 1024);
            }
            return;
        }
#pragma unroll
        for (int it = 0; it < ITER; ++it) {
            const int blk = it * Q_WAVES + wave;
            const int p = blk * 64 + lane;
            const int key = p / CPR;
            const size_t src = (size_t)min(k0 + key, lim - 1) * D + ((p % CPR) ^ pq_swz<D>(key)) * 8;
            dma16(ksrc + src, kb_lds + blk * 1024);
            dma16(vsrc + src, kb_lds + TILE * 2 + blk * 1024);
        }
    };

    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[db][v] = 0.f;
    // per-lane LDS byte addresses in buffer 0 (key blocks 32 rows further on,
    // and rows 16 further on, add immediates):
    //   kra[ks]: row fragments of K (key l32, dims 16*ks + 8*half + [0, 8));
    //            those of V are one tile further on;
    //   kta[k][db]: transposed K for keys 8*k + 4*half + (lane%16)/4, dims
    //               32*db + 16*((lane/16)%2) + 4*(lane%4) + [0, 4)
    uint32_t kra[D / 16], kta[2][NDB];
    {
        const uint32_t kbase = lds_addr(tiles[0][0]);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            kra[ks] = kbase + 2u * (uint32_t)(l32 * D + (((2 * ks + half) ^ pq_swz<D>(l32)) << 3));
        const int j = lane & 15;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int kr = 8 * k + 4 * half + (j >> 2);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const int d = db * 32 + (lane & 16) + 4 * (j & 3);
                kta[k][db] =
                    kbase + 2u * (uint32_t)(kr * D + (((d >> 3) ^ pq_swz<D>(kr)) << 3) + (d & 7));
            }
        }
    }
    const float c = g.c;

    auto step = [&](auto BUFC, int t) {
        constexpr int BUF = decltype(BUFC)::value;
        if (t + 1 < t_end) issue(IntC<BUF ^ 1>{}, t + 1);
        const bool ch = t >= n_ct;
        const int k0 = ch ? (t - n_ct) * Q_KT : t * Q_KT;
        const int lim = ch ? g.S : g.n;
#pragma unroll
        for (int kb = 0; kb < Q_KT / BR; ++kb) {
            const uint32_t ob = BUF * BUF_B + (uint32_t)(kb * BR) * 2 * D;
            // S^T = K Q^T and dP^T = V dO^T: element v is key
            // k0 + 32*kb + 8*(v/4) + 4*half + v%4 against this lane's row
            f32x16 s, dp;
#pragma unroll
            for (int v = 0; v < 16; ++v) s[v] = dp[v] = 0.f;
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                s = mfma32x32x16(as_bf16x8(lds_ld16(kra[ks] + ob)), qf[ks], s);
                dp = mfma32x32x16(as_bf16x8(lds_ld16(kra[ks] + ob + TILE * 2)), of[ks], dp);
            }
            bf16x8 sf[2];
            const int kk0 = k0 + kb * BR;
            if (rows_all && kk0 + BR <= lim && (!ch || kk0 + BR - 1 <= i_min)) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const float p = fast_exp2(fmaf(s[v], c, -l2r));
                    sf[v >> 3][v & 7] = (__bf16)(p * (dp[v] - drr));
                }
            } else {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int kk = kk0 + acc_row(v, half);
                    const bool vis = rok && kk < lim && (!ch || kk <= i);
                    const float p = vis ? fast_exp2(fmaf(s[v], c, -l2r)) : 0.f;
                    const float ds = vis ? p * (dp[v] - drr) : 0.f;
                    sf[v >> 3][v & 7] = (__bf16)ds;
                }
            }
            // dQ^T += K^T dS^T
#pragma unroll
            for (int hs = 0; hs < 2; ++hs) {
                const uint32_t o = ob + (uint32_t)(16 * hs) * 2 * D;
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const u32x2 lo = lds_ld_tr(kta[0][db] + o);
                    const u32x2 hi = lds_ld_tr(kta[1][db] + o);
                    acc[db] = mfma32x32x16(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}),
                                           sf[hs], acc[db]);
                }
            }
        }
        wait_tiles();
        __syncthreads();
    };

    if (t_begin < t_end) issue(IntC<0>{}, t_begin);
    wait_tiles();
    __syncthreads();
    for (int t = t_begin; t < t_end; t += 2) {
        step(IntC<0>{}, t);
        if (t + 1 < t_end) step(IntC<1>{}, t + 1);
    }
    if (!rok) return;
    // one key split: dQ itself; several: this split's partial (scaled later)
    const float sc = nsplit == 1 ? g.tau : 1.f;
    float* dqr = (nsplit == 1 ? dq : dq_part + (size_t)split * g.B * g.Hq * g.S * D) + head_row * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const int d = db * 32 + 8 * gq + 4 * half;
            *(f32x4*)(dqr + d) = sc * f32x4{acc[db][4 * gq + 0], acc[db][4 * gq + 1],
                                            acc[db][4 * gq + 2], acc[db][4 * gq + 3]};
        }
}

template <int D>
__global__ __launch_bounds__(Q_NT, 1) void bwd_dq_kernel(
    const BwdGeom g, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const uint16_t* __restrict__ kn,
    const uint16_t* __restrict__ vn, const uint16_t* __restrict__ dout,
    const float* __restrict__ l2, const float* __restrict__ drow, const int nsplit,
    float* __restrict__ dq, float* __restrict__ dq_part) {
    dq_body<D>(blockIdx.x, gridDim.x, g, q, kc, vc, kn, vn, dout, l2, drow, nsplit, dq, dq_part);
}

// dK/dV and dQ in one grid: the first n_dkdv workgroups are dK/dV key tiles,
// the rest dQ workgroups.  The two are independent, and the dQ workgroups,
// dispatched after every dK/dV one, fill the CUs that the last, partial
// round of dK/dV key tiles leaves idle (at the 128k shape 1088 key tiles
// make 4.25 rounds of 256).  Both halves take 8 waves and about 205 VGPRs
// per lane, so the fused kernel keeps one workgroup per CU.
template <int D>
__global__ __launch_bounds__(PQ_NT, 1) void bwd_dkdv_dq_kernel(
    const BwdGeom g, const int n_dkdv, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn,
    const uint16_t* __restrict__ dout, const float* __restrict__ l2,
    const float* __restrict__ drow, float* __restrict__ dkc, float* __restrict__ dvc,
    float* __restrict__ dkn, float* __restrict__ dvn, const int nsplit,
    float* __restrict__ dq, float* __restrict__ dq_part) {
    static_assert(PQ_NT == Q_NT, "one block size for both halves");
    const int L = blockIdx.x;
    if (L < n_dkdv)
        dkdv_pair_body<D>(L, g, q, kc, vc, kn, vn, dout, l2, drow, dkc, dvc, dkn, dvn);
    else
        dq_body<D>(L - n_dkdv, (int)gridDim.x - n_dkdv, g, q, kc, vc, kn, vn, dout, l2, drow,
                   nsplit, dq, dq_part);
}

// dQ = scale * (sum of the key splits' partials, in split order)
__global__ __launch_bounds__(256) void bwd_dq_reduce_kernel(const float* __restrict__ part,
                                                           int nsplit, long n4, float tau,
                                                           float* __restrict__ dq) {
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n4; i += (long)gridDim.x * 256) {
        f32x4 acc = ((const f32x4*)part)[i];
        for (int sp = 1; sp < nsplit; ++sp) acc += ((const f32x4*)part)[sp * n4 + i];
        ((f32x4*)dq)[i] = tau * acc;
    }
}

// Key splits of the query-major kernel: enough workgroups for the 256 CUs,
// at least 4 key tiles each; a function of the shape only (n = C assumed).
int bwd_dq_splits(const BwdGeom& g) {
    const int base = g.B * g.Hkv * ((g.R + Q_ROWS - 1) / Q_ROWS);
    const int max_tiles = (g.C + Q_KT - 1) / Q_KT + (g.S + Q_KT - 1) / Q_KT;
    int sp = (256 + base - 1) / base;
    sp = sp > 4 ? 4 : sp;
    const int cap = max_tiles / 4 < 1 ? 1 : max_tiles / 4;
    return sp > cap ? cap : sp;
}

template <int D>
hipError_t launch_bwd_d(const BwdGeom& g, const uint16_t* q, const uint16_t* kc,
                        const uint16_t* vc, const uint16_t* kn, const uint16_t* vn,
                        const float* out, const float* lse, const uint16_t* dout, float* dq,
                        float* dkc, float* dvc, float* dkn, float* dvn, void* ws,
                        hipStream_t stream, bool sync_debug, hipEvent_t* ev) {
    const int BH = g.B * g.Hkv;
    float* l2 = (float*)ws;
    float* drow = l2 + bwd_rows_padded(g);
    hipError_t err;
#define H2O_CHECK()                                  \
    do {                                             \
        err = hipGetLastError();                     \
        if (err != hipSuccess) return err;           \
        if (sync_debug) {                            \
            err = hipStreamSynchronize(stream);      \
            if (err != hipSuccess) return err;       \
        }                                            \
    } while (0)
#define H2O_EVENT(i)                                                               \
    do {                                                                           \
        if (ev && (err = hipEventRecord(ev[i], stream)) != hipSuccess) return err; \
    } while (0)
    H2O_EVENT(0);
    {
        const long threads = (long)BH * g.R * (D / 8);
        hipLaunchKernelGGL(bwd_prep_kernel<D>, dim3((unsigned)((threads + 255) / 256)), dim3(256),
                           0, stream, g, out, lse, dout, l2, drow);
        H2O_CHECK();
    }
    H2O_EVENT(1);
    const int n_rt = (g.R + Q_ROWS - 1) / Q_ROWS;
    const int nsplit = bwd_dq_splits(g);
    float* part = drow + bwd_rows_padded(g);
    if constexpr (D == 128) {
        // dK/dV and dQ in one grid (the dQ workgroups fill the dK/dV tail)
        const int n_kt = (g.C + PQ_KEYS - 1) / PQ_KEYS + (g.S + PQ_KEYS - 1) / PQ_KEYS;
        const int n_dkdv = BH * n_kt;
        hipLaunchKernelGGL(bwd_dkdv_dq_kernel<D>, dim3(n_dkdv + BH * n_rt * nsplit), dim3(PQ_NT),
                           0, stream, g, n_dkdv, q, kc, vc, kn, vn, dout, l2, drow, dkc, dvc,
                           dkn, dvn, nsplit, dq, part);
        H2O_CHECK();
        H2O_EVENT(2);
    } else {
        constexpr int KV_KEYS = kv_keys<D>();
        const int n_kt = (g.C + KV_KEYS - 1) / KV_KEYS + (g.S + KV_KEYS - 1) / KV_KEYS;
        hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3(BH * n_kt), dim3(KV_NT), 0, stream, g, q, kc,
                           vc, kn, vn, dout, l2, drow, dkc, dvc, dkn, dvn);
        H2O_CHECK();
        H2O_EVENT(2);
        hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3(BH * n_rt * nsplit), dim3(Q_NT), 0, stream, g,
                           q, kc, vc, kn, vn, dout, l2, drow, nsplit, dq, part);
        H2O_CHECK();
    }
    if (nsplit > 1) {
        const long n4 = (long)g.B * g.Hq * g.S * D / 4;
        long blocks = (n4 + 255) / 256;
        if (blocks > 8192) blocks = 8192;
        hipLaunchKernelGGL(bwd_dq_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                           part, nsplit, n4, g.tau, dq);
        H2O_CHECK();
    }
    H2O_EVENT(3);
    H2O_EVENT(4);
#undef H2O_CHECK
#undef H2O_EVENT
    return hipSuccess;
}

}  // namespace

size_t bwd_rows_padded(const BwdGeom& g) {
    const size_t rows = (size_t)g.B * g.Hkv * g.R;
    return (rows + 63) & ~(size_t)63;
}

size_t bwd_workspace_bytes(const BwdGeom& g) {
    const int nsplit = bwd_dq_splits(g);
    const size_t part = nsplit > 1 ? (size_t)nsplit * g.B * g.Hq * g.S * g.D : 0;
    return (2 * bwd_rows_padded(g) + part) * sizeof(float);
}

hipError_t launch_attention_bwd(const BwdGeom& g, const uint16_t* q, const uint16_t* kc,
                                const uint16_t* vc, const uint16_t* kn, const uint16_t* vn,
                                const float* out, const float* lse, const uint16_t* dout,
                                float* dq, float* dkc, float* dvc, float* dkn, float* dvn,
                                void* ws, hipStream_t stream, bool sync_debug,
                                hipEvent_t* ev5) {
    if (g.D == 64)
        return launch_bwd_d<64>(g, q, kc, vc, kn, vn, out, lse, dout, dq, dkc, dvc, dkn, dvn, ws,
                                stream, sync_debug, ev5);
    return launch_bwd_d<128>(g, q, kc, vc, kn, vn, out, lse, dout, dq, dkc, dvc, dkn, dvn, ws,
                             stream, sync_debug, ev5);
}

}  // namespace h2o
