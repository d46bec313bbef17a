// H2O cache policy on gfx950: score accumulation, choice of the slots to
// overwrite, and the scatter of the chunk into them.
//
// Method: "Learning how to Forget: Fine-tuning for Long-Context Sparse
// Attention" -- Chinese translation page §1 (a fixed number of slots; evict by
// policy once the cache is full) and §2 (summed attention weights as the H2O
// score); Korean summary page, glossary entry for H2O (entries that were
// attended to least are evicted).
#include "h2o_device.h"
#include "h2o_launch.h"

namespace h2o {
namespace {

// ---------------------------------------------------------------------------
// score accumulation: scores[j] += wsum[j] (j < n); new[t] = wsum[C + t]
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void score_accumulate_kernel(
    int BH, int C, int S, int n, float* __restrict__ scores,
    float* __restrict__ new_scores, const float* __restrict__ wsum) {
    const int W = C + S;
    const long total = (long)BH * W;
    for (long idx = (long)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (long)gridDim.x * blockDim.x) {
        const int bh = (int)(idx / W), j = (int)(idx % W);
        const float w = wsum[idx];
        if (j < n)
            scores[(size_t)bh * C + j] += w;
        else if (j >= C)
            new_scores[(size_t)bh * S + (j - C)] = w;
    }
}

// ---------------------------------------------------------------------------
// slot choice
// ---------------------------------------------------------------------------
// Order-preserving map of a score onto uint32: -0.0 == +0.0, NaN above +inf.
// Every mapped score is >= 0x007FFFFF (the image of -inf), so key 0 is free
// for empty slots, which are taken first.
__device__ __forceinline__ uint32_t score_key(float x) {
    uint32_t u = __float_as_uint(x);
    if (x != x) return 0xFFFFFFFFu;
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int SEL_T = 1024;   // threads per (b, kv head)

__device__ __forceinline__ uint32_t slot_key(const float* __restrict__ sc, int j, int n) {
    return (j < n) ? score_key(sc[j]) : 0u;
}

// Exclusive prefix sum over the block (1024 threads, 16 waves).
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t x, uint32_t* sh_wave) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t inc = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(inc, off, 64);
        if (lane >= off) inc += y;
    }
    if (lane == 63) sh_wave[wave] = inc;
    __syncthreads();
    if (wave == 0) {
        uint32_t t = (lane < SEL_T / 64) ? sh_wave[lane] : 0u;
        uint32_t ti = t;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t y = __shfl_up(ti, off, 64);
            if (lane >= off) ti += y;
        }
        if (lane < SEL_T / 64) sh_wave[lane] = ti - t;   // exclusive wave offsets
    }
    __syncthreads();
    const uint32_t res = sh_wave[wave] + inc - x;
    __syncthreads();
    return res;
}

// Add 1 to hist[bin] for every active lane.  Lanes of the wave whose bin
// equals the first active lane's bin are folded into a single atomic (the
// top digits of real scores are nearly all equal, which would otherwise
// serialise 64 same-address LDS atomics per instruction).
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t bin, bool active) {
    const unsigned long long act = __ballot(active);
    if (act == 0ull) return;
    const int lead = __builtin_ctzll(act);
    const uint32_t lead_bin = __shfl(bin, lead, 64);
    const bool same = active && bin == lead_bin;
    const unsigned long long m = __ballot(same);
    if ((int)(threadIdx.x & 63) == lead) atomicAdd(&hist[lead_bin], (uint32_t)__popcll(m));
    if (active && !same) atomicAdd(&hist[bin], 1u);
}

// One workgroup per (b, kv head).  Each thread holds the keys of a
// contiguous run of KPT slots in registers.  Radix select (4 passes of 8
// bits) finds the key T of the S-th smallest (key, slot) pair and how many
// slots with key T are taken; a slot-ordered compaction (block prefix sums
// over the threads' runs) then writes the chosen slots in increasing order.
template <int KPT>
__global__ __launch_bounds__(SEL_T) void evict_select_kernel(
    int C, int S, int n, const float* __restrict__ scores, int32_t* __restrict__ evict) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t sh_wave[SEL_T / 64];
    __shared__ uint32_t sh_digit, sh_k;
    __shared__ unsigned long long sh_min;

    const int bh = blockIdx.x, tid = threadIdx.x;
    const float* sc = scores + (size_t)bh * C;
    int32_t* out = evict + (size_t)bh * S;

    if (n + S <= C) {   // fill phase: append
        for (int t = tid; t < S; t += SEL_T) out[t] = n + t;
        return;
    }
    const int j0 = tid * KPT;
    uint32_t key[KPT];
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
        const int j = j0 + e;
        key[e] = (j < C) ? slot_key(sc, j, n) : 0xFFFFFFFFu;
    }
    // slots past C carry key ~0 and must never be counted or taken
    const int cnt = max(0, min(KPT, C - j0));

    if (S == 1) {   // cache full (n == C): lexicographic min of (key, slot)
        unsigned long long best = ~0ull;
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            const unsigned long long kj = ((unsigned long long)key[e] << 32) | (unsigned)(j0 + e);
            best = (e < cnt && kj < best) ? kj : best;
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const unsigned long long o = __shfl_xor(best, off, 64);
            best = o < best ? o : best;
        }
        if (tid == 0) sh_min = ~0ull;
        __syncthreads();
        if ((tid & 63) == 0) atomicMin(&sh_min, best);
        __syncthreads();
        if (tid == 0) out[0] = (int32_t)(sh_min & 0xFFFFFFFFull);
        return;
    }

    uint32_t prefix = 0u, mask = 0u, k = (uint32_t)S;   // k: 1-based rank
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int i = tid; i < 256; i += SEL_T) hist[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < KPT; ++e)
            hist_add(hist, (key[e] >> shift) & 255u, e < cnt && (key[e] & mask) == prefix);
        __syncthreads();
        if (tid < 64) {   // one wave finds the bucket holding rank k
            uint32_t h4[4], s4 = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) { h4[e] = hist[tid * 4 + e]; s4 += h4[e]; }
            uint32_t inc = s4;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t y = __shfl_up(inc, off, 64);
                if (tid >= off) inc += y;
            }
            uint32_t before = inc - s4;
            if (before < k && k <= inc) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (before < k && k <= before + h4[e]) {
                        sh_digit = (uint32_t)(tid * 4 + e);
                        sh_k = k - before;
                    }
                    before += h4[e];
                }
            }
        }
        __syncthreads();
        prefix |= sh_digit << shift;
        mask |= 255u << shift;
        k = sh_k;
        __syncthreads();
    }
    const uint32_t T = prefix;

    uint32_t n_eq = 0, n_lt = 0;
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
        n_eq += (e < cnt && key[e] == T);
        n_lt += (e < cnt && key[e] < T);
    }
    const uint32_t eq_before = block_exclusive_scan(n_eq, sh_wave);
    const uint32_t eq_take = (k > eq_before) ? min(k - eq_before, n_eq) : 0u;
    const uint32_t out_before = block_exclusive_scan(n_lt + eq_take, sh_wave);
    uint32_t o = out_before, eq_seen = 0;
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
        if (e >= cnt) break;
        bool take = key[e] < T;
        if (key[e] == T) {
            take = eq_seen < eq_take;
            ++eq_seen;
        }
        if (take) {
            if (o < (uint32_t)S) out[o] = j0 + e;   // never past the row, whatever the counts
            ++o;
        }
    }
}

// ---------------------------------------------------------------------------
// scatter: chunk token t -> slot evict[t]
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void kv_scatter_kernel(
    int C, int S, uint16_t* __restrict__ kc, uint16_t* __restrict__ vc,
    float* __restrict__ scores, int64_t* __restrict__ pos,
    const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn,
    const float* __restrict__ new_scores, const int32_t* __restrict__ evict,
    int64_t p0) {
    constexpr int TPR = D / 8;            // threads per row (16 B each)
    constexpr int TOK = 256 / (2 * TPR);  // tokens per workgroup
    const int bh = blockIdx.y, tid = threadIdx.x;
    const int tok = tid / (2 * TPR), which = (tid / TPR) & 1, c = tid % TPR;
    const int t = blockIdx.x * TOK + tok;
    if (t >= S) return;
    const int slot = evict[(size_t)bh * S + t];
    if (slot < 0 || slot >= C) return;   // out-of-range index: nothing written
    const uint16_t* src = (which ? vn : kn) + ((size_t)bh * S + t) * D + c * 8;
    uint16_t* dst = (which ? vc : kc) + ((size_t)bh * C + slot) * D + c * 8;
    *(u32x4*)dst = *(const u32x4*)src;
    if (which == 0 && c == 0) {
        scores[(size_t)bh * C + slot] = new_scores[(size_t)bh * S + t];
        if (pos) pos[(size_t)bh * C + slot] = p0 + t;
    }
}

}  // namespace

hipError_t launch_score_accumulate(int BH, int C, int S, int n, float* scores,
                                   float* new_scores, const float* wsum,
                                   hipStream_t stream) {
    const long total = (long)BH * (C + S);
    long blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(score_accumulate_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       BH, C, S, n, scores, new_scores, wsum);
    return hipGetLastError();
}

hipError_t launch_evict_select(int BH, int C, int S, int n, const float* scores,
                               int32_t* evict_idx, hipStream_t stream) {
    // keys per thread: the smallest supported run that covers C
    const int kpt = (C + SEL_T - 1) / SEL_T;
    if (kpt <= 4)
        hipLaunchKernelGGL(evict_select_kernel<4>, dim3(BH), dim3(SEL_T), 0, stream, C, S, n,
                           scores, evict_idx);
    else if (kpt <= 16)
        hipLaunchKernelGGL(evict_select_kernel<16>, dim3(BH), dim3(SEL_T), 0, stream, C, S, n,
                           scores, evict_idx);
    else if (kpt <= 64)
        hipLaunchKernelGGL(evict_select_kernel<64>, dim3(BH), dim3(SEL_T), 0, stream, C, S, n,
                           scores, evict_idx);
    else
        return hipErrorInvalidValue;   // rejected earlier by the shape check
    return hipGetLastError();
}

hipError_t launch_kv_scatter(int BH, int D, int C, int S, uint16_t* kc, uint16_t* vc,
                             float* scores, int64_t* pos, const uint16_t* kn,
                             const uint16_t* vn, const float* new_scores,
                             const int32_t* evict_idx, int64_t p0, hipStream_t stream) {
    if (D == 64) {
        constexpr int TOK = 256 / (2 * (64 / 8));
        hipLaunchKernelGGL(kv_scatter_kernel<64>, dim3((S + TOK - 1) / TOK, BH), dim3(256), 0,
                           stream, C, S, kc, vc, scores, pos, kn, vn, new_scores, evict_idx, p0);
    } else {
        constexpr int TOK = 256 / (2 * (128 / 8));
        hipLaunchKernelGGL(kv_scatter_kernel<128>, dim3((S + TOK - 1) / TOK, BH), dim3(256), 0,
                           stream, C, S, kc, vc, scores, pos, kn, vn, new_scores, evict_idx, p0);
    }
    return hipGetLastError();
}

}  // namespace h2o
