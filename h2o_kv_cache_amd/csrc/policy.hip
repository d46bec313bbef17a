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
// grid: (column blocks, BH); each thread handles columns j and j + 256*gridDim.x ...
__global__ __launch_bounds__(256) void score_accumulate_kernel(
    int BH, int C, int S, int n, float* __restrict__ scores,
    float* __restrict__ new_scores, const float* __restrict__ wsum) {
    const int W = C + S;
    const int bh = blockIdx.y;
    const float* wrow = wsum + (size_t)bh * W;
    for (int j = blockIdx.x * 256 + threadIdx.x; j < W; j += gridDim.x * 256) {
        if (j < n)
            scores[(size_t)bh * C + j] += wrow[j];
        else if (j >= C)
            new_scores[(size_t)bh * S + (j - C)] = wrow[j];
    }
}

// ---------------------------------------------------------------------------
// slot choice
// ---------------------------------------------------------------------------
constexpr int SEL_T = 1024;   // threads per (b, kv head)
constexpr int SEL_SLOTS = 4096;   // choices kept in LDS for the fused scatter

__device__ __forceinline__ uint32_t slot_key(const float* __restrict__ sc, int j, int n) {
    return (j < n) ? score_key(sc[j]) : 0u;
}

constexpr int SU = 16;   // 64-slot steps whose keys are loaded together

// Keys of slots base + 64*u + lane (u < SU) of a contiguous range ending at
// `last`: the SU loads are unconditional (index clamped to `last`) and are
// all issued before any is used -- the empty asm takes every loaded value,
// so the compiler cannot sink a load into a branch of its own; slots past
// `last` get key 0 and must be masked by the caller.
__device__ __forceinline__ void load_keys(uint32_t (&key)[SU], const float* __restrict__ sc,
                                          int base, int lane, int n, int last) {
    float x[SU];
#pragma unroll
    for (int u = 0; u < SU; ++u) x[u] = sc[min(base + 64 * u + lane, last)];
    asm volatile(""
                 : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]),
                   "+v"(x[6]), "+v"(x[7]), "+v"(x[8]), "+v"(x[9]), "+v"(x[10]), "+v"(x[11]),
                   "+v"(x[12]), "+v"(x[13]), "+v"(x[14]), "+v"(x[15]));
#pragma unroll
    for (int u = 0; u < SU; ++u) {
        const int j = base + 64 * u + lane;
        key[u] = (j < n && j <= last) ? score_key(x[u]) : 0u;
    }
}

// Add 1 to hist[bin] for every active lane.  Lanes of the wave whose bin
// equals the first active lane's bin are folded into a single atomic (the
// top digits of real scores are nearly all equal, which would otherwise
// serialise 64 same-address LDS atomics per instruction).
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t bin, bool active) {
    const unsigned long long act = __ballot(active);
    if (act == 0ull) return;
    const int lead = __builtin_ctzll(act);   // wave-uniform (from a ballot)
    const uint32_t lead_bin = __builtin_amdgcn_readlane(bin, lead);
    const bool same = active && bin == lead_bin;
    const unsigned long long m = __ballot(same);
    if ((int)(threadIdx.x & 63) == lead) atomicAdd(&hist[lead_bin], (uint32_t)__popcll(m));
    if (active && !same) atomicAdd(&hist[bin], 1u);
}

// Run by one wave (lanes 0-63): the bin of a 256-bin histogram that holds
// rank k (1-based, counting from bin 0), and the rank inside that bin.
__device__ __forceinline__ void find_bin(const uint32_t* hist, uint32_t k, uint32_t* sh_digit,
                                         uint32_t* sh_k) {
    const int lane = threadIdx.x & 63;
    uint32_t h4[4], s4 = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        h4[e] = hist[lane * 4 + e];
        s4 += h4[e];
    }
    uint32_t inc = s4;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(inc, off, 64);
        if (lane >= off) inc += y;
    }
    uint32_t before = inc - s4;
    if (before < k && k <= inc) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (before < k && k <= before + h4[e]) {
                *sh_digit = (uint32_t)(lane * 4 + e);
                *sh_k = k - before;
            }
            before += h4[e];
        }
    }
}

// Every wave computes the same result as find_bin from the shared histogram
// (no broadcast through LDS, hence no barrier after it): the digit of the bin
// that holds rank k and the rank inside that bin.  k must not exceed the
// histogram's total.
__device__ __forceinline__ void find_bin_wave(const uint32_t* hist, uint32_t k,
                                              uint32_t& digit, uint32_t& k_in) {
    const int lane = threadIdx.x & 63;
    uint32_t h4[4], s4 = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        h4[e] = hist[lane * 4 + e];
        s4 += h4[e];
    }
    uint32_t inc = s4;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(inc, off, 64);
        if (lane >= off) inc += y;
    }
    uint32_t before = inc - s4, d = 0, kk = 0;
    const bool here = before < k && k <= inc;
    if (here) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (before < k && k <= before + h4[e]) {
                d = (uint32_t)(lane * 4 + e);
                kk = k - before;
            }
            before += h4[e];
        }
    }
    const unsigned long long m = __ballot(here);
    const int src = m ? __builtin_ctzll(m) : 0;
    digit = __builtin_amdgcn_readlane(d, src);
    k_in = __builtin_amdgcn_readlane(kk, src);
}

// Exclusive prefix sums of two counts over the block (1024 threads).
__device__ __forceinline__ void block_exclusive_scan2(uint32_t x, uint32_t y, uint32_t* sh,
                                                      uint32_t& xb, uint32_t& yb) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t ix = x, iy = y;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t a = __shfl_up(ix, off, 64), c = __shfl_up(iy, off, 64);
        if (lane >= off) {
            ix += a;
            iy += c;
        }
    }
    if (lane == 63) {
        sh[wave] = ix;
        sh[SEL_T / 64 + wave] = iy;
    }
    __syncthreads();
    uint32_t ox = 0, oy = 0;
    for (int w = 0; w < wave; ++w) {   // wave-uniform loop over the earlier waves' totals
        ox += sh[w];
        oy += sh[SEL_T / 64 + w];
    }
    xb = ox + ix - x;
    yb = oy + iy - y;
}

// One workgroup per (b, kv head).  Each thread holds the keys of a
// contiguous run of KPT slots in registers.  Radix select (4 passes of 8
// bits) finds the key T of the S-th smallest (key, slot) pair and how many
// slots with key T are taken; a slot-ordered compaction (block prefix sums
// over the threads' runs) then writes the chosen slots in increasing order.
// The histograms rotate over three LDS buffers, so that a pass needs one
// barrier: pass p fills buffer p % 3 and clears buffer (p + 1) % 3, which
// the waves last read in pass p - 2 (before pass p - 1's barrier).  Passes
// over leading bytes that every key shares are skipped.
// DS > 0: the kernel also scatters the chunk into the chosen slots (the
// work of kv_scatter_kernel for head dim DS), after the choice is in `evict`.
template <int KPT, int DS>
__global__ __launch_bounds__(SEL_T) void evict_select_kernel(
    int C, int S, int n, float* __restrict__ scores, int32_t* __restrict__ evict,
    uint16_t* __restrict__ kc, uint16_t* __restrict__ vc, int64_t* __restrict__ pos,
    const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn,
    const float* __restrict__ new_scores, int64_t p0) {
    __shared__ uint32_t hist[3][256];
    __shared__ uint32_t sh_scan[2 * (SEL_T / 64)];
    __shared__ unsigned long long sh_min;
    __shared__ uint32_t sh_lohi[2][SEL_T / 64];   // per wave: smallest and largest key
    __shared__ int32_t sh_slot[DS > 0 ? SEL_SLOTS : 1];   // the choice, for the scatter

    const int bh = blockIdx.x, tid = threadIdx.x;
    float* sc = scores + (size_t)bh * C;
    int32_t* out = evict + (size_t)bh * S;

    // the scatter of chunk token t into slot out[t] (from sh_slot when S <=
    // SEL_SLOTS, else from `out`), once the choice is complete (written by
    // this workgroup before the barrier that precedes the call); a thread
    // moves up to 4 pieces of 16 bytes, all loaded before any is stored
    auto scatter = [&]() {
        if constexpr (DS > 0) {
            constexpr int TPR = DS / 8;   // 16-byte pieces per row
            constexpr int U = 4;
            const int total = S * 2 * TPR;
            for (int i0 = tid; i0 < total; i0 += U * SEL_T) {
                u32x4 v[U];
                int slot[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int i = i0 + u * SEL_T;
                    slot[u] = -1;
                    if (i >= total) continue;
                    const int t = i / (2 * TPR), which = (i / TPR) & 1, c = i % TPR;
                    slot[u] = S <= SEL_SLOTS ? sh_slot[t] : out[t];
                    v[u] = *(const u32x4*)((which ? vn : kn) + ((size_t)bh * S + t) * DS + c * 8);
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int i = i0 + u * SEL_T;
                    if (slot[u] < 0 || slot[u] >= C) continue;
                    const int t = i / (2 * TPR), which = (i / TPR) & 1, c = i % TPR;
                    *(u32x4*)((which ? vc : kc) + ((size_t)bh * C + slot[u]) * DS + c * 8) = v[u];
                    if (which == 0 && c == 0) {
                        sc[slot[u]] = new_scores[(size_t)bh * S + t];
                        if (pos) pos[(size_t)bh * C + slot[u]] = p0 + t;
                    }
                }
            }
        }
    };
    // record the choice of output position o (the scatter reads it back)
    auto put = [&](int o, int slot) {
        out[o] = slot;
        if constexpr (DS > 0)
            if (S <= SEL_SLOTS) sh_slot[o] = slot;
    };

    if (n + S <= C) {   // fill phase: append
        for (int t = tid; t < S; t += SEL_T) put(t, n + t);
        if constexpr (DS > 0) {
            __syncthreads();
            scatter();
        }
        return;
    }
    if (S == 1) {   // cache full (n == C): lexicographic min of (key, slot)
        // the minimum does not depend on which thread reads which slot, so
        // thread t takes slots t, t + SEL_T, ... (coalesced loads, all issued
        // before the compares)
        uint32_t kk[KPT];
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            const int j = e * SEL_T + tid;
            kk[e] = j < C ? slot_key(sc, j, n) : 0xFFFFFFFFu;
        }
        unsigned long long best = ~0ull;
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            const int j = e * SEL_T + tid;
            const unsigned long long kj = ((unsigned long long)kk[e] << 32) | (unsigned)j;
            best = (j < C && kj < best) ? kj : best;
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
        if (tid == 0) put(0, (int)(sh_min & 0xFFFFFFFFull));
        if constexpr (DS > 0) {
            __syncthreads();
            scatter();
        }
        return;
    }
    const int j0 = tid * KPT;
    uint32_t key[KPT];
    if ((C & 3) == 0) {   // 16-byte aligned rows: the run in 16-byte loads
        float4 x[KPT / 4];
#pragma unroll
        for (int e4 = 0; e4 < KPT / 4; ++e4)
            x[e4] = j0 + 4 * e4 < C ? *(const float4*)(sc + j0 + 4 * e4)
                                    : float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e4 = 0; e4 < KPT / 4; ++e4) {
            const float f[4] = {x[e4].x, x[e4].y, x[e4].z, x[e4].w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = j0 + 4 * e4 + u;
                key[4 * e4 + u] = j >= C ? 0xFFFFFFFFu : (j < n ? score_key(f[u]) : 0u);
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            const int j = j0 + e;
            key[e] = (j < C) ? slot_key(sc, j, n) : 0xFFFFFFFFu;
        }
    }
    // slots past C carry key ~0 and must never be counted or taken
    const int cnt = max(0, min(KPT, C - j0));

    // The leading bytes that every key shares need no pass: the smallest and
    // the largest key give them (and their pass would keep k).
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int e = 0; e < KPT; ++e)
        if (e < cnt) {
            lo = min(lo, key[e]);
            hi = max(hi, key[e]);
        }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        lo = min(lo, (uint32_t)__shfl_xor(lo, off, 64));
        hi = max(hi, (uint32_t)__shfl_xor(hi, off, 64));
    }
    if ((tid & 63) == 0) {
        sh_lohi[0][tid >> 6] = lo;
        sh_lohi[1][tid >> 6] = hi;
    }
    // all three buffers start cleared: the first pass that runs may be any
    for (int i = tid; i < 3 * 256; i += SEL_T) hist[i / 256][i % 256] = 0u;
    __syncthreads();
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
    for (int w = 0; w < SEL_T / 64; ++w) {
        kmin = min(kmin, sh_lohi[0][w]);
        kmax = max(kmax, sh_lohi[1][w]);
    }
    const uint32_t diff = kmin ^ kmax;
    const int first = diff == 0u ? 4 : __builtin_clz(diff) / 8;   // passes 0..first-1 skipped
    uint32_t mask = first >= 4 ? 0xFFFFFFFFu : (first == 0 ? 0u : ~0u << (32 - 8 * first));
    uint32_t prefix = kmin & mask, k = (uint32_t)S;   // k: 1-based rank
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
        if (pass < first) continue;   // workgroup-uniform
        const int shift = 24 - 8 * pass;
        uint32_t* h = hist[pass % 3];
        if (pass < 3)
            for (int i = tid; i < 256; i += SEL_T) hist[(pass + 1) % 3][i] = 0u;
#pragma unroll
        for (int e = 0; e < KPT; ++e)
            hist_add(h, (key[e] >> shift) & 255u, e < cnt && (key[e] & mask) == prefix);
        __syncthreads();
        uint32_t digit, k_in;
        find_bin_wave(h, k, digit, k_in);
        prefix |= digit << shift;
        mask |= 255u << shift;
        k = k_in;
    }
    const uint32_t T = prefix;

    uint32_t n_eq = 0, n_lt = 0;
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
        n_eq += (e < cnt && key[e] == T);
        n_lt += (e < cnt && key[e] < T);
    }
    // ties are taken in slot order: the threads before this one take
    // eq_prev = min(k, eq_before) of them, this one the next eq_take
    uint32_t eq_before, lt_before;
    block_exclusive_scan2(n_eq, n_lt, sh_scan, eq_before, lt_before);
    const uint32_t eq_prev = eq_before < k ? eq_before : k;
    const uint32_t eq_room = k - eq_prev;   // no wrap: eq_prev <= k
    const uint32_t eq_take = eq_room < n_eq ? eq_room : n_eq;
    uint32_t o = lt_before + eq_prev, eq_seen = 0;
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
        if (e >= cnt) break;
        bool take = key[e] < T;
        if (key[e] == T) {
            take = eq_seen < eq_take;
            ++eq_seen;
        }
        if (take) {
            if (o < (uint32_t)S) put((int)o, j0 + e);   // never past the row, whatever the counts
            ++o;
        }
    }
    if constexpr (DS > 0) {
        __syncthreads();
        scatter();
    }
}

// The same choice with the keys left in memory, for rows too long to hold in
// registers (more than SEL_T * 64 slots) and for the SnapKV keep list.  Wave w
// owns the contiguous slots [w*seg, (w+1)*seg) and walks them 64 at a time
// with coalesced loads, re-reading the keys (from L2) in every pass.  Slot
// order inside a 64-slot step comes from ballots, across steps from a running
// count, across waves from a scan of the 16 wave totals.
//   KEEP = false: out[0..k) = the k chosen slots (rows of `stride` floats,
//                 n valid; the fill phase appends as above)
//   KEEP = true : out[0..C-k) = the C - k slots not chosen (all C valid)
// Both lists are in increasing slot order.
constexpr int SEL_W = SEL_T / 64;

template <bool KEEP>
__global__ __launch_bounds__(SEL_T) void select_stream_kernel(
    int C, int k, int n, const float* __restrict__ scores, long stride,
    int32_t* __restrict__ out, long out_stride) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t sh_lt[SEL_W], sh_eq[SEL_W];
    __shared__ uint32_t sh_digit, sh_k;

    const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    const int wave = tid >> 6;
    const float* sc = scores + (size_t)bh * stride;
    int32_t* o = out + (size_t)bh * out_stride;
    const int n_out = KEEP ? C - k : k;

    if (!KEEP && n + k <= C) {   // fill phase: append
        for (int t = tid; t < k; t += SEL_T) o[t] = n + t;
        return;
    }
    if (k == 0) {   // KEEP only: every slot stays
        for (int j = tid; j < C; j += SEL_T) o[j] = j;
        return;
    }
    const int seg = (C + SEL_T - 1) / SEL_T * 64;
    const int s0 = min(C, wave * seg), s1 = min(C, s0 + seg);
    const unsigned long long below = (1ull << lane) - 1ull;

    uint32_t prefix = 0u, mask = 0u, kk = (uint32_t)k;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int i = tid; i < 256; i += SEL_T) hist[i] = 0u;
        __syncthreads();
        for (int base = s0; base < s1; base += 64 * SU) {
            uint32_t key[SU];
            bool in[SU];
            load_keys(key, sc, base, lane, n, s1 - 1);
#pragma unroll
            for (int u = 0; u < SU; ++u) in[u] = base + 64 * u + lane < s1;
#pragma unroll
            for (int u = 0; u < SU; ++u)
                hist_add(hist, (key[u] >> shift) & 255u, in[u] && (key[u] & mask) == prefix);
        }
        __syncthreads();
        if (tid < 64) find_bin(hist, kk, &sh_digit, &sh_k);
        __syncthreads();
        prefix |= sh_digit << shift;
        mask |= 255u << shift;
        kk = sh_k;
        __syncthreads();
    }
    const uint32_t T = prefix;   // key of the k-th smallest; kk of its ties are taken

    // per-wave counts below / at T, then the wave's share of the ties
    uint32_t n_lt = 0, n_eq = 0;
    for (int base = s0; base < s1; base += 64 * SU) {
        uint32_t key[SU];
        load_keys(key, sc, base, lane, n, s1 - 1);
#pragma unroll
        for (int u = 0; u < SU; ++u) {
            const int j = base + 64 * u + lane;
            n_lt += (uint32_t)__popcll(__ballot(j < s1 && key[u] < T));
            n_eq += (uint32_t)__popcll(__ballot(j < s1 && key[u] == T));
        }
    }
    if (lane == 0) {
        sh_lt[wave] = n_lt;
        sh_eq[wave] = n_eq;
    }
    __syncthreads();
    uint32_t eq_before = 0, taken = 0;
    for (int w = 0; w < wave; ++w) {
        const uint32_t e = sh_eq[w];
        const uint32_t take_w = kk > eq_before ? min(kk - eq_before, e) : 0u;
        taken += sh_lt[w] + take_w;
        eq_before += e;
    }
    const uint32_t eq_take = kk > eq_before ? min(kk - eq_before, n_eq) : 0u;

    uint32_t eq_seen = 0;
    for (int base0 = s0; base0 < s1; base0 += 64 * SU) {
      uint32_t keys[SU];
      load_keys(keys, sc, base0, lane, n, s1 - 1);
#pragma unroll
      for (int u = 0; u < SU; ++u) {
        const int base = base0 + 64 * u;
        const int j = base + lane;
        const bool in = j < s1;
        const uint32_t key = keys[u];
        const unsigned long long eqm = __ballot(in && key == T);
        const uint32_t eq_rank = eq_seen + (uint32_t)__popcll(eqm & below);
        const bool take = in && (key < T || (key == T && eq_rank < eq_take));
        const unsigned long long tm = __ballot(take);
        const uint32_t t_below = taken + (uint32_t)__popcll(tm & below);
        if (KEEP) {
            const uint32_t idx = (uint32_t)j - t_below;   // slots before j not taken
            if (in && !take && idx < (uint32_t)n_out) o[idx] = j;
        } else {
            if (take && t_below < (uint32_t)n_out) o[t_below] = j;
        }
        taken += (uint32_t)__popcll(tm);
        eq_seen += (uint32_t)__popcll(eqm);
      }
    }
}

// ---------------------------------------------------------------------------
// SnapKV compaction: output slot i < budget <- kept input slot keep[i];
// output slot budget + t <- chunk token t
// ---------------------------------------------------------------------------
// Each thread moves one 16-byte piece of a K or V row; a workgroup moves
// CP_ROWS rows, CP_UNROLL pieces per thread in flight.
constexpr int CP_UNROLL = 4;

template <int D>
__global__ __launch_bounds__(256) void kv_compact_kernel(
    int C, int S, int budget, int out_len, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int64_t* __restrict__ pos,
    const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn,
    const float* __restrict__ wsum, const int32_t* __restrict__ keep, int64_t p0,
    uint16_t* __restrict__ ko, uint16_t* __restrict__ vo, int64_t* __restrict__ pos_out,
    float* __restrict__ scores_out) {
    constexpr int TPR = D / 8;                 // 16-byte pieces per row
    constexpr int RPI = 256 / (2 * TPR);       // rows per unrolled step
    constexpr int CP_ROWS = RPI * CP_UNROLL;   // rows per workgroup
    const int bh = blockIdx.y, tid = threadIdx.x;
    const int which = (tid / TPR) & 1, c = tid % TPR, r_in = tid / (2 * TPR);
    const int total = budget + S;
    u32x4 v[CP_UNROLL];
    int dst[CP_UNROLL];
#pragma unroll
    for (int u = 0; u < CP_UNROLL; ++u) {
        const int i = blockIdx.x * CP_ROWS + u * RPI + r_in;
        dst[u] = -1;
        if (i >= total) continue;
        const uint16_t* src;
        if (i < budget) {
            const int slot = keep[(size_t)bh * budget + i];
            if (slot < 0 || slot >= C) continue;   // out-of-range index: nothing written
            src = (which ? vc : kc) + ((size_t)bh * C + slot) * D;
        } else {
            src = (which ? vn : kn) + ((size_t)bh * S + (i - budget)) * D;
        }
        v[u] = *(const u32x4*)(src + c * 8);
        dst[u] = i;
    }
#pragma unroll
    for (int u = 0; u < CP_UNROLL; ++u) {
        if (dst[u] < 0) continue;
        const int i = dst[u];
        *(u32x4*)((which ? vo : ko) + ((size_t)bh * out_len + i) * D + c * 8) = v[u];
        if (which == 0 && c == 0) {
            const bool kept = i < budget;
            const int slot = kept ? keep[(size_t)bh * budget + i] : 0;
            if (pos_out)
                pos_out[(size_t)bh * out_len + i] =
                    kept ? pos[(size_t)bh * C + slot] : p0 + (i - budget);
            if (scores_out)
                scores_out[(size_t)bh * out_len + i] =
                    wsum[(size_t)bh * (C + S) + (kept ? slot : C + (i - budget))];
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

// ---------------------------------------------------------------------------
// 8-bit cache rows: scale = amax / 127 and code = round-half-even(x / scale),
// both as correctly rounded fp32 divisions (so the codes are a function of
// the row alone); |code| <= 127; a row of zeros gets scale 0 and codes 0.
// D / 8 consecutive lanes hold one row, 8 values each.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void quantize_piece(const u32x4 x, bool ok, uint2& codes,
                                               float& scale) {
    constexpr int LPR = D / 8;
    float f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t w = x[e >> 1];
        f[e] = __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
    }
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(f[e]));
    if (!ok) amax = 0.f;
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    scale = amax / 127.f;
    uint32_t b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float c = (scale > 0.f) ? rintf(f[e] / scale) : 0.f;
        c = fminf(fmaxf(c, -127.f), 127.f);
        b[e] = (uint32_t)(int)c & 0xFFu;
    }
    codes.x = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
    codes.y = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
}

template <int D>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const uint16_t* __restrict__ x,
                                                            long rows, int8_t* __restrict__ codes,
                                                            float* __restrict__ scales) {
    constexpr int LPR = D / 8;
    const long row = ((long)blockIdx.x * 256 + threadIdx.x) / LPR;
    const int part = threadIdx.x % LPR;
    const bool ok = row < rows;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (ok) v = *(const u32x4*)(x + row * D + part * 8);
    uint2 c;
    float sc;
    quantize_piece<D>(v, ok, c, sc);
    if (!ok) return;
    *(uint2*)(codes + row * D + part * 8) = c;
    if (part == 0) scales[row] = sc;
}

// scatter into an 8-bit cache: chunk token t -> slot evict[t], quantised
template <int D>
__global__ __launch_bounds__(256) void kv_scatter_q8_kernel(
    int C, int S, int8_t* __restrict__ kc, float* __restrict__ ks, int8_t* __restrict__ vc,
    float* __restrict__ vs, float* __restrict__ scores, int64_t* __restrict__ pos,
    const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn,
    const float* __restrict__ new_scores, const int32_t* __restrict__ evict, int64_t p0) {
    constexpr int LPR = D / 8;
    constexpr int TOK = 256 / (2 * LPR);   // tokens per workgroup
    const int bh = blockIdx.y, tid = threadIdx.x;
    const int tok = tid / (2 * LPR), which = (tid / LPR) & 1, part = tid % LPR;
    const int t = blockIdx.x * TOK + tok;
    const bool in = t < S;
    const int slot = in ? evict[(size_t)bh * S + t] : -1;
    const bool ok = in && slot >= 0 && slot < C;   // out-of-range index: nothing written
    u32x4 v = {0u, 0u, 0u, 0u};
    if (in) v = *(const u32x4*)((which ? vn : kn) + ((size_t)bh * S + t) * D + part * 8);
    uint2 c;
    float sc;
    quantize_piece<D>(v, in, c, sc);
    if (!ok) return;
    const size_t row = (size_t)bh * C + slot;
    *(uint2*)((which ? vc : kc) + row * D + part * 8) = c;
    if (part == 0) (which ? vs : ks)[row] = sc;
    if (which == 0 && part == 0) {
        scores[row] = new_scores[(size_t)bh * S + t];
        if (pos) pos[row] = p0 + t;
    }
}

}  // namespace

hipError_t launch_quantize_rows(const uint16_t* x, long rows, int D, int8_t* codes,
                                float* scales, hipStream_t stream) {
    const long threads = rows * (D / 8);
    const unsigned blocks = (unsigned)((threads + 255) / 256);
    if (D == 64)
        hipLaunchKernelGGL(quantize_rows_kernel<64>, dim3(blocks), dim3(256), 0, stream, x,
                           rows, codes, scales);
    else
        hipLaunchKernelGGL(quantize_rows_kernel<128>, dim3(blocks), dim3(256), 0, stream, x,
                           rows, codes, scales);
    return hipGetLastError();
}

hipError_t launch_kv_scatter_q8(int BH, int D, int C, int S, int8_t* kc, float* ks, int8_t* vc,
                                float* vs, float* scores, int64_t* pos, const uint16_t* kn,
                                const uint16_t* vn, const float* new_scores,
                                const int32_t* evict_idx, int64_t p0, hipStream_t stream) {
    if (D == 64) {
        constexpr int TOK = 256 / (2 * (64 / 8));
        hipLaunchKernelGGL(kv_scatter_q8_kernel<64>, dim3((S + TOK - 1) / TOK, BH), dim3(256),
                           0, stream, C, S, kc, ks, vc, vs, scores, pos, kn, vn, new_scores,
                           evict_idx, p0);
    } else {
        constexpr int TOK = 256 / (2 * (128 / 8));
        hipLaunchKernelGGL(kv_scatter_q8_kernel<128>, dim3((S + TOK - 1) / TOK, BH), dim3(256),
                           0, stream, C, S, kc, ks, vc, vs, scores, pos, kn, vn, new_scores,
                           evict_idx, p0);
    }
    return hipGetLastError();
}

hipError_t launch_score_accumulate(int BH, int C, int S, int n, float* scores,
                                   float* new_scores, const float* wsum,
                                   hipStream_t stream) {
    // about 2048 workgroups in all, at least one per (b, kv head)
    int bx = (C + S + 255) / 256;
    const int cap = (2048 + BH - 1) / BH;
    if (bx > cap) bx = cap;
    hipLaunchKernelGGL(score_accumulate_kernel, dim3((unsigned)bx, (unsigned)BH), dim3(256), 0,
                       stream, BH, C, S, n, scores, new_scores, wsum);
    return hipGetLastError();
}

hipError_t launch_evict_select(int BH, int C, int S, int n, const float* scores,
                               int32_t* evict_idx, hipStream_t stream) {
    // keys per thread: the smallest supported run that covers C
    const int kpt = (C + SEL_T - 1) / SEL_T;
    float* sc = const_cast<float*>(scores);   // read only without a scatter
#define H2O_SEL(KPT)                                                                    \
    hipLaunchKernelGGL((evict_select_kernel<KPT, 0>), dim3(BH), dim3(SEL_T), 0, stream, C, S, \
                       n, sc, evict_idx, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, \
                       (int64_t)0)
    if (kpt > 64)
        hipLaunchKernelGGL(select_stream_kernel<false>, dim3(BH), dim3(SEL_T), 0, stream, C, S,
                           n, scores, (long)C, evict_idx, (long)S);
    else if (kpt <= 4)
        H2O_SEL(4);
    else if (kpt <= 16)
        H2O_SEL(16);
    else
        H2O_SEL(64);
#undef H2O_SEL
    return hipGetLastError();
}

// The fused kernel moves the chunk with one workgroup per (b, kv head): worth
// it for a short chunk (up to four 16-byte pieces per thread; S <= 128 at
// D = 128), while a long chunk moves faster in kv_scatter_kernel's grid.
bool select_scatter_fuses(int C, int S, int D) {
    return (C + SEL_T - 1) / SEL_T <= 64 && S * 2 * (D / 8) <= 4 * SEL_T;
}

hipError_t launch_select_scatter(int BH, int D, int C, int S, int n, float* scores,
                                 int32_t* evict_idx, uint16_t* kc, uint16_t* vc, int64_t* pos,
                                 const uint16_t* kn, const uint16_t* vn,
                                 const float* new_scores, int64_t p0, hipStream_t stream) {
    const int kpt = (C + SEL_T - 1) / SEL_T;
#define H2O_SEL(KPT, DS)                                                                   \
    hipLaunchKernelGGL((evict_select_kernel<KPT, DS>), dim3(BH), dim3(SEL_T), 0, stream, C, S, \
                       n, scores, evict_idx, kc, vc, pos, kn, vn, new_scores, p0)
    if (D == 64) {
        if (kpt <= 4)
            H2O_SEL(4, 64);
        else if (kpt <= 16)
            H2O_SEL(16, 64);
        else
            H2O_SEL(64, 64);
    } else {
        if (kpt <= 4)
            H2O_SEL(4, 128);
        else if (kpt <= 16)
            H2O_SEL(16, 128);
        else
            H2O_SEL(64, 128);
    }
#undef H2O_SEL
    return hipGetLastError();
}

hipError_t launch_snapkv_select(int BH, int C, int S, int n, int budget, const float* wsum,
                                int32_t* keep_idx, hipStream_t stream) {
    if (budget == 0) return hipSuccess;   // nothing is kept
    hipLaunchKernelGGL(select_stream_kernel<true>, dim3(BH), dim3(SEL_T), 0, stream, n,
                       n - budget, n, wsum, (long)C + S, keep_idx, (long)budget);
    return hipGetLastError();
}

hipError_t launch_kv_compact(int BH, int D, int C, int S, int budget, int out_len,
                             const uint16_t* kc, const uint16_t* vc, const int64_t* pos,
                             const uint16_t* kn, const uint16_t* vn, const float* wsum,
                             const int32_t* keep_idx, int64_t p0, uint16_t* ko, uint16_t* vo,
                             int64_t* pos_out, float* scores_out, hipStream_t stream) {
    const int total = budget + S;
    if (D == 64) {
        constexpr int ROWS = 256 / (2 * (64 / 8)) * CP_UNROLL;
        hipLaunchKernelGGL(kv_compact_kernel<64>, dim3((total + ROWS - 1) / ROWS, BH), dim3(256),
                           0, stream, C, S, budget, out_len, kc, vc, pos, kn, vn, wsum, keep_idx,
                           p0, ko, vo, pos_out, scores_out);
    } else {
        constexpr int ROWS = 256 / (2 * (128 / 8)) * CP_UNROLL;
        hipLaunchKernelGGL(kv_compact_kernel<128>, dim3((total + ROWS - 1) / ROWS, BH),
                           dim3(256), 0, stream, C, S, budget, out_len, kc, vc, pos, kn, vn,
                           wsum, keep_idx, p0, ko, vo, pos_out, scores_out);
    }
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
