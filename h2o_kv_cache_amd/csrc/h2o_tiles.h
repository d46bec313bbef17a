// LDS tile machinery shared by the gfx950 attention kernels: XCD-aware
// workgroup order, swizzled row-major K/V tiles in LDS filled by
// global_load_lds_dwordx4, and the per-lane MFMA operand reads from them.
#pragma once

#include "h2o_device.h"
#include "h2o_launch.h"

namespace h2o {
namespace {

// Workgroups are dispatched round-robin over the 8 XCDs (linear id L runs on
// XCD L % 8).  Re-index so that each XCD receives one contiguous run of the
// (bh, split, qt) work list: the row tiles that read the same K/V tiles then
// share one XCD's L2.
// decode_block for workgroup L of N (a part of a larger grid).
__device__ __forceinline__ void decode_block_at(int L, int N, int n_qt, int nsplit, int& qt,
                                                int& bh, int& split) {
    const int q8 = N >> 3, r8 = N & 7, x = L & 7, j = L >> 3;
    const int lam = x * q8 + min(x, r8) + j;
    qt = lam % n_qt;
    const int rest = lam / n_qt;
    split = rest % nsplit;
    bh = rest / nsplit;
}

__device__ __forceinline__ void decode_block(int n_qt, int nsplit, int& qt, int& bh,
                                             int& split) {
    decode_block_at(blockIdx.x, gridDim.x, n_qt, nsplit, qt, bh, split);
}

// LDS tiles are ROWS x D bf16, row-major, with the 16-byte chunks of each row
// XOR-swizzled so that the MFMA operand reads hit distinct banks (64 banks of
// 4 bytes: 256 bytes per cycle):
//   K tiles (ds_read_b128: 16 lanes read one chunk of 16 consecutive rows):
//       chunk ^ (key mod 16)
//   V tiles (ds_read_b64_tr_b16: 32 lanes read an aligned run of four chunks,
//       64 bytes, from each of 4 consecutive rows): chunk ^ (CPR/4)*(key mod 4)
//       moves the four runs to four disjoint bank groups (at D = 64, where two
//       rows share a 256-byte bank line, rows 2 apart differ in chunk bit 2).
//       Measured: no bank-conflict cycles, against two extra cycles per read
//       for chunk ^ 2*(key mod 8) at D = 128.
template <int D, bool VT>
__device__ __forceinline__ int tile_swz(int key) {
    constexpr int CPR = D / 8;
    return VT ? (CPR / 4) * (key & 3) : (key & (CPR - 1));
}

// Element offset of (key, 16-byte chunk) in a K (VT = false) or V tile.
template <int D, bool VT>
__device__ __forceinline__ int tile_off(int key, int chunk) {
    return key * D + ((chunk ^ tile_swz<D, VT>(key)) << 3);
}

// One 16-byte HBM -> LDS copy per lane (global_load_lds_dwordx4): lane l
// writes bytes [16*l, 16*l + 16) past the wave-uniform LDS address `lds`.
// Written as inline asm on purpose: the compiler then keeps no record of the
// asynchronous LDS write, so it does not stall reads of the *other* tile
// buffer behind it (it would otherwise wait for every outstanding load before
// each transposed LDS read).  The asm has no register outputs; completion is
// awaited explicitly with wait_tiles() before the barrier that publishes the
// tile, and before the workgroup exits.
// The asm sets M0 (the LDS address of the copy).  The compiler treats M0 as
// reserved and warns about the clobber; that is safe only while no code the
// compiler generates for these kernels keeps a value in M0, which holds for
// every kernel of this library (their gfx950 assembly has no M0 operand
// outside these asm blocks: no v_movrel indexing, no LDS-direct loads).
__device__ __forceinline__ void dma16(const uint16_t* gptr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds), "v"(gptr)
                 : "memory", "m0");
}

// dma16 with the non-temporal hint (rows read once; see dma16_s_nt).
__device__ __forceinline__ void dma16_nt(const uint16_t* gptr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt"
                 :
                 : "s"(lds), "v"(gptr)
                 : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One 4-byte HBM -> LDS copy per lane (global_load_lds_dword): lane l writes
// bytes [4*l, 4*l + 4) past the wave-uniform LDS address `lds`.  Same
// contract as dma16.
__device__ __forceinline__ void dma4(const float* gptr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off"
                 :
                 : "s"(lds), "v"(gptr)
                 : "memory", "m0");
}

// Issue the HBM -> LDS copy of one ROWS x D tile: each wave instruction fills
// 1 KiB of LDS, and each lane fetches the global chunk that belongs at its
// LDS slot.  Rows past `lim` re-read row lim-1, a valid row whose weight is
// masked to zero.
template <int D, bool VT, int NW = kWaves, int ROWS = kKeyTile>
__device__ __forceinline__ void issue_tile(uint16_t* tile, const uint16_t* __restrict__ src,
                                           int key0, int lim, int wave, int lane) {
    constexpr int CPR = D / 8;
    constexpr int ITER = ROWS * CPR / (NW * 64);
    static_assert(ITER * NW * 64 == ROWS * CPR, "tile must split into whole 1 KiB blocks");
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(tile));
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        const int blk = it * NW + wave;              // 1 KiB block of the tile
        const int p = blk * 64 + lane;               // LDS chunk slot
        const int key = p / CPR;
        const int chunk = (p % CPR) ^ tile_swz<D, VT>(key);
        const int gkey = min(key0 + key, lim - 1);
        dma16(src + (size_t)gkey * D + chunk * 8, base + blk * 1024);
    }
}

// One 16-byte HBM -> LDS copy per lane with a wave-uniform 64-bit base in
// SGPRs and a 32-bit per-lane byte offset (the instruction's scalar-base
// form): lane l writes bytes [16*l, 16*l + 16) past the wave-uniform LDS
// address `lds`.  Same contract as dma16.
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}

// dma16_s with the non-temporal hint, for rows that are read exactly once
// (the few-row passes stream every K/V row once): the stream then does not
// displace cached lines that are reused -- in the one-token step, the
// logits the tail reads back.  Same contract as dma16.
__device__ __forceinline__ void dma16_s_nt(const void* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                 :
                 : "s"(lds), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}

__device__ __forceinline__ const uint16_t* uniform_ptr(const uint16_t* p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const uint16_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// The copy of issue_tile for a tile whose ROWS rows all exist: the lanes'
// byte offsets inside a tile are fixed, so they are formed once, and each
// tile only moves the scalar base (row key0 of the source).  NT: the copies
// carry the non-temporal hint (rows read once).
template <int D, bool VT, int NW = kWaves, int ROWS = kKeyTile, bool NT = false>
struct TileCopy {
    static constexpr int CPR = D / 8;
    static constexpr int ITER = ROWS * CPR / (NW * 64);
    static_assert(ITER * NW * 64 == ROWS * CPR, "tile must split into whole 1 KiB blocks");
    uint32_t voff[ITER];
    __device__ __forceinline__ TileCopy(int wave, int lane) {
#pragma unroll
        for (int it = 0; it < ITER; ++it) {
            const int p = (it * NW + wave) * 64 + lane;
            const int key = p / CPR;
            const int chunk = (p % CPR) ^ tile_swz<D, VT>(key);
            voff[it] = 2u * (uint32_t)(key * D + chunk * 8);
        }
    }
    // rows key0 .. key0 + ROWS - 1 of src; `rows` = src + key0 * D
    __device__ __forceinline__ void issue(uint16_t* tile, const uint16_t* rows, int wave) const {
        const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(tile));
        const uint16_t* sb = uniform_ptr(rows);
#pragma unroll
        for (int it = 0; it < ITER; ++it) {
            if constexpr (NT)
                dma16_s_nt(sb, voff[it], base + (it * NW + wave) * 1024);
            else
                dma16_s(sb, voff[it], base + (it * NW + wave) * 1024);
        }
    }
};

// 8-bit cache tiles: ROWS x D int8 codes, row-major and unswizzled (they are
// converted to bf16 tiles, not read as MFMA operands), copied by waves
// 0..NW-1 in 1 KiB blocks; rows past `lim` re-read row lim-1.  The per-row
// scales of the same rows go to `ksc` / `vsc` (ROWS floats each) with one
// 4-byte copy per lane: wave SW_K copies the K scales, wave SW_V the V
// scales (ROWS == 64).
//   SWZ: chunk c of row `key` is stored at chunk position c ^ (key mod CPR),
//   so that 32 lanes reading the same chunk of 32 rows spread over the banks.
template <int D>
__device__ __forceinline__ int i8_swz(int key) { return key & (D / 16 - 1); }

//   V tiles read with the 8-bit transposed read: a 16-lane group reads 8
//   rows key0 + {0,1,2,3,8,9,10,11} (key0 a multiple of 4 with bit 3 clear);
//   chunk ^ ((key mod 4) | (key bit 3 moved to bit 2)) gives them 8 distinct
//   chunk positions (4 at D = 64, where a row has only 4 chunks).
template <int D>
__device__ __forceinline__ int i8_swz_v(int key) {
    return D >= 128 ? ((key & 3) | ((key >> 1) & 4)) : (key & 3);
}

// Tiles of the 16-row pass (32 rows per wave).  K: a 16-lane group reads one
// chunk of 16 consecutive rows; chunk ^ (key * CPR / 16 mod CPR) puts the 16
// rows (and the two 8-byte halves the two groups of a half-wave read) on
// distinct banks.  V, 8-bit transposed read: a 16-lane group reads rows
// 4g + {0,1,2,3} and 16 + 4g + {0,1,2,3}; the swizzle below gives the 16 rows
// of a half-wave distinct banks (checked for D = 64 and 128).
template <int D>
__device__ __forceinline__ int i8_swz_k16(int key) {
    return (key * (D / 16) / 16) & (D / 16 - 1);
}
template <int D>
__device__ __forceinline__ int i8_swz_v16(int key) {
    return D >= 128 ? (((key >> 1) & 3) | (((key >> 4) & 1) << 2))
                    : (((key >> 2) & 1) | (((key >> 4) & 1) << 1));
}

// SWZ: 0 none, 1 i8_swz (K tiles), 2 i8_swz_v (V tiles), 3 i8_swz_k16 and
// 4 i8_swz_v16 (16-row pass); NT: non-temporal copies (rows read once)
template <int D, int NW, int ROWS = kKeyTile, int SWZ = 0, bool NT = false>
__device__ __forceinline__ void issue_tile_i8(uint8_t* tile, const int8_t* __restrict__ src,
                                              int key0, int lim, int wave, int lane) {
    constexpr int CPR = D / 16;                  // 16-byte chunks per row
    constexpr int NBLK = ROWS * CPR / 64;        // 1 KiB blocks per tile
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(tile));
#pragma unroll
    for (int blk0 = 0; blk0 < NBLK; blk0 += NW) {
        const int blk = blk0 + wave;
        if (blk < NBLK) {
            const int p = blk * 64 + lane;
            const int key = p / CPR;
            const int sw = SWZ == 1   ? i8_swz<D>(key)
                           : SWZ == 2 ? i8_swz_v<D>(key)
                           : SWZ == 3 ? i8_swz_k16<D>(key)
                           : SWZ == 4 ? i8_swz_v16<D>(key)
                                      : 0;
            const int c = (p % CPR) ^ sw;
            const int gkey = min(key0 + key, lim - 1);
            const uint16_t* g = (const uint16_t*)(src + (size_t)gkey * D + c * 16);
            if constexpr (NT)
                dma16_nt(g, base + blk * 1024);
            else
                dma16(g, base + blk * 1024);
        }
    }
}

template <int SW_K, int SW_V>
__device__ __forceinline__ void issue_scales(float* ksc, float* vsc, const float* __restrict__ ks,
                                             const float* __restrict__ vs, int key0, int lim,
                                             int wave, int lane) {
    const int gkey = min(key0 + lane, lim - 1);
    if (wave == SW_K) dma4(ks + gkey, __builtin_amdgcn_readfirstlane(lds_addr(ksc)));
    if (wave == SW_V) dma4(vs + gkey, __builtin_amdgcn_readfirstlane(lds_addr(vsc)));
}

// 16 int8 codes (4 dwords) -> two 8-element bf16 chunks: exact (codes are
// integers of at most 7 bits), or times `s` rounded to nearest even.
__device__ __forceinline__ float i8_at(uint32_t w, int k) {
    return (float)(int)(int8_t)(w >> (8 * k));
}

__device__ __forceinline__ void i8x16_to_bf16(const u32x4 in, u32x4& lo, u32x4& hi) {
    uint32_t out[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const uint32_t w = in[p >> 1];
        const int k = 2 * (p & 1);
        // an integer of at most 8 significant bits: its bf16 is the high half
        out[p] = pack_hi(__float_as_uint(i8_at(w, k)), __float_as_uint(i8_at(w, k + 1)));
    }
    lo = u32x4{out[0], out[1], out[2], out[3]};
    hi = u32x4{out[4], out[5], out[6], out[7]};
}

// 8 int8 codes (2 dwords) -> one exact bf16 chunk
__device__ __forceinline__ bf16x8 i8x8_to_bf16(const uint2 in) {
    uint32_t out[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t w = (p < 2) ? in.x : in.y;
        const int k = 2 * (p & 1);
        out[p] = pack_hi(__float_as_uint(i8_at(w, k)), __float_as_uint(i8_at(w, k + 1)));
    }
    return as_bf16x8(u32x4{out[0], out[1], out[2], out[3]});
}

// 8-bit transposed LDS read (ds_read_b64_tr_b8).  In each 16-lane group,
// output lane i receives byte i % 8 of the 8-byte pieces that input lanes
// 2b + i / 8 (b = 0..7) point at, as its bytes b = 0..7.
typedef int i32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 lds_read_tr8(const uint8_t* p) {
    const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) i32x2*)p);
    return uint2{(uint32_t)v.x, (uint32_t)v.y};
}

__device__ __forceinline__ void i8x16_to_bf16_scaled(const u32x4 in, float s, u32x4& lo,
                                                     u32x4& hi) {
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(i8_at(in[e >> 2], e & 3) * s);
        b[e] = (__bf16)(i8_at(in[2 + (e >> 2)], e & 3) * s);
    }
    lo = __builtin_bit_cast(u32x4, a);
    hi = __builtin_bit_cast(u32x4, b);
}

// All of this wave's outstanding tile copies (and other memory ops) done.
__device__ __forceinline__ void wait_tiles() { __builtin_amdgcn_s_waitcnt(0); }

typedef short i16x4 __attribute__((ext_vector_type(4)));

// Per-lane byte offsets of the MFMA operand reads inside a tile.  Only these
// depend on the lane; the key block, k-step and buffer add compile-time or
// per-tile constants, which fold into the LDS instructions' immediate offset.
//   k[ks]: K fragment of k-step ks (rows l32 of key block 0, dims
//          16*ks + 8*half + [0, 8));
//   v[db]: transposed V read of dim block db for keys 4*half + [0, 4) of key
//          block 0.  In each 16-lane group, input lane j reads dims
//          4*(j%4)..+3 of key j/4 of its group's 4 keys; the hardware hands
//          output lane i dim i of those 4 keys (ds_read_b64_tr_b16).
template <int D>
struct LdsOffsets {
    uint32_t k[D / 16];
    uint32_t v[D / 32];
    __device__ __forceinline__ explicit LdsOffsets(int lane) {
        const int l32 = lane & 31, half = lane >> 5, j = lane & 15;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            k[ks] = 2u * (uint32_t)tile_off<D, false>(l32, 2 * ks + half);
        const int key = 4 * half + (j >> 2);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const int d = db * 32 + (lane & 16) + 4 * (j & 3);
            v[db] = 2u * (uint32_t)(tile_off<D, true>(key, d >> 3) + (d & 7));
        }
    }
};

__device__ __forceinline__ u32x4 lds_read16(const uint16_t* tile, uint32_t byte_off) {
    return *(const u32x4*)((const char*)tile + byte_off);
}

__device__ __forceinline__ u32x2 lds_read_tr(const uint16_t* tile, uint32_t byte_off) {
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)((const char*)tile + byte_off));
    return __builtin_bit_cast(u32x2, v);
}

}  // namespace
}  // namespace h2o
