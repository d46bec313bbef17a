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
__device__ __forceinline__ void decode_block(int n_qt, int nsplit, int& qt, int& bh,
                                             int& split) {
    const int L = blockIdx.x, N = gridDim.x;
    const int q8 = N >> 3, r8 = N & 7, x = L & 7, j = L >> 3;
    const int lam = x * q8 + min(x, r8) + j;
    qt = lam % n_qt;
    const int rest = lam / n_qt;
    split = rest % nsplit;
    bh = rest / nsplit;
}

// LDS tiles are ROWS x D bf16, row-major, with the 16-byte chunks of each row
// XOR-swizzled so that the MFMA operand reads hit distinct banks:
//   K tiles (ds_read_b128 of one chunk from 16 consecutive rows):
//       chunk ^ (key mod 16)
//   V tiles (ds_read_b64_tr_b16: an aligned pair of chunks from 4 consecutive
//       rows per 16-lane group): chunk ^ 2*(key mod 8), which keeps pairs
//       together and gives the 4 rows distinct pairs.
template <int D, bool VT>
__device__ __forceinline__ int tile_swz(int key) {
    constexpr int CPR = D / 8;
    return VT ? 2 * (key & (CPR / 2 - 1)) : (key & (CPR - 1));
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
__device__ __forceinline__ void dma16(const uint16_t* gptr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds), "v"(gptr)
                 : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
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
