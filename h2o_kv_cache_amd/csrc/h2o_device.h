// Device-side helpers shared by the gfx950 kernels of libh2o.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace h2o {

// log2(e): the kernels work in base 2 (v_exp_f32 computes 2^x).
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// One 32x32x16 bf16 MFMA, fp32 accumulate.  Operand layout used throughout:
//   A (32 x 16): lane l holds row l%32, the 8 k-values of half l/32;
//   B (16 x 32): lane l holds column l%32, the 8 k-values of half l/32;
//   C (32 x 32): lane l holds column l%32 and rows 8*(v/4) + 4*(l/32) + v%4
//                in element v = 0..15.
__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8 a, const bf16x8 b,
                                               const f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int acc_row(int v, int half) {
    return 8 * (v >> 2) + 4 * half + (v & 3);
}

__device__ __forceinline__ float fast_exp2(float x) {
    return __builtin_amdgcn_exp2f(x);
}

__device__ __forceinline__ float fast_log2(float x) {
    return __builtin_amdgcn_logf(x);
}

// Exchange with the lane 32 positions away (the other half of the wave).
__device__ __forceinline__ float xor32(float x) {
    return __shfl_xor(x, 32, 64);
}

// bf16 bit patterns of two 16-bit halves into one dword.
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
    return (a & 0xFFFFu) | (b << 16);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
    // one byte permute: bytes 2, 3 of a, then bytes 2, 3 of b (selector
    // values 0-3 pick bytes of the second operand, 4-7 of the first)
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
    return __builtin_bit_cast(bf16x8, v);
}

// Order-preserving map of a score onto uint32: -0.0 == +0.0, NaN above +inf.
// Every mapped score is >= 0x007FFFFF (the image of -inf), so key 0 is free
// for empty slots, which are taken first.
__device__ __forceinline__ uint32_t score_key(float x) {
    uint32_t u = __float_as_uint(x);
    if (x != x) return 0xFFFFFFFFu;
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace h2o
