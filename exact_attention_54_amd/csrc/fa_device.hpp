// Device helpers shared by the gfx950 attention kernels: vector types, the
// MFMA wrapper, exp2, the LDS XOR swizzle and 64-lane wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kNegInf = -__builtin_huge_valf();

// D[32x32] += A[32x16] * B[16x32], fp16 inputs, fp32 accumulation.
// Lane l supplies A[l % 32][8 * (l / 32) + t] and B[8 * (l / 32) + t][l % 32]
// for t = 0..7, and holds D[8 * (j / 4) + 4 * (l / 32) + j % 4][l % 32] in
// accumulator element j = 0..15.
__device__ __forceinline__ f32x16 mfma_32x32x16(h8 a, h8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// 2^x on the transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Byte offset of 16-byte chunk c of row r in an LDS array whose rows hold C
// chunks, XOR-swizzled so that 16 consecutive rows reading the same chunk
// column land on 16 distinct 16-byte bank groups of a 256-byte bank line.
// This is the bank-conflict-free permutation of "Adaptive High-Performance
// Attention Kernels in CUDA" (Lever B), sized for the 64 x 4-byte LDS bank
// line of gfx950.
template <int C>
__device__ __forceinline__ uint32_t swz(int r, int c) {
  static_assert(C == 4 || C == 8 || C == 16 || C == 32, "chunks per row");
  if constexpr (C >= 16) {
    const int line = r * (C / 16) + (c >> 4);
    const int slot = (c & 15) ^ (r & 15);
    return (uint32_t)(line * 256 + slot * 16);
  } else {
    constexpr int RPL = 16 / C;  // rows per 256-byte line
    const int line = r / RPL;
    const int slot = (r % RPL) * C + (c ^ (line & (C - 1)));
    return (uint32_t)(line * 256 + slot * 16);
  }
}

// Maximum / sum of x over the two 32-lane halves of a wavefront.
__device__ __forceinline__ float xhalf_max(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
__device__ __forceinline__ float xhalf_sum(float x) { return x + __shfl_xor(x, 32); }

__device__ __forceinline__ h8 as_h8(u32x4 v) { return __builtin_bit_cast(h8, v); }

// Packs the low (hi_half = false) or high halves of two dwords: result low
// 16 bits from a, high 16 bits from b.
__device__ __forceinline__ uint32_t pack_halves(uint32_t a, uint32_t b, bool hi_half) {
  return __builtin_amdgcn_perm(b, a, hi_half ? 0x07060302u : 0x05040100u);
}

}  // namespace fa
