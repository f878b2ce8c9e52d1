// Device helpers shared by the gfx950 attention kernels: vector types, the
// MFMA wrapper, exp2, the LDS XOR swizzle and 64-lane wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kNegInf = -__builtin_huge_valf();
// Online softmax in the prefill: the reference max starts at kMRunInit (far
// below any score) and moves only when a lane's share of a tile's row sum
// exceeds kPSumMax, which bounds every p of the tile (p <= 2^15 keeps fp16
// P finite and at full relative precision).
constexpr float kMRunInit = -1.0e30f;
constexpr float kPSumMax = 32768.0f;
// Split-D forward: row-max growth (log2 units) tolerated before its reference
// max moves (then O and l are rescaled); in between p <= 2^8.
constexpr float kLazyRescale = 8.0f;

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
__host__ __device__ __forceinline__ uint32_t swz(int r, int c) {
  static_assert(C == 4 || C == 8 || C == 16 || C == 32 || C == 64 || C == 128, "chunks per row");
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

// Inverse of swz<C>: the (row, chunk) stored at 16-byte slot `slot` of
// 256-byte line `line`.
template <int C>
__host__ __device__ __forceinline__ void swz_inv(int line, int slot, int& r, int& c) {
  if constexpr (C >= 16) {
    r = line / (C / 16);
    c = (line % (C / 16)) * 16 + (slot ^ (r & 15));
  } else {
    constexpr int RPL = 16 / C;
    r = line * RPL + slot / C;
    c = (slot % C) ^ (line & (C - 1));
  }
}

// Row-major [key][d] layout for V tiles read with ds_read_b64_tr_b16: a
// transposed read touches 4 consecutive key rows x 4 consecutive 16-byte
// chunks, and the XOR below spreads those 16 chunks over the 16 bank groups
// of a 256-byte line.  With 4 chunks per row (D = 32) those 4 rows are one
// whole line already.
template <int C>
__host__ __device__ __forceinline__ uint32_t vswz(int r, int c) {
  static_assert(C == 4 || C == 8 || C == 16 || C == 32 || C == 64 || C == 128, "chunks per row");
  if constexpr (C == 4) {
    return (uint32_t)(r * 64 + c * 16);
  } else if constexpr (C >= 16) {
    const int line = r * (C / 16) + (c >> 4);
    const int slot = (c & 15) ^ (4 * (r & 3));
    return (uint32_t)(line * 256 + slot * 16);
  } else {
    const int line = r >> 1;
    const int slot = (r & 1) * 8 + (c ^ (4 * (line & 1)));
    return (uint32_t)(line * 256 + slot * 16);
  }
}
template <int C>
__host__ __device__ __forceinline__ void vswz_inv(int line, int slot, int& r, int& c) {
  if constexpr (C == 4) {
    r = line * 4 + slot / 4;
    c = slot % 4;
  } else if constexpr (C >= 16) {
    r = line / (C / 16);
    c = (line % (C / 16)) * 16 + (slot ^ (4 * (r & 3)));
  } else {
    r = line * 2 + slot / 8;
    c = (slot % 8) ^ (4 * (line & 1));
  }
}

typedef _Float16 h4v __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// i % 4 of the 8-byte blocks addressed by group lanes i / 4 + 4 j, j = 0..3.
// So if group lane 4 j + a points at row key_j, columns d0 + 4 a .. + 3 of
// a row-major array, lane i gets column d0 + i of rows key_0..key_3.
__device__ __forceinline__ h4v lds_read_tr16(const char* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  return __builtin_bit_cast(h4v, v);
}

// Direct global -> LDS copies through a buffer resource (a load past the
// buffer's end writes zeros), issued from inline asm: the compiler then
// does not count them as pending LDS writes.  Issued through the builtin it
// waits for every outstanding copy before each LDS read it cannot tell
// apart from their destinations (the transposed V reads of the prefill
// among them), which cut the prefetch distance to a fraction of a tile; the
// kernels order the copies themselves and wait with s_waitcnt vmcnt before
// the barrier that publishes the data.  rs: the four descriptor dwords;
// lds_addr: the wave-uniform LDS byte address (M0) that lane l's 16 (dma16)
// or 4 (dma4) bytes land at plus 16 l (4 l).
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  u32x4 r;
  // the descriptor goes to scalar registers; the values are uniform, and
  // readfirstlane lets the compiler place them there in every caller
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = 0x00020000u;
  return r;
}
__device__ __forceinline__ void dma16(u32x4 rs, uint32_t lds_addr, uint32_t voff) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "{m0}"(lds_addr));
}
__device__ __forceinline__ void dma4(u32x4 rs, uint32_t lds_addr, uint32_t voff) {
  asm volatile("buffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "{m0}"(lds_addr));
}
__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}

// Maximum / sum of x over the two 32-lane halves of a wavefront, on the
// VALU: v_permlane32_swap(x, x) returns the low half of x in both halves
// and the high half in both halves (pinned by a GPU probe test).
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ h8 as_h8(u32x4 v) { return __builtin_bit_cast(h8, v); }

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// Raw buffer resource over `bytes` bytes at `base`: loads past the end read
// 0 and stores past the end are dropped by the address unit, which is how
// the kernels handle ragged sequence tails without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}

// sum += a.x * b.x + a.y * b.y in fp32 (v_dot2_f32_f16).
__device__ __forceinline__ float dot2(h2 a, h2 b, float sum) { return __builtin_amdgcn_fdot2(a, b, sum, false); }

// Waits until every vector-memory load of this wavefront has returned
// (s_waitcnt vmcnt(0); expcnt and lgkmcnt left unconstrained).  Placed
// before a loop, it tells the compiler's wait-count tracking that loads
// issued earlier need no waits inside the loop.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Wait until at most N vector memory operations of this wavefront are
// outstanding (they complete in issue order, so all but the last N issued).
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// True on every lane if pred holds on any lane of the wavefront.
__device__ __forceinline__ bool wave_any(bool pred) { return __builtin_amdgcn_ballot_w64(pred) != 0; }

// Packs the low (hi_half = false) or high halves of two dwords: result low
// 16 bits from a, high 16 bits from b.
__device__ __forceinline__ uint32_t pack_halves(uint32_t a, uint32_t b, bool hi_half) {
  return __builtin_amdgcn_perm(b, a, hi_half ? 0x07060302u : 0x05040100u);
}

}  // namespace fa
