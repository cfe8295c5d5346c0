// Shared device types and helpers for the gfx950 Orthros kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace orthros {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

// bf16 bit pattern <-> fp32. The conversion to bf16 rounds to nearest even (the compiler
// lowers the cast to the gfx950 packed convert instruction).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Elements are addressed with 64-bit offsets: the largest tensors here exceed 2^31 elements.
typedef int64_t idx_t;

// A value every lane of the wavefront holds alike, read back as a scalar (values computed by
// vector instructions, such as 64-bit divisions, otherwise stay in vector registers).
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Physical block index -> logical block index so that consecutive logical blocks run on the
// same XCD (blocks are dealt to the 8 XCDs round-robin by physical index), sharing its L2.
__device__ __forceinline__ uint32_t xcd_swizzle(uint32_t phys, uint32_t total) {
  constexpr uint32_t kXcds = 8;
  const uint32_t xcd = phys % kXcds;
  const uint32_t k = phys / kXcds;
  const uint32_t per = total / kXcds;
  const uint32_t rem = total % kXcds;
  const uint32_t start = xcd * per + (xcd < rem ? xcd : rem);
  return start + k;
}

// Work order for blocks of unequal length (causal rows, or keys with rows only after them):
// logical block lid -> (pair, block index counted from the longest), grouping the blocks of a
// few pairs at a time so that they run together and their operands stay in one XCD's L2, and
// running each group's blocks longest first. `conc` is the number of work-groups one XCD runs
// at once; a group holds about that many blocks. (Ordering all pairs' longest blocks first
// spread every pair over every XCD: the 2048-token causal rows read their keys and values
// from memory 4-5 times over.)
__device__ __forceinline__ void grouped_order(uint32_t lid, int pairs, int nblk, int conc,
                                              int& from_longest, int& pair) {
  const int gp0 = conc / nblk < 1 ? 1 : (conc / nblk > pairs ? pairs : conc / nblk);
  const uint32_t gsz = (uint32_t)gp0 * (uint32_t)nblk;
  const int grp = (int)(lid / gsz);
  const int r = (int)(lid % gsz);
  const int p0 = grp * gp0;
  const int gp = gp0 < pairs - p0 ? gp0 : pairs - p0;  // the last group may hold fewer pairs
  from_longest = r / gp;
  pair = p0 + r % gp;
}

}  // namespace orthros
