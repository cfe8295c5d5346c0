// LDS staging and matrix-core operand helpers shared by the gfx950 attention kernels.
#pragma once

#include "common.h"

namespace orthros {

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ bf16x8 cat_tr(s16x4 lo, s16x4 hi) {
  s16x4 v8[2] = {lo, hi};
  return __builtin_bit_cast(bf16x8, v8);
}
__device__ __forceinline__ float lane_pair_max(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float lane_pair_sum(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// One wave-wide 16-byte-per-lane copy from global memory straight into LDS: lane i reads
// `base` + off_i (a scalar base and a 32-bit per-lane offset, so no vector address arithmetic)
// and fills bytes 16 i .. 16 i + 15 from the LDS address `lds`. Issued as inline assembly so
// the compiler does not make every later LDS read wait for it (it cannot tell the copy's
// destination slot from the slots being read); the kernel waits for these copies itself before
// the barrier that publishes them. M0, which carries the LDS address, is restored afterwards.
__device__ __forceinline__ void copy_to_lds(const void* base, uint32_t off, uint32_t lds) {
  // (base and lds are the same in every lane; read them as scalars so the operands below are
  // scalar registers whatever the compiler kept them in)
  base = reinterpret_cast<const void*>(uniform64(reinterpret_cast<int64_t>(base)));
  lds = __builtin_amdgcn_readfirstlane(lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(off), "s"(base)
      : "memory");
}
// The same with a 64-bit global address per lane (each lane's source may lie anywhere), for
// data read once: the copy carries the non-temporal hint. A stream of these copies reads
// ~7.2 TB/s on this part with the hint and ~6.1 TB/s without (8 GiB, one 4-wave block per CU).
__device__ __forceinline__ void stream_to_lds_at(const void* addr, uint32_t lds) {
  lds = __builtin_amdgcn_readfirstlane(lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(addr)
      : "memory");
}
// The same with 4 bytes per lane: active lane i fills bytes 4 i .. 4 i + 3 from `lds`.
__device__ __forceinline__ void copy_to_lds_b32(const void* base, uint32_t off, uint32_t lds) {
  base = reinterpret_cast<const void*>(uniform64(reinterpret_cast<int64_t>(base)));
  lds = __builtin_amdgcn_readfirstlane(lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(off), "s"(base)
      : "memory");
}
__device__ __forceinline__ void wait_lds_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Scheduling hint for one region: NPRE LDS reads first, then NM times {1 MFMA, NDS LDS reads,
// NV vector instructions}, so the vector work issues in the shadow of the matrix cores.
template <int NM, int NPRE, int NDS, int NV>
__device__ __forceinline__ void interleave() {
  __builtin_amdgcn_sched_group_barrier(0x100, NPRE, 0);
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, NDS, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
  }
}

}  // namespace orthros
