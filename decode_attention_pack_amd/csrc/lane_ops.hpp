// lane_ops.hpp -- cross-lane moves of a 64-lane gfx950 wave used by the
// decode kernels: DPP moves within 16-lane rows and the gfx950 lane-swap
// instructions between rows and halves.
#pragma once

#include <hip/hip_runtime.h>

namespace kivi {

// DPP move of v within 16-lane rows: ctrl 0x121..0x12F rotate right by
// 1..15, 0x140 mirror (lane i <- 15 - i), 0x141 half mirror (i <- 7 - i
// within 8 lanes), 0x00..0xFF quad permutation.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Reductions over the 16 lanes of a row (DPP row rotations by 8, 4, 2, 1).
__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, dpp_mov<0x128>(v));
  v = fmaxf(v, dpp_mov<0x124>(v));
  v = fmaxf(v, dpp_mov<0x122>(v));
  v = fmaxf(v, dpp_mov<0x121>(v));
  return v;
}
__device__ __forceinline__ float row_sum(float v) {
  v += dpp_mov<0x128>(v);
  v += dpp_mov<0x124>(v);
  v += dpp_mov<0x122>(v);
  v += dpp_mov<0x121>(v);
  return v;
}

// v_permlane16_swap a, b exchanges the odd 16-lane rows of a with the even
// rows of b: afterwards a holds rows (a0, b0, a2, b2) and b holds
// (a1, b1, a3, b3).  v_permlane32_swap a, b exchanges the upper half of a
// with the lower half of b: a = (a_lo, b_lo), b = (a_hi, b_hi).  Inline
// assembly: the compiler builtin for these returns the first register twice
// in this toolchain.  The nops cover the VALU-write/swap-read hazard.
__device__ __forceinline__ void lane_swap16(float &a, float &b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void lane_swap32(float &a, float &b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
// Four swaps behind one pair of nops (the four pairs are distinct registers).
__device__ __forceinline__ void lane_swap16x4(float &a0, float &b0, float &a1, float &b1,
                                              float &a2, float &b2, float &a3, float &b3) {
  asm volatile(
      "s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\tv_permlane16_swap_b32 %2, %3\n\t"
      "v_permlane16_swap_b32 %4, %5\n\tv_permlane16_swap_b32 %6, %7\n\ts_nop 1"
      : "+v"(a0), "+v"(b0), "+v"(a1), "+v"(b1), "+v"(a2), "+v"(b2), "+v"(a3), "+v"(b3));
}
__device__ __forceinline__ void lane_swap32x4(float &a0, float &b0, float &a1, float &b1,
                                              float &a2, float &b2, float &a3, float &b3) {
  asm volatile(
      "s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\tv_permlane32_swap_b32 %2, %3\n\t"
      "v_permlane32_swap_b32 %4, %5\n\tv_permlane32_swap_b32 %6, %7\n\ts_nop 1"
      : "+v"(a0), "+v"(b0), "+v"(a1), "+v"(b1), "+v"(a2), "+v"(b2), "+v"(a3), "+v"(b3));
}

// Sum / max over the 4 lane groups (lanes l, l^16, l^32, l^48): with a and b
// both holding x, a swap leaves x[l] and x[l ^ 16] (or x[l ^ 32]) in a, b.
__device__ __forceinline__ float group_sum(float v) {
  float a = v, b = v;
  lane_swap16(a, b);
  v = a + b;
  a = v;
  b = v;
  lane_swap32(a, b);
  return a + b;
}
__device__ __forceinline__ float group_max(float v) {
  float a = v, b = v;
  lane_swap16(a, b);
  v = fmaxf(a, b);
  a = v;
  b = v;
  lane_swap32(a, b);
  return fmaxf(a, b);
}

}  // namespace kivi
