// Wavefront helpers shared by the decode kernels: matrix-core products on fp16
// operands, fp16 packing, DPP reductions and intra-wavefront LDS ordering.
#pragma once
#include "dqk_internal.h"

namespace dqk {
namespace wave {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));


__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a),
                                                __builtin_bit_cast(half8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t f16_pair(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}
__device__ __forceinline__ float f16_low(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_high(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Order LDS traffic between lanes of one wavefront (no workgroup barrier).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Cross-lane reductions with DPP moves (no LDS traffic).  `idn` fills lanes the
// move does not write, so it must be the identity of the operation.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float dpp_mov(float idn, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, idn),
                                                              __builtin_bit_cast(int, v), CTRL,
                                                              ROWS, 0xf, false));
}
__device__ __forceinline__ float row16_max(float x) {   // every lane: max over its 16-lane row
  x = fmaxf(x, dpp_mov<0xB1>(x, x));   // quad_perm [1,0,3,2]  (max is idempotent: fill = x)
  x = fmaxf(x, dpp_mov<0x4E>(x, x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_mov<0x141>(x, x));  // row_half_mirror
  x = fmaxf(x, dpp_mov<0x140>(x, x));  // row_mirror
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {   // every lane: sum over its 16-lane row
  x += dpp_mov<0xB1>(0.0f, x);
  x += dpp_mov<0x4E>(0.0f, x);
  x += dpp_mov<0x141>(0.0f, x);
  x += dpp_mov<0x140>(0.0f, x);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {    // uniform result
  x = row16_max(x);
  x = fmaxf(x, dpp_mov<0x142, 0xa>(x, x));  // row_bcast:15
  x = fmaxf(x, dpp_mov<0x143, 0xc>(x, x));  // row_bcast:31
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}
__device__ __forceinline__ float wave_sum(float x) {    // uniform result
  x = row16_sum(x);
  x += dpp_mov<0x142, 0xa>(0.0f, x);
  x += dpp_mov<0x143, 0xc>(0.0f, x);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// Keeps a constant in a VGPR so (x & m) | c selects one v_and_or_b32 (gfx9 VOP3
// takes no literals and at most one scalar operand).
__device__ __forceinline__ uint32_t in_vgpr(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

}  // namespace wave
}  // namespace dqk
