// Internal declarations shared by the HIP sources of libdqk (not installed):
// the host-side part (dqk_host.h) and the device helpers every kernel uses.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dqk_host.h"

namespace dqk {

// fp32 -> binary16 bits: round to nearest even (the hardware conversion), with
// subnormals, and finite values past the largest binary16 clamped to +-65504.
__device__ __forceinline__ uint16_t f16_bits(float x) {
  x = fminf(fmaxf(x, -65504.0f), 65504.0f);
  _Float16 h = (_Float16)x;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_value(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

__device__ __forceinline__ float bf16_value(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// Code u of a 2-bit group with scale s stands for s*(2u-3).
__device__ __forceinline__ float level_of(uint32_t u) { return (float)(int)(2u * u) - 3.0f; }

// 2-bit code of x for the grid s*{-3,-1,1,3}: thresholds -2s, 0, 2s, ties upward.
__device__ __forceinline__ uint32_t code_of(float x, float two_s) {
  return (uint32_t)(x >= -two_s) + (uint32_t)(x >= 0.0f) + (uint32_t)(x >= two_s);
}

// Element offsets of the planes for one unit (batch row b, KV head g).
__host__ __device__ __forceinline__ size_t unit_index(const dqk_cache &c, int b, int g) {
  return (size_t)b * c.num_kv_heads + g;
}

}  // namespace dqk
