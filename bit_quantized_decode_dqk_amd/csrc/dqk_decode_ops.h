// Operand helpers shared by the matrix-core decode kernels: fp16 packing with
// mixed-precision FMAs, packed 16-bit shifts, the 2-bit value-code operands and
// the LDS-only workgroup barrier.  See the decode kernels for how a 2-bit code
// becomes an exact fp16 subnormal operand.
#pragma once
#include "dqk_internal.h"
#include "dqk_wave.h"

namespace dqk {
namespace dops {

using namespace wave;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kOneF16x2 = 0x3C003C00u;
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit elements, range-checked (gfx9)
constexpr uint32_t kFar = 0x40000000u;   // offset past every plane: the load returns zero

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// c ? b : a on two values the compiler may not fold into an indexed load
// (an array indexed by a lane-dependent value would go to scratch memory).
__device__ __forceinline__ float sel2(bool c, float a, float b) {
  asm volatile("" : "+v"(a), "+v"(b));
  return c ? b : a;
}

// fp16(a * (fp16 in half SH of s)) written to the low half of d, one rounding.
template <int SH>
__device__ __forceinline__ uint32_t mixlo(float a, uint32_t s) {
  uint32_t d;
  if constexpr (SH == 0)
    asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "=v"(d) : "v"(a), "v"(s));
  else
    asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "=v"(d) : "v"(a), "v"(s));
  return d;
}
// the same into the high half of d (the low half is kept).
template <int SH>
__device__ __forceinline__ uint32_t mixhi(uint32_t d, float a, uint32_t s) {
  if constexpr (SH == 0)
    asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "+v"(d) : "v"(a), "v"(s));
  else
    asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "+v"(d) : "v"(a), "v"(s));
  return d;
}
// fp16(a * (half SH of s) - (half HH of h)) into the low half: what the fp16 number in
// h leaves out of the exact product, rounded once.
template <int SH, int HH>
__device__ __forceinline__ uint32_t reslo(float a, uint32_t s, uint32_t h) {
  uint32_t d;
  if constexpr (SH == 0 && HH == 0)
    asm("v_fma_mixlo_f16 %0, %1, %2, -%3 op_sel:[0,0,0] op_sel_hi:[0,1,1]" : "=v"(d) : "v"(a), "v"(s), "v"(h));
  else if constexpr (SH == 0 && HH == 1)
    asm("v_fma_mixlo_f16 %0, %1, %2, -%3 op_sel:[0,0,1] op_sel_hi:[0,1,1]" : "=v"(d) : "v"(a), "v"(s), "v"(h));
  else if constexpr (SH == 1 && HH == 0)
    asm("v_fma_mixlo_f16 %0, %1, %2, -%3 op_sel:[0,1,0] op_sel_hi:[0,1,1]" : "=v"(d) : "v"(a), "v"(s), "v"(h));
  else
    asm("v_fma_mixlo_f16 %0, %1, %2, -%3 op_sel:[0,1,1] op_sel_hi:[0,1,1]" : "=v"(d) : "v"(a), "v"(s), "v"(h));
  return d;
}
template <int SH, int HH>
__device__ __forceinline__ uint32_t reshi(uint32_t d, float a, uint32_t s, uint32_t h) {
  if constexpr (SH == 0 && HH == 0)
    asm("v_fma_mixhi_f16 %0, %1, %2, -%3 op_sel:[0,0,0] op_sel_hi:[0,1,1]" : "+v"(d) : "v"(a), "v"(s), "v"(h));
  else if constexpr (SH == 0 && HH == 1)
    asm("v_fma_mixhi_f16 %0, %1, %2, -%3 op_sel:[0,0,1] op_sel_hi:[0,1,1]" : "+v"(d) : "v"(a), "v"(s), "v"(h));
  else if constexpr (SH == 1 && HH == 0)
    asm("v_fma_mixhi_f16 %0, %1, %2, -%3 op_sel:[0,1,0] op_sel_hi:[0,1,1]" : "+v"(d) : "v"(a), "v"(s), "v"(h));
  else
    asm("v_fma_mixhi_f16 %0, %1, %2, -%3 op_sel:[0,1,1] op_sel_hi:[0,1,1]" : "+v"(d) : "v"(a), "v"(s), "v"(h));
  return d;
}

// acc + (fp16 in the low half of h) * k, one mixed-precision FMA.
__device__ __forceinline__ float mix_acc(float acc, uint32_t h, float k) {
  float d;
  asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "=v"(d) : "v"(h), "v"(k), "v"(acc));
  return d;
}

// Shift both 16-bit halves of x left / right by the amounts in the halves of s.
__device__ __forceinline__ uint32_t pk_shl16(uint32_t x, uint32_t s) {
  uint32_t d;
  asm("v_pk_lshlrev_b16 %0, %1, %2" : "=v"(d) : "v"(s), "v"(x));
  return d;
}
__device__ __forceinline__ uint32_t pk_shr16(uint32_t x, uint32_t s) {
  uint32_t d;
  asm("v_pk_lshrrev_b16 %0, %1, %2" : "=v"(d) : "v"(s), "v"(x));
  return d;
}

// Value code word (16 tokens of one channel, token c at bits 2c) -> B operand of
// K chunk 0 (tokens 0,8,1,9,2,10,3,11) or 1 (tokens 4,12,5,13,6,14,7,15).
__device__ __forceinline__ u32x4 value_operand(uint32_t w, int kc2) {
  if (kc2 == 0) return u32x4{w & 0x00030003u, w & 0x000C000Cu, w & 0x00300030u, w & 0x00C000C0u};
  const uint32_t s = w >> 6;
  return u32x4{w & 0x03000300u, s & 0x00300030u, s & 0x00C000C0u, s & 0x03000300u};
}

// Bit position pair k of token c (mod 8) of a value word after value_operand.
__device__ __forceinline__ int value_k(int c) {
  const int m = c & 7;
  return m < 5 ? m : m - 3;   // 0,1,2,3,4,2,3,4
}

// fp16 bits of 2^e for e >= -24 (subnormal below 2^-14; e >= 16 gives the infinity pattern).
__device__ __forceinline__ uint32_t pow2_bits(int e) {
  if (e >= 16) return 0x7C00u;
  return e >= -14 ? (uint32_t)(e + 15) << 10 : 1u << (e + 24);
}

// Workgroup barrier that publishes this wavefront's LDS writes (no wait on
// outstanding global loads, which stay in flight across it).
__device__ __forceinline__ void block_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace dops
}  // namespace dqk
