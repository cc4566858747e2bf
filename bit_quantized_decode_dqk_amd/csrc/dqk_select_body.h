// Query transform and per-head channel selection: the body of one workgroup,
// shared by the selection kernel and the fused append + selection kernel.
//
// Dual-QK (arXiv abstract; tech.dede.sh summary, "Paired transforms instead of
// shared rotation"): the query transform q' = q A concentrates query energy so
// that dynamic channel pruning keeps few channels; "Results at 128K context"
// evaluates it at 40% query-channel sparsity.  Here each query head keeps
// channel 0 (the protected channel) and the keep-1 other channels of largest
// |q'|, equal magnitudes going to the lower index; the kept set is written in
// ascending order.
//
// One workgroup of 256 lanes per (batch row, KV head) serves the group's query
// heads: every output is an fp32 FMA chain over input channels in ascending
// order (bit-reproducible); then each wavefront finds one head's exact top-k by
// a bitwise search over the magnitudes' bit patterns with ballots, and ballot
// prefixes give each kept channel its ascending slot.  Built with
// -ffp-contract=off.
#pragma once
#include "dqk_internal.h"

#include <type_traits>

namespace dqk {
namespace selb {

constexpr int kThreads = 256;

__device__ __forceinline__ int popc(unsigned long long m) { return __popcll(m); }

// Exact top-(k) of one head's |q'| over channels 1..D-1 inside one wavefront:
// lane l holds channels l and l+64.  Magnitudes are non-negative floats, so
// their bit patterns order like the values; a bitwise search from the top bit
// finds the k-th largest pattern T, channels above T are kept, and of the
// channels equal to T the lowest indices are kept.  The search stops early once
// exactly k patterns are at or above the prefix found so far: that set is then
// the answer (the full search would end on a T with the same set).  Writes
// idx[0..keep) ascending.
template <int D>
__device__ void select_one_head(const float *mag, int keep, int32_t *idx) {
  const int lane = threadIdx.x & 63;
  const unsigned long long below = (1ull << lane) - 1ull;
  const int c0 = lane, c1 = lane + 64;
  const bool v0 = c0 >= 1 && c0 < D, v1 = c1 < D;
  const uint32_t k0 = v0 ? __float_as_uint(mag[c0]) : 0u;
  const uint32_t k1 = v1 ? __float_as_uint(mag[c1]) : 0u;
  const int want = keep - 1;             // channels to keep besides channel 0
  bool s0 = false, s1 = false;
  if (want > 0) {
    uint32_t t = 0;
    for (int bit = 30; bit >= 0; --bit) {
      const uint32_t cand = t | (1u << bit);
      const int n = popc(__ballot(v0 && k0 >= cand)) + popc(__ballot(v1 && k1 >= cand));
      if (n >= want) {
        t = cand;
        if (n == want) break;
      }
    }
    const unsigned long long g0 = __ballot(v0 && k0 > t), g1 = __ballot(v1 && k1 > t);
    const unsigned long long e0 = __ballot(v0 && k0 == t), e1 = __ballot(v1 && k1 == t);
    const int need = want - popc(g0) - popc(g1);   // equal channels still to take
    const int r0 = popc(e0 & below), r1 = popc(e0) + popc(e1 & below);
    s0 = (v0 && k0 > t) || (v0 && k0 == t && r0 < need);
    s1 = (v1 && k1 > t) || (v1 && k1 == t && r1 < need);
  }
  if (c0 == 0) s0 = true;                // the protected channel
  const unsigned long long m0 = __ballot(s0), m1 = __ballot(s1);
  if (s0) idx[popc(m0 & below)] = c0;
  if (s1) idx[popc(m0) + popc(m1 & below)] = c1;
}

// One workgroup per (batch row, KV head); the G query heads of the group share
// A_g.  Thread j forms q'_c for column c = j % D of the heads of its thread
// group j / D (G heads spread over kThreads / D groups); each wavefront then
// selects for every fourth head.
template <int D, int G, bool BF16>
__device__ __forceinline__ void select_block(int block, const void *q,
                                             const float *__restrict__ amat, int hq, int hkv,
                                             int keep, float *q_prime, int32_t *sel_idx) {
  __shared__ __attribute__((aligned(16))) float qs[G][D];
  __shared__ float mag[G][D];
  const int b = block / hkv, g = block % hkv;
  const size_t row0 = (size_t)b * hq + (size_t)g * G;
  const int j = threadIdx.x, wave = j >> 6;
  // The query rows and lane j's whole column of A_g are loaded together: the
  // setup is one round trip.
  constexpr int QJ = (G * D + kThreads - 1) / kThreads;
  float qv[QJ];
#pragma unroll
  for (int k = 0; k < QJ; ++k) {
    const int e = min(j + kThreads * k, G * D - 1);   // unconditional loads (no branch between them)
    if constexpr (BF16)
      qv[k] = bf16_value(static_cast<const uint16_t *>(q)[row0 * D + e]);
    else
      qv[k] = static_cast<const float *>(q)[row0 * D + e];
  }
  constexpr int NGRP = kThreads / D;            // thread groups (one per D threads)
  constexpr int HPT = (G + NGRP - 1) / NGRP;    // heads per thread
  const int col = j % D, grp = j / D;           // grp is uniform in a wavefront
  float a[D];
  const float *acol = amat + (size_t)g * D * D + col;
#pragma unroll
  for (int r = 0; r < D; ++r) a[r] = acol[(size_t)r * D];
#pragma unroll
  for (int k = 0; k < QJ; ++k) {   // clamped like the loads: the last element may be written twice
    const int e = min(j + kThreads * k, G * D - 1);
    qs[e / D][e % D] = qv[k];
  }
  // A's column is used here so that its loads are issued before the barrier,
  // together with the query loads (A is read-only: the compiler would otherwise
  // move them past the barrier, a second round trip)
#pragma unroll
  for (int r = 0; r < D; ++r) asm volatile("" ::"v"(a[r]));
  __syncthreads();
  // thread group GRP's heads as compile-time rows of qs (a runtime head index
  // makes the compiler hoist every LDS read of the chain at once)
  auto chain = [&](auto grp_c) {
    constexpr int GRP = decltype(grp_c)::value;
    float acc[HPT];
#pragma unroll
    for (int i = 0; i < HPT; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int r = 0; r < D; ++r)
#pragma unroll
      for (int i = 0; i < HPT; ++i) {
        acc[i] = __builtin_fmaf(qs[min(GRP * HPT + i, G - 1)][r], a[r], acc[i]);
      }
#pragma unroll
    for (int i = 0; i < HPT; ++i) {
      const int h = GRP * HPT + i;
      if (h < G) {
        q_prime[(row0 + h) * D + col] = acc[i];
        mag[h][col] = fabsf(acc[i]);
      }
    }
  };
  static_assert(NGRP <= 4, "thread groups");
  switch (grp) {   // uniform in a wavefront
    case 0: chain(std::integral_constant<int, 0>{}); break;
    case 1: if constexpr (NGRP > 1) chain(std::integral_constant<int, 1>{}); break;
    case 2: if constexpr (NGRP > 2) chain(std::integral_constant<int, 2>{}); break;
    default: if constexpr (NGRP > 3) chain(std::integral_constant<int, 3>{}); break;
  }
  __syncthreads();
  for (int h = wave; h < G; h += kThreads / 64) select_one_head<D>(mag[h], keep, sel_idx + (row0 + h) * keep);
}

}  // namespace selb
}  // namespace dqk
