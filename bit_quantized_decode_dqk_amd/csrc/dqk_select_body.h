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
// A workgroup of 256 lanes serves one query head (two for head_dim 64): every
// output is an fp32 FMA chain over input channels in ascending order
// (bit-reproducible); then one wavefront per head finds the head's exact top-k
// by a bitwise search over the magnitudes' bit patterns with ballots, and
// ballot prefixes give each kept channel its ascending slot.  Built with
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

// Heads per workgroup: one thread group of D lanes per head, and at most half
// of the workgroup's lanes, so that a workgroup reads A_g (D*D floats) at most
// twice: for D = 128 one head per workgroup.  The G heads of a KV head
// therefore take several workgroups, each on its own CU: the per-CU load of A_g
// sets the length of the setup.
template <int D>
constexpr int heads_per_block() { return kThreads / D >= 4 ? kThreads / D / 2 : 1; }

template <int D, int G>
constexpr int blocks_per_unit() { return (G + heads_per_block<D>() - 1) / heads_per_block<D>(); }

// Workgroup BLOCK serves (batch row, KV head) BLOCK / blocks_per_unit and, of
// that group's query heads, the heads_per_block heads from (BLOCK mod
// blocks_per_unit) * heads_per_block on.  Thread j of thread group t (j / D)
// forms q'_c for column c = j % D of head t; each of the first waves then
// selects one head.
template <int D, int G, bool BF16>
__device__ __forceinline__ void select_block(int block, const void *q,
                                             const float *__restrict__ amat, int hq, int hkv,
                                             int keep, float *q_prime, int32_t *sel_idx) {
  constexpr int HPB = heads_per_block<D>(), NSUB = blocks_per_unit<D, G>();
  static_assert(HPB * D <= kThreads && HPB * 64 <= kThreads, "one thread group and one wave per head");
  __shared__ float qs[HPB][D];
  __shared__ float mag[HPB][D];
  const int unit = block / NSUB, h0 = (block % NSUB) * HPB;
  const int b = unit / hkv, g = unit % hkv;
  const size_t row0 = (size_t)b * hq + (size_t)g * G + h0;
  const int j = threadIdx.x, wave = j >> 6;
  const int col = j % D, grp = j / D;                 // grp is uniform in a wavefront
  const int nh = min(HPB, G - h0);                    // heads of this workgroup
  // The query value and the lane's whole column of A_g are loaded together:
  // the setup is one round trip.  Thread groups without a head load nothing.
  float a[D];
  if (grp < nh) {
    const size_t e = (row0 + grp) * D + col;
    float qv;
    if constexpr (BF16)
      qv = bf16_value(static_cast<const uint16_t *>(q)[e]);
    else
      qv = static_cast<const float *>(q)[e];
    const float *acol = amat + (size_t)g * D * D + col;
#pragma unroll
    for (int r = 0; r < D; ++r) a[r] = acol[(size_t)r * D];
    qs[grp][col] = qv;
    // A's column is used here so that its loads are issued before the
    // barrier, together with the query load (A is read-only: the compiler
    // would otherwise move them past the barrier, a second round trip)
#pragma unroll
    for (int r = 0; r < D; ++r) asm volatile("" ::"v"(a[r]));
  }
  __syncthreads();
  // the thread group's row of qs at a compile-time index (a runtime row makes
  // the compiler hoist every LDS read of the chain at once)
  auto chain = [&](auto grp_c) {
    constexpr int GRP = decltype(grp_c)::value;
    float acc = 0.0f;
#pragma unroll
    for (int r = 0; r < D; ++r) acc = __builtin_fmaf(qs[GRP][r], a[r], acc);
    q_prime[(row0 + GRP) * D + col] = acc;
    mag[GRP][col] = fabsf(acc);
  };
  static_assert(HPB <= 2, "thread groups with a head");
  if (grp == 0 && nh > 0) chain(std::integral_constant<int, 0>{});
  else if constexpr (HPB > 1) { if (grp == 1 && nh > 1) chain(std::integral_constant<int, 1>{}); }
  __syncthreads();
  if (wave < nh) select_one_head<D>(mag[wave], keep, sel_idx + (row0 + wave) * keep);
}

}  // namespace selb
}  // namespace dqk
