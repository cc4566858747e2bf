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
// (bit-reproducible); then every channel's rank in the order (|q'| descending,
// index ascending) is counted exactly -- the workgroup's wavefronts each
// compare against a slice of the channels -- the channels of rank below keep-1
// are kept, and ballot prefixes give each kept channel its ascending slot.  Built with
// -ffp-contract=off.
#pragma once
#include "dqk_internal.h"

#include <type_traits>

namespace dqk {
namespace selb {

constexpr int kThreads = 256;

__device__ __forceinline__ int popc(unsigned long long m) { return __popcll(m); }

// Order key of channel c with magnitude |q'_c|: non-negative floats order like
// their bit patterns, and the low bits (D-1-c) put the lower index first among
// equal magnitudes, so every channel's key is distinct and the larger key
// comes first.  Channel 0 gets key 0: it is kept apart from the competition
// and no key counted against another is ever 0 (a key is counted when it is
// larger).
template <int D>
__device__ __forceinline__ uint64_t order_key(float x, int c) {
  static_assert(D <= 128, "index field of 7 bits");
  return c == 0 ? 0ull : ((uint64_t)__float_as_uint(fabsf(x)) << 7) | (uint64_t)(D - 1 - c);
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
  constexpr int WPH = kThreads / 64 / HPB;      // wavefronts per head in the ranking
  constexpr int SL = D / WPH;                   // channels each wavefront compares against
  constexpr int CPL = D / 64;                   // channels per lane
  static_assert(D % 64 == 0 && SL % 2 == 0, "whole wavefronts and key pairs");
  __shared__ __attribute__((aligned(16))) uint64_t key[HPB][D];
  __shared__ uint32_t part[HPB][WPH][D];
  const int unit = block / NSUB, h0 = (block % NSUB) * HPB;
  const int b = unit / hkv, g = unit % hkv;
  const size_t row0 = (size_t)b * hq + (size_t)g * G + h0;
  const int j = threadIdx.x, wave = j >> 6;
  const int col = j % D, grp = j / D;                 // grp is uniform in a wavefront
  const int nh = min(HPB, G - h0);                    // heads of this workgroup
  // The lane's whole column of A_g is loaded at once (thread groups without a
  // head load nothing); the chain below consumes its rows in order as they land.
  float a[D];
  if (grp < nh) {
    const float *acol = amat + (size_t)g * D * D + col;
#pragma unroll
    for (int r = 0; r < D; ++r) a[r] = acol[(size_t)r * D];
  }
  // The query row is the same for every lane of the thread group: it is read
  // from memory as the chain goes (uniform addresses, no LDS and no barrier), so
  // that each FMA waits only for its own row of A and element of q.  (Staging q
  // in LDS made every chain wait at a barrier for the whole column of A.)
  auto chain = [&](auto grp_c) {
    constexpr int GRP = decltype(grp_c)::value;
    const size_t qrow = (row0 + GRP) * D;
    float acc = 0.0f;
#pragma unroll
    for (int r = 0; r < D; ++r) {
      float qv;
      if constexpr (BF16)
        qv = bf16_value(static_cast<const uint16_t *>(q)[qrow + r]);
      else
        qv = static_cast<const float *>(q)[qrow + r];
      acc = __builtin_fmaf(qv, a[r], acc);
    }
    q_prime[(row0 + GRP) * D + col] = acc;
    key[GRP][col] = order_key<D>(acc, col);
  };
  static_assert(HPB <= 2, "thread groups with a head");
  if (grp == 0 && nh > 0) chain(std::integral_constant<int, 0>{});
  else if constexpr (HPB > 1) { if (grp == 1 && nh > 1) chain(std::integral_constant<int, 1>{}); }
  __syncthreads();
  // Rank of channel c: the number of channels whose key is larger.  Wavefront
  // w counts, for head w / WPH, against channels [SL * (w % WPH), + SL).
  const int lane = j & 63;
  {
    const int hh = wave / WPH, p = wave % WPH;
    if (hh < nh) {
      uint64_t mine[CPL];
      uint32_t r[CPL];
#pragma unroll
      for (int i = 0; i < CPL; ++i) { mine[i] = key[hh][lane + 64 * i]; r[i] = 0; }
      const uint64_t *ks = &key[hh][SL * p];
#pragma unroll
      for (int e = 0; e < SL; ++e)
#pragma unroll
        for (int i = 0; i < CPL; ++i) r[i] += ks[e] > mine[i] ? 1u : 0u;
#pragma unroll
      for (int i = 0; i < CPL; ++i) part[hh][p][lane + 64 * i] = r[i];
    }
  }
  __syncthreads();
  // Wavefront h keeps channel 0 and the channels of rank below keep - 1 of its
  // head and writes their indices in ascending order.
  if (wave < nh) {
    const unsigned long long below = (1ull << lane) - 1ull;
    int base = 0;
    int32_t *idx = sel_idx + (row0 + wave) * keep;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = lane + 64 * i;
      uint32_t rank = 0;
#pragma unroll
      for (int p = 0; p < WPH; ++p) rank += part[wave][p][c];
      const bool s = c == 0 || (int)rank < keep - 1;
      const unsigned long long m = __ballot(s);
      if (s) idx[base + popc(m & below)] = c;
      base += popc(m);
    }
  }
}

// Group-shared selection (one kept set per KV head): workgroup BLOCK serves
// (batch row, KV head) BLOCK.  Thread j holds column c = j % D of A_g and forms
// q'_c of the group's heads grp, grp + NGRP, ... (grp = j / D, NGRP = 256 / D
// thread groups), each one fp32 FMA chain over input channels in ascending
// order, as in select_block; the column of A_g is read once for the whole
// group.  Channel c's score is then |q'_{0,c}| + |q'_{1,c}| + ... in fp32 from
// +0 in ascending head order, ranked exactly like |q'_c| above (the order key of
// a non-negative score), and the first wavefront writes the kept set of the
// unit to sel_idx[BLOCK][keep] in ascending order.
template <int D, int G, bool BF16>
__device__ __forceinline__ void select_shared_block(int block, const void *q,
                                                    const float *__restrict__ amat, int hq,
                                                    int hkv, int keep, float *q_prime,
                                                    int32_t *sel_idx) {
  constexpr int NGRP = kThreads / D;            // thread groups: heads in flight at once
  constexpr int HPG = (G + NGRP - 1) / NGRP;    // heads per thread group at most
  constexpr int WPH = kThreads / 64;            // wavefronts ranking the one score row
  constexpr int SL = D / WPH;                   // channels each wavefront compares against
  constexpr int CPL = D / 64;                   // channels per lane
  static_assert(D % 64 == 0 && SL % 2 == 0, "whole wavefronts and key pairs");
  __shared__ float qs[G][D];
  __shared__ float qps[G][D];
  __shared__ __attribute__((aligned(16))) uint64_t key[D];
  __shared__ uint32_t part[WPH][D];
  const int unit = block;
  const int b = unit / hkv, g = unit % hkv;
  const size_t row0 = (size_t)b * hq + (size_t)g * G;
  const int j = threadIdx.x, wave = j >> 6, lane = j & 63;
  const int col = j % D, grp = j / D;           // grp is uniform in a wavefront
  // the group's query rows and the lane's column of A_g, loaded together (one round trip)
  float a[D];
  const float *acol = amat + (size_t)g * D * D + col;
#pragma unroll
  for (int r = 0; r < D; ++r) a[r] = acol[(size_t)r * D];
  for (int e = j; e < G * D; e += kThreads) {
    const size_t at = row0 * D + e;
    float qv;
    if constexpr (BF16)
      qv = bf16_value(static_cast<const uint16_t *>(q)[at]);
    else
      qv = static_cast<const float *>(q)[at];
    qs[e / D][e % D] = qv;
  }
#pragma unroll
  for (int r = 0; r < D; ++r) asm volatile("" ::"v"(a[r]));
  __syncthreads();
  // q' of head H (a compile-time row, so that the chain's LDS reads are not all
  // hoisted at once)
  auto chain = [&](auto h_c) {
    constexpr int H = decltype(h_c)::value;
    float acc = 0.0f;
#pragma unroll
    for (int r = 0; r < D; ++r) acc = __builtin_fmaf(qs[H][r], a[r], acc);
    q_prime[(row0 + H) * D + col] = acc;
    qps[H][col] = acc;
  };
  auto chains = [&](auto grp_c) {
    constexpr int GR = decltype(grp_c)::value;
    if constexpr (GR + 0 * NGRP < G) chain(std::integral_constant<int, GR + 0 * NGRP>{});
    if constexpr (HPG > 1 && GR + 1 * NGRP < G) chain(std::integral_constant<int, GR + 1 * NGRP>{});
    if constexpr (HPG > 2 && GR + 2 * NGRP < G) chain(std::integral_constant<int, GR + 2 * NGRP>{});
    if constexpr (HPG > 3 && GR + 3 * NGRP < G) chain(std::integral_constant<int, GR + 3 * NGRP>{});
    if constexpr (HPG > 4 && GR + 4 * NGRP < G) chain(std::integral_constant<int, GR + 4 * NGRP>{});
    if constexpr (HPG > 5 && GR + 5 * NGRP < G) chain(std::integral_constant<int, GR + 5 * NGRP>{});
    if constexpr (HPG > 6 && GR + 6 * NGRP < G) chain(std::integral_constant<int, GR + 6 * NGRP>{});
    if constexpr (HPG > 7 && GR + 7 * NGRP < G) chain(std::integral_constant<int, GR + 7 * NGRP>{});
  };
  static_assert(HPG <= 8 && NGRP <= 4, "heads per thread group, thread groups");
  if (grp == 0) chains(std::integral_constant<int, 0>{});
  else if (grp == 1) { if constexpr (NGRP > 1) chains(std::integral_constant<int, 1>{}); }
  else if (grp == 2) { if constexpr (NGRP > 2) chains(std::integral_constant<int, 2>{}); }
  else { if constexpr (NGRP > 3) chains(std::integral_constant<int, 3>{}); }
  __syncthreads();
  // the group's score of each channel, summed over heads in ascending order
  for (int c = j; c < D; c += kThreads) {
    float sc = 0.0f;
#pragma unroll
    for (int h = 0; h < G; ++h) sc = sc + fabsf(qps[h][c]);
    key[c] = order_key<D>(sc, c);
  }
  __syncthreads();
  {
    uint64_t mine[CPL];
    uint32_t r[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) { mine[i] = key[lane + 64 * i]; r[i] = 0; }
    const uint64_t *ks = &key[SL * wave];
#pragma unroll
    for (int e = 0; e < SL; ++e)
#pragma unroll
      for (int i = 0; i < CPL; ++i) r[i] += ks[e] > mine[i] ? 1u : 0u;
#pragma unroll
    for (int i = 0; i < CPL; ++i) part[wave][lane + 64 * i] = r[i];
  }
  __syncthreads();
  if (wave == 0) {
    const unsigned long long below = (1ull << lane) - 1ull;
    int base = 0;
    int32_t *idx = sel_idx + (size_t)unit * keep;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = lane + 64 * i;
      uint32_t rank = 0;
#pragma unroll
      for (int p = 0; p < WPH; ++p) rank += part[p][c];
      const bool s = c == 0 || (int)rank < keep - 1;
      const unsigned long long m = __ballot(s);
      if (s) idx[base + popc(m & below)] = c;
      base += popc(m);
    }
  }
}

}  // namespace selb
}  // namespace dqk
