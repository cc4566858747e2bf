// Append step (the body of one workgroup, shared by the append kernel and the
// fused append + selection kernel): key transform, channel-0 protection, per-channel key groups,
// per-token value groups, 2-bit packing -- fused in one kernel.
//
// Dual-QK (arXiv abstract; tech.dede.sh summary, "Paired transforms instead of
// shared rotation" and "Throughput on SGLang"): new keys go through the key
// transform k' = k B, keys and values are stored in 2 bits with an fp16 scale
// per group of 32, and channel 0 of the key is protected (kept in fp16 here).
//
// One workgroup handles one 32-token key group of one (batch row, KV head):
// the new tokens of that group are transformed (each output one fp32 FMA chain
// over input channels in ascending order, so the result is reproducible bit for
// bit), channel 0 goes to fp16, and either the group is complete -- then every
// channel 1..d-1 is quantized over its 32 tokens and packed as 8 bytes -- or the
// exact values go to the tail rows.  Value rows are quantized per token in
// 32-channel groups; their codes are merged into the 16-token words of the
// channel-blocked value plane.  Built with -ffp-contract=off.
#pragma once
#include "dqk_internal.h"

namespace dqk {
namespace appb {

constexpr int kThreads = 256;

// BULK workgroups write the transformed keys over the new keys once every
// thread is through with the transform (a smaller workgroup footprint, so that
// more of them share a compute unit); the others keep both.
template <int D, bool BULK>
struct __attribute__((aligned(16))) AppendSmem {
  float kx[kGroup][D];                 // new keys of the group (fp32)
  float kpo[BULK ? 1 : kGroup][D];     // transformed keys (not BULK)
  float vx[kGroup][D];                 // new values (fp32)
  float v2s[kGroup][D / kGroup];       // 2*scale per (token, value group)
  __device__ __forceinline__ float (*kp())[D] {
    if constexpr (BULK) return kx;
    else return kpo;
  }
};

template <bool BF16>
__device__ __forceinline__ float load_in(const void *p, size_t i) {
  if constexpr (BF16) return bf16_value(static_cast<const uint16_t *>(p)[i]);
  else return static_cast<const float *>(p)[i];
}

// bcol: this thread's column j = tid % D of B_g, all D rows, loaded at kernel
// start before anything waits (used by appends of at most one token per thread
// slot).  Otherwise the rows of B are streamed from bmat: one output channel per
// thread, or in BULK workgroups 4 channels x 4 tokens per thread (16-byte loads
// of B rows and of the inputs in LDS).  Every form runs the same FMA chain per
// output in the same order, so they agree bit for bit.
template <int D, bool BF16, bool BULK>
__device__ __forceinline__ void store_group(const dqk_cache &c, int b, int g, int grp, int L, int n,
                                            const void *k_new, const void *v_new,
                                            const float (&bcol)[D], const float *__restrict__ bmat,
                                            int max_new, AppendSmem<D, BULK> &sm) {
  const int tid = threadIdx.x;
  float (*kp)[D] = sm.kp();
  const int lo = max(L, grp * kGroup);
  const int hi = min(L + n, grp * kGroup + kGroup);
  const int cnt = hi - lo;                    // new tokens in this group, 1..32
  const size_t unit = unit_index(c, b, g);
  const size_t row0 = (unit * (size_t)max_new + (size_t)(lo - L)) * D;

  // The group's value words (two 16-token words per channel, one per thread)
  // are read now, in flight with the inputs, and rewritten at the end.
  static_assert(2 * D <= kThreads, "one value word per thread");
  const int vch = tid % D, vhalf = (tid / D) & 1;
  const int wlo = grp * kGroup + vhalf * 16;
  const int va = max(wlo, lo), vz = min(wlo + 16, hi);   // new tokens of this word: [va, vz)
  uint32_t *wp = c.v_codes + (unit * (size_t)(c.capacity / 16) + (size_t)(wlo >> 4)) * D + vch;
  const uint32_t wold = *wp;

  if constexpr (BULK) {
    // the whole group's inputs in one round trip: every load is issued before
    // any is written to LDS (indices past the new tokens are clamped to the
    // last element and not written)
    constexpr int EPT = kGroup * D / kThreads;
    float kv[EPT], vv[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int ec = min(tid + kThreads * j, cnt * D - 1);
      kv[j] = load_in<BF16>(k_new, row0 + ec);
      vv[j] = load_in<BF16>(v_new, row0 + ec);
    }
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int e = tid + kThreads * j;
      if (e < cnt * D) {
        sm.kx[e / D][e % D] = kv[j];
        sm.vx[e / D][e % D] = vv[j];
      }
    }
  } else {
    // two elements of k and of v per thread in flight; the second index is
    // clamped to the last element, which is then written twice with the same
    // value (no branch, so no load waits behind another)
    for (int e0 = tid; e0 < cnt * D; e0 += 2 * kThreads) {
      const int e1 = min(e0 + kThreads, cnt * D - 1);
      const float k0 = load_in<BF16>(k_new, row0 + e0), v0 = load_in<BF16>(v_new, row0 + e0);
      const float k1 = load_in<BF16>(k_new, row0 + e1), v1 = load_in<BF16>(v_new, row0 + e1);
      sm.kx[e0 / D][e0 % D] = k0;
      sm.vx[e0 / D][e0 % D] = v0;
      sm.kx[e1 / D][e1 % D] = k1;
      sm.vx[e1 / D][e1 % D] = v1;
    }
  }
  __syncthreads();

  // k' = k B, each output one FMA chain over the input channels in ascending order
  if constexpr (BULK) {
    // 4 output channels x TPT tokens per thread: per step of 4 input channels, 4 rows
    // of B (16-byte loads; the next step's in flight) and TPT 16-byte LDS reads of the
    // tokens' inputs feed 16 TPT FMAs.  bmat is 16-byte aligned for this form.
    typedef float f4 __attribute__((ext_vector_type(4)));
    constexpr int CG = D / 4, TG = kThreads / CG, TPT = kGroup / TG;
    const int cj = 4 * (tid % CG), tr = TPT * (tid / CG);
    const f4 *brow = reinterpret_cast<const f4 *>(bmat + (size_t)g * D * D + cj);   // row i: brow[i * D / 4]
    float acc[TPT][4];
#pragma unroll
    for (int rr = 0; rr < TPT; ++rr)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) acc[rr][jj] = 0.0f;
    f4 bq[4], bn[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) bq[ii] = brow[(size_t)ii * (D / 4)];
#pragma unroll 2
    for (int i0 = 0; i0 < D; i0 += 4) {
      const int i1 = i0 + 4 < D ? i0 + 4 : i0;   // the last step re-reads its own rows
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) bn[ii] = brow[(size_t)(i1 + ii) * (D / 4)];
      f4 kq[TPT];
#pragma unroll
      for (int rr = 0; rr < TPT; ++rr) kq[rr] = *reinterpret_cast<const f4 *>(&sm.kx[tr + rr][i0]);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
#pragma unroll
        for (int rr = 0; rr < TPT; ++rr)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) acc[rr][jj] = __builtin_fmaf(kq[rr][ii], bq[ii][jj], acc[rr][jj]);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) bq[ii] = bn[ii];
    }
    __syncthreads();   // every thread is through with the new keys, which the results overwrite
#pragma unroll
    for (int rr = 0; rr < TPT; ++rr)
      if (tr + rr < cnt) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) kp[tr + rr][cj + jj] = acc[rr][jj];
      }
  } else {
    constexpr int S = kThreads / D;           // token slots per channel
    constexpr int R = kGroup / S;             // tokens per thread at most
    const int j = tid % D, r0 = tid / D;
    if (cnt <= S) {                            // decode-step appends: one token per thread
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < D; ++i) acc = __builtin_fmaf(sm.kx[r0][i], bcol[i], acc);
      if (r0 < cnt) kp[r0][j] = acc;
    } else {
      // rows of B fetched kBRows at a time, the next batch in flight while the
      // current one is used (the FMA order per output is unchanged)
      constexpr int kBRows = 16;
      const float *bc = bmat + (size_t)g * D * D + j;
      float acc[R];
#pragma unroll
      for (int m = 0; m < R; ++m) acc[m] = 0.0f;
      float bv[kBRows], bn[kBRows];
#pragma unroll
      for (int r = 0; r < kBRows; ++r) bv[r] = bc[(size_t)r * D];
#pragma unroll 1
      for (int i0 = 0; i0 < D; i0 += kBRows) {   // (a full unroll would spill)
        const int i1 = i0 + kBRows < D ? i0 + kBRows : i0;   // the last batch re-reads itself
#pragma unroll
        for (int r = 0; r < kBRows; ++r) bn[r] = bc[(size_t)(i1 + r) * D];
#pragma unroll
        for (int r = 0; r < kBRows; ++r)
#pragma unroll
          for (int m = 0; m < R; ++m)
            acc[m] = __builtin_fmaf(sm.kx[r0 + m * S][i0 + r], bv[r], acc[m]);
#pragma unroll
        for (int r = 0; r < kBRows; ++r) bv[r] = bn[r];
      }
#pragma unroll
      for (int m = 0; m < R; ++m)
        if (r0 + m * S < cnt) kp[r0 + m * S][j] = acc[m];
    }
  }
  __syncthreads();

  uint16_t *ch0 = c.k_ch0 + unit * (size_t)c.capacity;
  for (int r = tid; r < cnt; r += kThreads) ch0[lo + r] = f16_bits(kp[r][0]);

  if (hi == grp * kGroup + kGroup) {
    // The group is complete: quantize channels 1..D-1 over its 32 tokens.
    const float *tail = c.k_tail + unit * (size_t)kGroup * D;
    for (int ch = 1 + tid; ch < D; ch += kThreads) {
      float x[kGroup];
      float mx = 0.0f;
#pragma unroll
      for (int r = 0; r < kGroup; ++r) {
        const int p = grp * kGroup + r;
        x[r] = p < lo ? tail[(size_t)r * D + ch] : kp[p - lo][ch];
        mx = fmaxf(mx, fabsf(x[r]));
      }
      const uint16_t sb = f16_bits(mx / 3.0f);
      const float two_s = 2.0f * f16_value(sb);
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        w0 |= code_of(x[r], two_s) << (2 * r);
        w1 |= code_of(x[r + 16], two_s) << (2 * r);
      }
      uint8_t *row = c.k_codes + (unit * D + ch) * (size_t)(c.capacity / 4);
      *reinterpret_cast<uint2 *>(row + (size_t)grp * 8) = make_uint2(w0, w1);
      c.k_scales[(unit * D + ch) * (size_t)(c.capacity / kGroup) + grp] = sb;
    }
  } else {
    float *tail = c.k_tail + unit * (size_t)kGroup * D;
    for (int e = tid; e < cnt * D; e += kThreads)
      tail[(size_t)((lo + e / D) & 31) * D + e % D] = kp[e / D][e % D];
  }

  // Value scales: one per (new token, 32-channel group).
  constexpr int VG = D / kGroup;
  uint16_t *vsc = c.v_scales + unit * (size_t)c.capacity * VG;
  for (int e = tid; e < cnt * VG; e += kThreads) {
    const int r = e / VG, jg = e % VG;
    float mx = 0.0f;
#pragma unroll
    for (int i = 0; i < kGroup; ++i) mx = fmaxf(mx, fabsf(sm.vx[r][jg * kGroup + i]));
    const uint16_t sb = f16_bits(mx / 3.0f);
    vsc[(size_t)(lo + r) * VG + jg] = sb;
    sm.v2s[r][jg] = 2.0f * f16_value(sb);
  }
  __syncthreads();

  // Value codes: merge the new tokens' codes into the word read at the start
  // (a word without new tokens is written back unchanged).
  uint32_t w = wold;
  for (int p = va; p < vz; ++p) {
    const int sh = 2 * (p & 15);
    const uint32_t u = code_of(sm.vx[p - lo][vch], sm.v2s[p - lo][vch / kGroup]);
    w = (w & ~(3u << sh)) | (u << sh);
  }
  if (tid < 2 * D) *wp = w;
  __syncthreads();
}

// BULK: appends of many tokens per row (prefill), which never use a held column of
// B; such workgroups load none, and hold no registers for one.
template <int D, bool BF16, bool BULK = false>
__device__ __forceinline__ void append_block(int block, const dqk_cache &c, const void *k_new,
                                             const void *v_new, const float *__restrict__ bmat,
                                             const int32_t *__restrict__ n_new, int max_new,
                                             int blocks_per_unit) {
  __shared__ AppendSmem<D, BULK> sm;
  const int unit = block / blocks_per_unit;
  const int bi = block % blocks_per_unit;
  const int b = unit / c.num_kv_heads, g = unit % c.num_kv_heads;
  // column tid % D of B_g, in flight together with the length.  Only threads
  // whose token slot tid / D can hold a new token use it (a group gets at most
  // max_new of them); the others load nothing, which halves the workgroup's
  // reads of B_g for one-token appends.
  float bcol[D];
  if constexpr (!BULK) {
    if ((int)(threadIdx.x / D) < max_new) {
      const float *bp = bmat + (size_t)g * D * D + threadIdx.x % D;
#pragma unroll
      for (int i = 0; i < D; ++i) bcol[i] = bp[(size_t)i * D];
    } else {
#pragma unroll
      for (int i = 0; i < D; ++i) bcol[i] = 0.0f;
    }
  }
  const int L = c.lengths[b];
  const int n = max(0, min(min(n_new[b], max_new), c.capacity - L));
  if (n <= 0) return;
  const int g0 = L / kGroup, g1 = (L + n - 1) / kGroup;
  // The first group may read old tail rows while the last (unfinished) group
  // writes tail rows; then one workgroup does both, first before last.
  const bool merged = g1 > g0 && (L % kGroup) != 0 && ((L + n) % kGroup) != 0;
  const int ngroups = g1 - g0 + 1;
  if (bi < ngroups && !(merged && bi == ngroups - 1)) {
    store_group<D, BF16, BULK>(c, b, g, g0 + bi, L, n, k_new, v_new, bcol, bmat, max_new, sm);
    if (merged && bi == 0)
      store_group<D, BF16, BULK>(c, b, g, g1, L, n, k_new, v_new, bcol, bmat, max_new, sm);
  }
  // Length commit: every workgroup of the row (with or without a group to store)
  // counts itself in on the row's arrival counter once all of its wavefronts
  // have read the length (the barrier); the last of the row's num_kv_heads *
  // blocks_per_unit workgroups writes the new length, and the counter wraps
  // back to zero for the next append.  So no wavefront of the row can read the
  // new length in this launch.
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned total = (unsigned)(c.num_kv_heads * blocks_per_unit);
    unsigned *arrivals = reinterpret_cast<unsigned *>(c.lengths + c.batch);
    if (atomicInc(&arrivals[b], total - 1) == total - 1) c.lengths[b] = L + n;
  }
}

}  // namespace appb
}  // namespace dqk
