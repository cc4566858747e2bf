// Decode attention over the 2-bit cache with pruned query channels, split over
// the sequence; both contractions run on the matrix cores (MFMA).
//
// Dual-QK (arXiv abstract; tech.dede.sh summary, "Throughput on SGLang"):
// pruning removes key channels from reads and keys/values are stored in 2 bits,
// which is where the decode speedup comes from.  A work item is one
// (batch row, KV head, split of the sequence) and serves every query head of
// the GQA group.  Only the union U of the group's kept key channels is read:
// their 2-bit rows (channel-major, so a dropped channel costs no bytes), their
// per-group scales, channel 0's fp16 row and, for the unfinished last group,
// the exact tail.  Each head's logit uses only its own kept channels (its
// coefficient is zero on the others).  Values are never pruned.
//
// Arithmetic.  A 2-bit code u becomes the fp16 number v = 1 + u/4 by OR-ing the
// code into the mantissa (exact), and the level 2u-3 equals 8v - 11, so for any
// weights a: sum a (2u-3) = 8 sum a v - 11 sum a.  Both sums come from
// v_mfma_f32_16x16x32_f16 with fp32 accumulation:
//  - logits, per 32-token key group g: A[row][k] = q'_{h,U[k]} * scale * s_{U[k],g}
//    (scaled by 2^-E_h so |A| <= 65504) split into an fp16 high and low part
//    (rows h and G+h, about 22 significant bits), B[k][t] = v of key U[k] at
//    token t; a second product with B = 1 gives sum a.  The logit is
//    2^E_h * 8 (C - 1.375 C1) plus the fp32 channel-0 term;
//  - values, per 32 tokens: A[h][t] = p_{h,t} * s_{t,j} * 2^F in fp16 (p the
//    softmax numerator, s the value scale of channel group j, F a power of two
//    that puts the largest scaled scale below 2^15), B[t][c] = v of value (t, c);
//    sum a is accumulated alongside from the same fp16 numbers.
// The split is done in two passes: all logits of the split into LDS, one max
// per head, then the value pass with the final numerators (no rescaling).
//
// Work layout: 256 lanes (4 wavefronts), 256-token tiles staged through LDS.
// Key codes are re-interleaved while staging (v_perm byte transposes) so that
// one 8-byte LDS read gives a lane its 8 channels x 4 tokens; each wavefront
// builds the A operands of its groups in a compact layout and reads them back in
// MFMA layout.  Values: each wavefront owns d/4 output channels.  The partial
// (max, sum, output) of every head goes to the workspace for the combine.
#include "dqk_internal.h"

namespace dqk {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTile = 256;                      // tokens staged per tile
constexpr int kTileGroups = kTile / kGroup;     // 8 key groups per tile
constexpr uint32_t kOne2 = 0x3C003C00u;         // two fp16 1.0 (code 0)
constexpr uint32_t kCode2 = 0x03000300u;        // code bits -> fp16 mantissa bits 8..9

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

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {  // sum over the 16 lanes of a row
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

template <int D, int G>
struct Smem {
  union {
    struct {
      uint32_t y[D / 8][kTile / 4][2];  // key codes: channel octet, token quad, (4 ch, 4 ch)
      float sig[kTileGroups][D];        // key scales of the tile's groups, U order
      float ch0[kTile];                 // channel-0 keys of the tile
    } k;
    struct {
      uint32_t w[kTile / 16][D];        // value code words of the tile
      float sig[kTile][D / kGroup];     // value scales * 2^F
    } v;
  } st;
  uint32_t a[kWaves][D / 32][64][4];    // per-wavefront MFMA A operands
  float z[G][kMaxSplitTokensTimesG / G];  // logits of the split, then numerators
  float coefc[G][D];                    // q' * sm * log2(e) by channel (0 if dropped)
  float coefs[G][D];                    // coefc in U order * 2^-E_h (0 past |U|)
  float e8[G];                          // 8 * 2^E_h
  float redm[G][kWaves], redl[G][kWaves];
  float redf[kWaves];
  int hmask[D];
  int16_t ulist[D];
  int wcount[2];
};

template <int D, int G>
__global__ __launch_bounds__(kThreads, 2) void decode_kernel(dqk_cache c,
                                                             const float *__restrict__ qp,
                                                             const int32_t *__restrict__ sel,
                                                             int hq, int keep, float scale2,
                                                             int split, int nsplit,
                                                             float *__restrict__ ws) {
  __shared__ Smem<D, G> sm;
  constexpr int VG = D / kGroup;      // value scale groups per token
  constexpr int KCM = D / 32;         // K-chunks of 32 union slots (max)
  constexpr int OCT = D / 8;          // channel octets
  constexpr int NTW = D / 64;         // value N-tiles (16 channels) per wavefront
  constexpr int KQ = D / 8;           // union-slot octets per head
  constexpr int AREP = (KQ * G + 63) / 64;    // compact key A items per lane
  constexpr int AREPV = (16 * G + 63) / 64;   // compact value A items per lane
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, kg = lane >> 4;
  const int item = blockIdx.x;
  const int unit = item / nsplit, s = item % nsplit;
  const int b = unit / c.num_kv_heads, g = unit % c.num_kv_heads;
  const int len = max(0, min(c.lengths[b], c.capacity));
  const int t_begin = s * split;
  const int t_end = min(t_begin + split, len);
  float *wsp = ws + (size_t)item * G * (D + kPartialHead);
  if (t_begin >= t_end) {
    for (int e = tid; e < G * (D + kPartialHead); e += kThreads)
      wsp[e] = (e % (D + kPartialHead) == 0) ? -INFINITY : 0.0f;
    return;
  }

  const size_t kc_stride = (size_t)(c.capacity / 4);
  const size_t ks_stride = (size_t)(c.capacity / kGroup);
  const uint8_t *kcodes = c.k_codes + unit * (size_t)D * kc_stride;
  const uint16_t *kscales = c.k_scales + unit * (size_t)D * ks_stride;
  const uint16_t *c0row = c.k_ch0 + unit * (size_t)c.capacity;
  const float *tail = c.k_tail + unit * (size_t)kGroup * D;
  const uint32_t *vwords = c.v_codes + unit * (size_t)(c.capacity / 16) * D;
  const uint16_t *vscales = c.v_scales + unit * (size_t)c.capacity * VG;
  const int t_body = (len / kGroup) * kGroup;
  const int code_end = min(t_body, t_end);

  // ---------------------------------------------------------------- setup
  for (int e = tid; e < G * D; e += kThreads) sm.coefc[e / D][e % D] = 0.0f;
  for (int e = tid; e < D; e += kThreads) sm.hmask[e] = 0;
  {
    uint32_t *a = &sm.a[0][0][0][0];
    for (int e = tid; e < kWaves * KCM * 64 * 4; e += kThreads) a[e] = 0u;
  }
  __syncthreads();
  const size_t row0 = (size_t)b * hq + (size_t)g * G;
  for (int e = tid; e < G * keep; e += kThreads) {
    const int h = e / keep;
    const int ch = sel[(row0 + h) * keep + e % keep];
    if (ch >= 0 && ch < D) {
      atomicOr(&sm.hmask[ch], 1 << h);
      sm.coefc[h][ch] = qp[(row0 + h) * D + ch] * scale2;
    }
  }
  __syncthreads();
  {
    const bool f = tid < D && tid >= 1 && sm.hmask[tid] != 0;
    const unsigned long long m = __ballot(f);
    if (lane == 0 && wave < 2) sm.wcount[wave] = __popcll(m);
    // largest |coefficient| of each head over channels >= 1
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float v = (tid >= 1 && tid < D) ? fabsf(sm.coefc[h][tid]) : 0.0f;
      const float mx = wave_max(v);
      if (lane == 0) sm.redm[h][wave] = mx;
    }
    __syncthreads();
    if (f) sm.ulist[__popcll(m & ((1ull << lane) - 1ull)) + (wave == 1 ? sm.wcount[0] : 0)] = (int16_t)tid;
  }
  // scale exponent of the value pass: 2^F * max value scale of the split < 2^15
  float vmax = 0.0f;
  for (int t = t_begin + tid; t < t_end; t += kThreads) {
#pragma unroll
    for (int j = 0; j < VG; ++j) vmax = fmaxf(vmax, f16_value(vscales[(size_t)t * VG + j]));
  }
  vmax = wave_max(vmax);
  if (lane == 0) sm.redf[wave] = vmax;
  __syncthreads();
  const int nu = sm.wcount[0] + sm.wcount[1];
  const int nkc = (nu + 31) / 32;
  for (int e = tid; e < G * D; e += kThreads) {
    const int h = e / D, i = e % D;
    float mx = sm.redm[h][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, sm.redm[h][w]);
    int ex = 0;
    if (mx > 0.0f) frexpf(mx, &ex);
    sm.coefs[h][i] = i < nu ? sm.coefc[h][sm.ulist[i]] * ldexpf(1.0f, -ex) : 0.0f;
    if (i == 0) sm.e8[h] = ldexpf(8.0f, ex);
  }
  float fscale;
  {
    float vm = sm.redf[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) vm = fmaxf(vm, sm.redf[w]);
    int ev = 0;
    if (vm > 0.0f) frexpf(vm, &ev);
    fscale = ldexpf(1.0f, 15 - ev);
  }
  __syncthreads();

  // my fixed share of the compact A build: (head, 8 consecutive union slots)
  float myc[AREP][8];
#pragma unroll
  for (int rep = 0; rep < AREP; ++rep) {
    const int it = lane + 64 * rep;
#pragma unroll
    for (int i = 0; i < 8; ++i) myc[rep][i] = it < KQ * G ? sm.coefs[it / KQ][8 * (it % KQ) + i] : 0.0f;
  }

  // ---------------------------------------------------------------- key pass
  for (int tile0 = t_begin; tile0 < t_end; tile0 += kTile) {
    {  // stage key codes, re-interleaved: thread = (octet, 16-token block)
      const int o = tid >> 4, wb = tid & 15;
      const int tok = tile0 + 16 * wb;
      if (o < OCT) {
        uint32_t x[8];
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) {
          const int i = 8 * o + cc;
          x[cc] = (i < nu && tok < code_end)
                      ? *reinterpret_cast<const uint32_t *>(kcodes + (size_t)sm.ulist[i] * kc_stride + (tok >> 2))
                      : 0u;
        }
        uint32_t y0[4], y1[4];
        {
          const uint32_t a = __builtin_amdgcn_perm(x[0], x[2], 0x05010400u);
          const uint32_t bb = __builtin_amdgcn_perm(x[1], x[3], 0x05010400u);
          const uint32_t a2 = __builtin_amdgcn_perm(x[0], x[2], 0x07030602u);
          const uint32_t b2 = __builtin_amdgcn_perm(x[1], x[3], 0x07030602u);
          y0[0] = __builtin_amdgcn_perm(bb, a, 0x05040100u);
          y0[1] = __builtin_amdgcn_perm(bb, a, 0x07060302u);
          y0[2] = __builtin_amdgcn_perm(b2, a2, 0x05040100u);
          y0[3] = __builtin_amdgcn_perm(b2, a2, 0x07060302u);
        }
        {
          const uint32_t a = __builtin_amdgcn_perm(x[4], x[6], 0x05010400u);
          const uint32_t bb = __builtin_amdgcn_perm(x[5], x[7], 0x05010400u);
          const uint32_t a2 = __builtin_amdgcn_perm(x[4], x[6], 0x07030602u);
          const uint32_t b2 = __builtin_amdgcn_perm(x[5], x[7], 0x07030602u);
          y1[0] = __builtin_amdgcn_perm(bb, a, 0x05040100u);
          y1[1] = __builtin_amdgcn_perm(bb, a, 0x07060302u);
          y1[2] = __builtin_amdgcn_perm(b2, a2, 0x05040100u);
          y1[3] = __builtin_amdgcn_perm(b2, a2, 0x07060302u);
        }
        u32x4 *dst = reinterpret_cast<u32x4 *>(&sm.st.k.y[o][4 * wb][0]);
        dst[0] = u32x4{y0[0], y1[0], y0[1], y1[1]};
        dst[1] = u32x4{y0[2], y1[2], y0[3], y1[3]};
      }
    }
    if (tid < D) {  // key scales of the tile's groups (zero past the coded tokens)
#pragma unroll
      for (int gg = 0; gg < kTileGroups; ++gg) {
        const int grp = tile0 / kGroup + gg;
        sm.st.k.sig[gg][tid] = (tid < nu && grp * kGroup < code_end)
                                   ? f16_value(kscales[(size_t)sm.ulist[tid] * ks_stride + grp])
                                   : 0.0f;
      }
    }
    {
      const int t = tile0 + tid;
      sm.st.k.ch0[tid] = t < t_end ? f16_value(c0row[t]) : 0.0f;
    }
    __syncthreads();

    // wavefront w: key groups 2w and 2w+1 of the tile
#pragma unroll 1
    for (int gq = 0; gq < 2; ++gq) {
      const int gg = 2 * wave + gq;
      if (tile0 + kGroup * gg >= t_end) break;  // wavefront-uniform
      // compact A build: (head h, union slots 8kq..8kq+7) -> rows h (high) and G+h (low)
#pragma unroll
      for (int rep = 0; rep < AREP; ++rep) {
        const int it = lane + 64 * rep;
        if (it < KQ * G) {
          const int h = it / KQ, kq = it % KQ;
          const float *sg = &sm.st.k.sig[gg][8 * kq];
          uint32_t hi[4], lo[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float a0 = myc[rep][2 * i] * sg[2 * i];
            const float a1 = myc[rep][2 * i + 1] * sg[2 * i + 1];
            hi[i] = f16_pair(a0, a1);
            lo[i] = f16_pair(a0 - f16_low(hi[i]), a1 - f16_high(hi[i]));
          }
          const int kcx = kq >> 2, kgx = kq & 3;
          *reinterpret_cast<u32x4 *>(&sm.a[wave][kcx][16 * kgx + h][0]) = u32x4{hi[0], hi[1], hi[2], hi[3]};
          *reinterpret_cast<u32x4 *>(&sm.a[wave][kcx][16 * kgx + G + h][0]) = u32x4{lo[0], lo[1], lo[2], lo[3]};
        }
      }
      wave_sync();
      f32x4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = acc0, accs = acc0;
      const int r2 = 2 * (n16 & 3);
      const u32x4 ones = {kOne2, kOne2, kOne2, kOne2};
      for (int kc = 0; kc < nkc; ++kc) {
        const u32x4 A = *reinterpret_cast<const u32x4 *>(&sm.a[wave][kc][lane][0]);
        const int oct = 4 * kc + kg;
        const uint32_t *y = &sm.st.k.y[oct][8 * gg + (n16 >> 2)][0];
        const uint32_t y00 = y[0], y01 = y[1];           // N-tile 0 (tokens 0..15 of the group)
        const uint32_t y10 = y[8], y11 = y[9];           // N-tile 1 (quad + 4)
        const u32x4 b0 = {((y00 >> r2) & kCode2) | kOne2, ((y00 << (8 - r2)) & kCode2) | kOne2,
                          ((y01 >> r2) & kCode2) | kOne2, ((y01 << (8 - r2)) & kCode2) | kOne2};
        const u32x4 b1 = {((y10 >> r2) & kCode2) | kOne2, ((y10 << (8 - r2)) & kCode2) | kOne2,
                          ((y11 >> r2) & kCode2) | kOne2, ((y11 << (8 - r2)) & kCode2) | kOne2};
        acc0 = mfma16(A, b0, acc0);
        acc1 = mfma16(A, b1, acc1);
        accs = mfma16(A, ones, accs);
      }
      wave_sync();
      // rows r = 4*kg + i; high part row h, low part row G+h
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const f32x4 acc = nt == 0 ? acc0 : acc1;
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = acc[i] - 1.375f * accs[i];
        const int tokl = kGroup * gg + 16 * nt + n16;   // token within the tile
        const int t = tile0 + tokl;
        const float x0 = sm.st.k.ch0[tokl];
        if (G >= 4) {
          constexpr int OFF = 4 * G;  // lanes between high and low rows
          float w[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) w[i] = v[i] + __shfl_xor(v[i], OFF, 64);
          if (kg < G / 4) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int h = 4 * kg + i;
              const float zz = fmaf(sm.e8[h], w[i], sm.coefc[h][0] * x0);
              sm.z[h][t - t_begin] = t < t_end ? zz : -INFINITY;
            }
          }
        } else if (kg == 0) {
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float zz = fmaf(sm.e8[h], v[h] + v[G + h], sm.coefc[h][0] * x0);
            sm.z[h][t - t_begin] = t < t_end ? zz : -INFINITY;
          }
        }
      }
    }
    __syncthreads();
  }

  // tokens of the unfinished last group: exact fp32 tail keys
  {
    const int ta = max(t_begin, t_body);
    const int nt = t_end - ta;
    for (int e = tid; e < G * max(nt, 0); e += kThreads) {
      const int h = e / nt, t = ta + e % nt;
      float zz = sm.coefc[h][0] * f16_value(c0row[t]);
      for (int i = 0; i < nu; ++i) {
        const int ch = sm.ulist[i];
        zz = fmaf(sm.coefc[h][ch], tail[(size_t)(t & 31) * D + ch], zz);
      }
      sm.z[h][t - t_begin] = zz;
    }
  }
  __syncthreads();

  // ---------------------------------------------------------------- softmax
  const int nv = t_end - t_begin;
  const int nvp = (nv + kTile - 1) / kTile * kTile;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mx = -INFINITY;
    for (int t = tid; t < nv; t += kThreads) mx = fmaxf(mx, sm.z[h][t]);
    mx = wave_max(mx);
    if (lane == 0) sm.redm[h][wave] = mx;
  }
  __syncthreads();
  float mrow[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mx = sm.redm[h][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, sm.redm[h][w]);
    mrow[h] = mx;
    float ls = 0.0f;
    for (int t = tid; t < nvp; t += kThreads) {
      const float p = t < nv ? exp2f(sm.z[h][t] - mx) : 0.0f;
      sm.z[h][t] = p;
      ls += p;
    }
    ls = wave_sum(ls);
    if (lane == 0) sm.redl[h][wave] = ls;
  }
  __syncthreads();

  // ---------------------------------------------------------------- value pass
  // rows G..2G-1 of my A buffer held low parts: clear them
#pragma unroll
  for (int kc = 0; kc < KCM; ++kc)
    if (n16 >= G && n16 < 2 * G)
      *reinterpret_cast<u32x4 *>(&sm.a[wave][kc][lane][0]) = u32x4{0u, 0u, 0u, 0u};
  wave_sync();
  const int jgrp = (wave * NTW * 16) / kGroup;   // value scale group of my channels
  f32x4 vacc[NTW];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) vacc[nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float spart[AREPV];
#pragma unroll
  for (int rep = 0; rep < AREPV; ++rep) spart[rep] = 0.0f;

  for (int tile0 = t_begin; tile0 < t_end; tile0 += kTile) {
    for (int e = tid; e < (kTile / 16) * (D / 4); e += kThreads) {
      const int blk = e / (D / 4), c4 = e % (D / 4);
      const int tokb = tile0 + 16 * blk;
      u32x4 w = {0u, 0u, 0u, 0u};
      if (tokb < t_end) w = *reinterpret_cast<const u32x4 *>(vwords + (size_t)(tokb >> 4) * D + 4 * c4);
      *reinterpret_cast<u32x4 *>(&sm.st.v.w[blk][4 * c4]) = w;
    }
    {
      const int t = tile0 + tid;
#pragma unroll
      for (int j = 0; j < VG; ++j)
        sm.st.v.sig[tid][j] = t < t_end ? f16_value(vscales[(size_t)t * VG + j]) * fscale : 0.0f;
    }
    __syncthreads();
#pragma unroll 1
    for (int kc = 0; kc < kTile / 32; ++kc) {
      const int kt0 = tile0 + 32 * kc;
      if (kt0 >= t_end) break;   // uniform
      // compact numerators: (head h, pair pi) -> A dword pi&3 of lane 16*(pi>>2) + h
#pragma unroll
      for (int rep = 0; rep < AREPV; ++rep) {
        const int it = lane + 64 * rep;
        if (it < 16 * G) {
          const int h = it >> 4, pi = it & 15;
          const int kgx = pi >> 2, ii = pi & 3;
          const int r0 = 2 * (kgx & 1), d = ii & 1;
          const int tl = 16 * (kgx >> 1) + (ii < 2 ? 4 + r0 + d : r0 + d);
          const int zt = kt0 - t_begin;
          const float p0 = sm.z[h][zt + tl] * sm.st.v.sig[32 * kc + tl][jgrp];
          const float p1 = sm.z[h][zt + tl + 8] * sm.st.v.sig[32 * kc + tl + 8][jgrp];
          const uint32_t pk = f16_pair(p0, p1);
          spart[rep] += f16_low(pk) + f16_high(pk);
          sm.a[wave][0][16 * kgx + h][ii] = pk;
        }
      }
      wave_sync();
      const u32x4 A = *reinterpret_cast<const u32x4 *>(&sm.a[wave][0][lane][0]);
      const int blk = 2 * kc + (kg >> 1);
      const int r0 = 2 * (kg & 1);
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const int ch = (wave * NTW + nt) * 16 + n16;
        const uint32_t w = sm.st.v.w[blk][ch];
        const u32x4 bv = {((w >> (2 * r0)) & kCode2) | kOne2, ((w >> (2 * r0 + 2)) & kCode2) | kOne2,
                          ((w << (8 - 2 * r0)) & kCode2) | kOne2, ((w << (6 - 2 * r0)) & kCode2) | kOne2};
        vacc[nt] = mfma16(A, bv, vacc[nt]);
      }
      wave_sync();
    }
    __syncthreads();
  }

  // ---------------------------------------------------------------- partials
  float ssum[AREPV];
#pragma unroll
  for (int rep = 0; rep < AREPV; ++rep) ssum[rep] = row16_sum(spart[rep]);
  const float inv_f = 1.0f / fscale;
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int ch = (wave * NTW + nt) * 16 + n16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * kg + i;                    // C row of this register
      // sum of the numerators of head h: lanes 16*(h%4).. of compact repeat h/4
      const int hh = h < G ? h : 0;
      float sh = 0.0f;
#pragma unroll
      for (int rep = 0; rep < AREPV; ++rep) {
        const float x = __shfl(ssum[rep], 16 * (hh % 4), 64);
        if (rep == hh / 4) sh = x;
      }
      if (h < G) wsp[h * (D + kPartialHead) + kPartialHead + ch] = (8.0f * vacc[nt][i] - 11.0f * sh) * inv_f;
    }
  }
  if (tid < G) {
    float ls = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) ls += sm.redl[tid][w];
    wsp[tid * (D + kPartialHead) + 0] = mrow[tid];
    wsp[tid * (D + kPartialHead) + 1] = ls;
  }
}

template <int D, int G>
hipError_t launch_decode_t(const dqk_cache &c, const float *qp, const int32_t *sel, int hq,
                           int keep, float scale2, int split, float *out, float *ws,
                           hipStream_t s) {
  const int nsplit = num_splits(c.capacity, split);
  const int items = c.batch * c.num_kv_heads * nsplit;
  hipLaunchKernelGGL((decode_kernel<D, G>), dim3((unsigned)items), dim3(kThreads), 0, s, c, qp,
                     sel, hq, keep, scale2, split, nsplit, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_combine(ws, c.batch, hq, c.num_kv_heads, D, nsplit, out, s);
}

template <int D>
hipError_t launch_decode_d(const dqk_cache &c, const float *qp, const int32_t *sel, int hq,
                           int keep, float scale2, int split, float *out, float *ws,
                           hipStream_t s) {
  switch (hq / c.num_kv_heads) {
    case 1: return launch_decode_t<D, 1>(c, qp, sel, hq, keep, scale2, split, out, ws, s);
    case 2: return launch_decode_t<D, 2>(c, qp, sel, hq, keep, scale2, split, out, ws, s);
    case 4: return launch_decode_t<D, 4>(c, qp, sel, hq, keep, scale2, split, out, ws, s);
    default: return launch_decode_t<D, 8>(c, qp, sel, hq, keep, scale2, split, out, ws, s);
  }
}

}  // namespace

hipError_t launch_decode(const dqk_cache &c, const float *q_prime, const int32_t *sel_idx, int hq,
                         int keep, float sm_scale, int split, float *out, float *ws,
                         hipStream_t s) {
  const float scale2 = sm_scale * 1.4426950408889634f;  // logits in log2 units
  if (c.head_dim == 64) return launch_decode_d<64>(c, q_prime, sel_idx, hq, keep, scale2, split, out, ws, s);
  return launch_decode_d<128>(c, q_prime, sel_idx, hq, keep, scale2, split, out, ws, s);
}

}  // namespace dqk
