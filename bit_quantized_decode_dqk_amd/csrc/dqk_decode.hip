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
#include "dqk_wave.h"

namespace dqk {
namespace {

using namespace wave;

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr uint32_t kOne2 = 0x3C003C00u;         // two fp16 1.0 (code 0)
constexpr uint32_t kCode2 = 0x03000300u;        // code bits -> fp16 mantissa bits 8..9

constexpr int kTok = 64;   // tokens per wavefront tile (two key groups)
constexpr int kYRow = kTok / 4 * 2 + 8;   // dwords per channel octet in the key staging, padded


template <int D, int G>
struct Cfg {
  static constexpr int VG = D / kGroup;        // value scale groups per token
  static constexpr int KCM = D / 32;           // key K-chunks of 32 union slots (max)
  static constexpr int OCT = D / 8;            // channel octets
  static constexpr int NTT = D / 16;           // value N-tiles of 16 channels
  static constexpr int KQ = D / 8;             // union-slot octets per head
  static constexpr int AREP = (KQ * G + 63) / 64;
  static constexpr int NGB = G <= 4 ? 2 : 1;   // key groups whose A operands are built together
  static constexpr int HS = (G + 3) / 4;       // head sets of the compact numerator build
  static constexpr int VWR = D / 64;           // 16-byte value chunks per lane per tile
  static constexpr int KEY_A = NGB * KCM * 4 * (2 * G) * 4;   // rows 2h (high), 2h+1 (low)
  static constexpr int VAL_A = 2 * VG * 4 * G * 4;
  static constexpr int ABUF = KEY_A > VAL_A ? KEY_A : VAL_A;   // dwords
};

template <int D, int G>
struct __attribute__((aligned(16))) WaveSmem {
  union {
    struct {
      uint32_t y[D / 8][kYRow];        // key codes: channel octet, (token quad, 4 ch + 4 ch), padded
      float ksig[2][D];                // key scales of the tile's two groups, U order
      float ch0[kTok];                 // channel-0 keys
      uint32_t vw[kTok / 16][D + 16];  // value code words (rows padded against bank conflicts)
      float vsig[D / kGroup][kTok];    // value scales, by value group
    } st;
    float merge[G][D];                 // this wavefront's output at the end of the split
  } u;
  float z[G][kTok + 1];                // logits, then numerators, of the tile (padded rows)
  uint32_t abuf[Cfg<D, G>::ABUF];      // MFMA A operands (compact build, MFMA-layout reads)
  float mstate[G], lstate[G];
};

template <int D, int G>
struct __attribute__((aligned(16))) Smem {
  WaveSmem<D, G> w[kWaves];
  float coefc[G][D];                   // q' * sm * log2(e) by channel (0 if dropped)
  float coefs[G][D];                   // coefc in U order * 2^-E_h (0 past |U|)
  float e8[G];                         // 8 * 2^E_h
  float redm[G][kWaves];
  int hmask[D];
  int16_t ulist[D];
  int wcount[2];
};

template <int D, int G>
__global__ __launch_bounds__(kThreads, 2) void decode_kernel(dqk_cache c,
                                                             const float *__restrict__ qp,
                                                             const int32_t *__restrict__ sel,
                                                             int shared, int hq, int keep, float scale2,
                                                             int split, int nsplit,
                                                             float *__restrict__ ws,
                                                             float *__restrict__ out) {
  using K = Cfg<D, G>;
  __shared__ Smem<D, G> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, kg = lane >> 4;
  // Split-major order: the short last split of every sequence is launched last.
  const int units = c.batch * c.num_kv_heads;
  const int unit = blockIdx.x % units, s = blockIdx.x / units;
  const int item = unit * nsplit + s;
  const int b = unit / c.num_kv_heads, g = unit % c.num_kv_heads;
  const int len = max(0, min(c.lengths[b], c.capacity));
  const int t_begin = s * split;
  const int t_end = min(t_begin + split, len);
  float *wsp = ws + (size_t)item * G * (D + kPartialHead);
  // out != nullptr: a single split per row, whose normalized output is written
  // directly (what the combine makes of one partial); an empty row gives zeros
  float *outp = out ? out + ((size_t)b * hq + (size_t)g * G) * D : nullptr;
  if (t_begin >= t_end) {
    if (outp) {
      for (int e = tid; e < G * D; e += kThreads) outp[e] = 0.0f;
    } else {
      for (int e = tid; e < G * (D + kPartialHead); e += kThreads)
        wsp[e] = (e % (D + kPartialHead) == 0) ? -INFINITY : 0.0f;
    }
    return;
  }

  const size_t kc_stride = (size_t)(c.capacity / 4);
  const size_t ks_stride = (size_t)(c.capacity / kGroup);
  const uint8_t *kcodes = c.k_codes + unit * (size_t)D * kc_stride;
  const uint16_t *kscales = c.k_scales + unit * (size_t)D * ks_stride;
  const uint16_t *c0row = c.k_ch0 + unit * (size_t)c.capacity;
  const float *tail = c.k_tail + unit * (size_t)kGroup * D;
  const uint32_t *vwords = c.v_codes + unit * (size_t)(c.capacity / 16) * D;
  const uint16_t *vscales = c.v_scales + unit * (size_t)c.capacity * K::VG;
  const int t_body = (len / kGroup) * kGroup;
  const int code_end = min(t_body, t_end);

  // ---------------------------------------------------------------- setup (whole workgroup)
  for (int e = tid; e < G * D; e += kThreads) sm.coefc[e / D][e % D] = 0.0f;
  for (int e = tid; e < D; e += kThreads) sm.hmask[e] = 0;
  __syncthreads();
  const size_t row0 = (size_t)b * hq + (size_t)g * G;
  for (int e = tid; e < G * keep; e += kThreads) {
    const int h = e / keep;
    // the head's kept set: its own row, or its KV head's shared one
    const int ch = sel[(shared ? (size_t)unit : row0 + h) * keep + e % keep];
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
#pragma unroll
    for (int h = 0; h < G; ++h) {   // largest |coefficient| of each head over channels >= 1
      const float v = (tid >= 1 && tid < D) ? fabsf(sm.coefc[h][tid]) : 0.0f;
      const float mx = wave_max(v);
      if (lane == 0) sm.redm[h][wave] = mx;
    }
    __syncthreads();
    if (f) sm.ulist[__popcll(m & ((1ull << lane) - 1ull)) + (wave == 1 ? sm.wcount[0] : 0)] = (int16_t)tid;
  }
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
  __syncthreads();

  // ---------------------------------------------------------------- per-wavefront state
  WaveSmem<D, G> &W = sm.w[wave];
  float myc[K::AREP][8];   // my share of the key A build: (head, 8 union slots)
#pragma unroll
  for (int rep = 0; rep < K::AREP; ++rep) {
    const int it = lane + 64 * rep;
#pragma unroll
    for (int i = 0; i < 8; ++i) myc[rep][i] = it < K::KQ * G ? sm.coefs[it / K::KQ][8 * (it % K::KQ) + i] : 0.0f;
  }
  // my staging share: key code rows of channel octet lane/4, scale rows of channels lane, lane+64
  const int so = lane >> 2, swb = lane & 3;

  const int nv = t_end - t_begin;
  const int ntiles = (nv + kTok - 1) / kTok;

  // prefetch registers
  uint32_t px[8];
  uint16_t pks[2][2];
  uint16_t pc0;
  u32x4 pvw[K::VWR];
  uint16_t pvs[K::VG];

  // Loads of the next tile: addresses are clamped to the unit's first element when
  // the data is absent, and the value is replaced by zero (no branches).
  auto issue = [&](int tk) {
    const int p0 = t_begin + kTok * tk;
    const int tok = p0 + 16 * swb;
    const bool tok_ok = tok < code_end;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const int i = 8 * so + cc;
      const bool ok = so < K::OCT && i < nu && tok_ok;
      const size_t off = ok ? (size_t)sm.ulist[i] * kc_stride + (tok >> 2) : 0;
      const uint32_t x = *reinterpret_cast<const uint32_t *>(kcodes + off);
      px[cc] = ok ? x : 0u;
    }
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int i = lane + 64 * cc;
      const bool ok = i < nu;
      const size_t row = ok ? (size_t)sm.ulist[i] * ks_stride : 0;
#pragma unroll
      for (int gq = 0; gq < 2; ++gq) {
        const int grp = p0 / kGroup + gq;
        const bool okg = ok && grp * kGroup < code_end;
        const uint16_t x = kscales[okg ? row + grp : 0];
        pks[cc][gq] = okg ? x : (uint16_t)0;
      }
    }
    {
      const bool ok = p0 + lane < t_end;
      const uint16_t x = c0row[ok ? p0 + lane : 0];
      pc0 = ok ? x : (uint16_t)0;
    }
#pragma unroll
    for (int r = 0; r < K::VWR; ++r) {
      const int e = lane + 64 * r;
      const int blk = e / (D / 4), c4 = e % (D / 4);
      const int tokb = p0 + 16 * blk;
      const bool ok = tokb < t_end;
      const u32x4 x = *reinterpret_cast<const u32x4 *>(vwords + (ok ? (size_t)(tokb >> 4) * D + 4 * c4 : 0));
      pvw[r] = ok ? x : u32x4{0u, 0u, 0u, 0u};
    }
    {
      const bool ok = p0 + lane < t_end;
      const size_t base = ok ? (size_t)(p0 + lane) * K::VG : 0;
#pragma unroll
      for (int j = 0; j < K::VG; ++j) {
        const uint16_t x = vscales[base + j];
        pvs[j] = ok ? x : (uint16_t)0;
      }
    }
  };

  auto commit = [&]() {
    if (so < K::OCT) {
      uint32_t y0[4], y1[4];
      {
        const uint32_t a = __builtin_amdgcn_perm(px[0], px[2], 0x05010400u);
        const uint32_t bb = __builtin_amdgcn_perm(px[1], px[3], 0x05010400u);
        const uint32_t a2 = __builtin_amdgcn_perm(px[0], px[2], 0x07030602u);
        const uint32_t b2 = __builtin_amdgcn_perm(px[1], px[3], 0x07030602u);
        y0[0] = __builtin_amdgcn_perm(bb, a, 0x05040100u);
        y0[1] = __builtin_amdgcn_perm(bb, a, 0x07060302u);
        y0[2] = __builtin_amdgcn_perm(b2, a2, 0x05040100u);
        y0[3] = __builtin_amdgcn_perm(b2, a2, 0x07060302u);
      }
      {
        const uint32_t a = __builtin_amdgcn_perm(px[4], px[6], 0x05010400u);
        const uint32_t bb = __builtin_amdgcn_perm(px[5], px[7], 0x05010400u);
        const uint32_t a2 = __builtin_amdgcn_perm(px[4], px[6], 0x07030602u);
        const uint32_t b2 = __builtin_amdgcn_perm(px[5], px[7], 0x07030602u);
        y1[0] = __builtin_amdgcn_perm(bb, a, 0x05040100u);
        y1[1] = __builtin_amdgcn_perm(bb, a, 0x07060302u);
        y1[2] = __builtin_amdgcn_perm(b2, a2, 0x05040100u);
        y1[3] = __builtin_amdgcn_perm(b2, a2, 0x07060302u);
      }
      u32x4 *dst = reinterpret_cast<u32x4 *>(&W.u.st.y[so][8 * swb]);
      dst[0] = u32x4{y0[0], y1[0], y0[1], y1[1]};
      dst[1] = u32x4{y0[2], y1[2], y0[3], y1[3]};
    }
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int i = lane + 64 * cc;
      if (i < D) {
        W.u.st.ksig[0][i] = f16_value(pks[cc][0]);
        W.u.st.ksig[1][i] = f16_value(pks[cc][1]);
      }
    }
    W.u.st.ch0[lane] = f16_value(pc0);
#pragma unroll
    for (int r = 0; r < K::VWR; ++r) {
      const int e = lane + 64 * r;
      const int blk = e / (D / 4), c4 = e % (D / 4);
      *reinterpret_cast<u32x4 *>(&W.u.st.vw[blk][4 * c4]) = pvw[r];
    }
#pragma unroll
    for (int j = 0; j < K::VG; ++j) W.u.st.vsig[j][lane] = f16_value(pvs[j]);
  };

  float m_run[G], l_run[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.0f;
  }
  bool f_set = false;
  int f_run = 0;
  f32x4 vacc[K::NTT];
#pragma unroll
  for (int nt = 0; nt < K::NTT; ++nt) vacc[nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float spart[K::HS][K::VG];   // sum of the fp16 numerators per (head, value group)
#pragma unroll
  for (int hs = 0; hs < K::HS; ++hs)
#pragma unroll
    for (int j = 0; j < K::VG; ++j) spart[hs][j] = 0.0f;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  const u32x4 ones = {kOne2, kOne2, kOne2, kOne2};
  const uint32_t vmask = in_vgpr(kCode2), vone = in_vgpr(kOne2);

  if (wave < ntiles) {
    issue(wave);
    commit();
  }
  wave_sync();

  for (int tk = wave; tk < ntiles; tk += kWaves) {
    const int tile0 = t_begin + kTok * tk;
    const bool more = tk + kWaves < ntiles;
    if (more) issue(tk + kWaves);   // in flight during this tile's compute

    // ---- logits of the tile's two key groups
#pragma unroll
    for (int gb = 0; gb < 2 / K::NGB; ++gb) {
#pragma unroll
      for (int q = 0; q < K::NGB; ++q) {
        const int gq = gb * K::NGB + q;
        if (tile0 + kGroup * gq < t_end) {
#pragma unroll
          for (int rep = 0; rep < K::AREP; ++rep) {
            const int it = lane + 64 * rep;
            if (it < K::KQ * G) {
              const int h = it / K::KQ, kq = it % K::KQ;
              const float *sg = &W.u.st.ksig[gq][8 * kq];
              uint32_t hi[4], lo[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float a0 = myc[rep][2 * i] * sg[2 * i];
                const float a1 = myc[rep][2 * i + 1] * sg[2 * i + 1];
                hi[i] = f16_pair(a0, a1);
                lo[i] = f16_pair(a0 - f16_low(hi[i]), a1 - f16_high(hi[i]));
              }
              const int base = ((q * K::KCM + (kq >> 2)) * 4 + (kq & 3)) * (2 * G);
              *reinterpret_cast<u32x4 *>(&W.abuf[4 * (base + 2 * h)]) = u32x4{hi[0], hi[1], hi[2], hi[3]};
              *reinterpret_cast<u32x4 *>(&W.abuf[4 * (base + 2 * h + 1)]) = u32x4{lo[0], lo[1], lo[2], lo[3]};
            }
          }
        }
      }
      wave_sync();
#pragma unroll
      for (int q = 0; q < K::NGB; ++q) {
        const int gq = gb * K::NGB + q;
        if (tile0 + kGroup * gq >= t_end) {   // wavefront-uniform: group past the split end
          for (int e = lane; e < G * kGroup; e += 64) W.z[e / kGroup][kGroup * gq + e % kGroup] = -INFINITY;
          continue;
        }
        f32x4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = acc0, accs = acc0;
        const int r2 = 2 * (n16 & 3);
        for (int kc = 0; kc < nkc; ++kc) {
          const u32x4 A = n16 < 2 * G
                              ? *reinterpret_cast<const u32x4 *>(&W.abuf[4 * (((q * K::KCM + kc) * 4 + kg) * (2 * G) + n16)])
                              : zero4;
          const uint32_t *y = &W.u.st.y[4 * kc + kg][2 * (8 * gq + (n16 >> 2))];
          const uint32_t y00 = y[0], y01 = y[1], y10 = y[8], y11 = y[9];
          const u32x4 b0 = {((y00 >> r2) & vmask) | vone, ((y00 << (8 - r2)) & vmask) | vone,
                            ((y01 >> r2) & vmask) | vone, ((y01 << (8 - r2)) & vmask) | vone};
          const u32x4 b1 = {((y10 >> r2) & vmask) | vone, ((y10 << (8 - r2)) & vmask) | vone,
                            ((y11 >> r2) & vmask) | vone, ((y11 << (8 - r2)) & vmask) | vone};
          acc0 = mfma16(A, b0, acc0);
          acc1 = mfma16(A, b1, acc1);
          accs = mfma16(A, ones, accs);
        }
        // C rows 4kg..4kg+3 = (high, low) of heads 2kg and 2kg+1: the sum stays in the lane
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const f32x4 acc = nt == 0 ? acc0 : acc1;
          const int tokl = kGroup * gq + 16 * nt + n16;   // token within the tile
          const int t = tile0 + tokl;
          const float x0 = W.u.st.ch0[tokl];
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int h = 2 * kg + i;
            if (h < G) {
              const float v = (acc[2 * i] + acc[2 * i + 1]) - 1.375f * (accs[2 * i] + accs[2 * i + 1]);
              const float zz = fmaf(sm.e8[h], v, sm.coefc[h][0] * x0);
              W.z[h][tokl] = t < t_end ? zz : -INFINITY;
            }
          }
        }
      }
      wave_sync();
    }

    // ---- tokens of the unfinished last group: exact fp32 tail keys
    if (tile0 + kTok > t_body && t_body < t_end) {
      const int ta = max(tile0, t_body), tb = min(tile0 + kTok, t_end);
      const int nt = tb - ta;
      for (int e = lane; e < G * nt; e += 64) {
        const int h = e / nt, t = ta + e % nt;
        float zz = sm.coefc[h][0] * f16_value(c0row[t]);
        for (int i = 0; i < nu; ++i) {
          const int ch = sm.ulist[i];
          zz = fmaf(sm.coefc[h][ch], tail[(size_t)(t & 31) * D + ch], zz);
        }
        W.z[h][t - tile0] = zz;
      }
      wave_sync();
    }

    // ---- online softmax over the tile (lane = token)
    float ra[4];            // factor of C row 4kg+i (head of that row)
    float rs[K::HS];        // factor of head 4hs+kg (compact numerator sums)
    bool moved = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = 1.0f;
#pragma unroll
    for (int hs = 0; hs < K::HS; ++hs) rs[hs] = 1.0f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float zv = W.z[h][lane];
      const float m_new = fmaxf(m_run[h], wave_max(zv));
      const float al = exp2f(m_run[h] - m_new);
      const float p = exp2f(zv - m_new);
      l_run[h] = fmaf(l_run[h], al, wave_sum(p));
      m_run[h] = m_new;
      W.z[h][lane] = p;
      moved = moved || al != 1.0f;
      if (h < 4) ra[h] = al;
      else ra[h - 4] = (kg & 1) ? al : ra[h - 4];
      rs[h >> 2] = ((h & 3) == kg) ? al : rs[h >> 2];
    }
    // value scale exponent: 2^f * (largest value scale seen) < 2^15
    float vmx = 0.0f;
#pragma unroll
    for (int j = 0; j < K::VG; ++j) vmx = fmaxf(vmx, W.u.st.vsig[j][lane]);
    vmx = wave_max(vmx);
    int fe = 0;
    if (vmx > 0.0f) frexpf(vmx, &fe);
    const int f_tile = 15 - fe;
    const int f_new = f_set ? min(f_run, f_tile) : f_tile;
    const float factor = f_set ? ldexpf(1.0f, f_new - f_run) : 1.0f;
    f_run = f_new;
    f_set = true;
    const float fs = ldexpf(1.0f, f_new);
    // rescale the running sums only when a head's max or the exponent moved (uniform test)
    if (moved || factor != 1.0f) {
#pragma unroll
      for (int nt = 0; nt < K::NTT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) vacc[nt][i] *= ra[i] * factor;
#pragma unroll
      for (int hs = 0; hs < K::HS; ++hs)
#pragma unroll
        for (int j = 0; j < K::VG; ++j) spart[hs][j] *= rs[hs] * factor;
    }
    wave_sync();

    // ---- compact numerators p * s * 2^f -> A operands (row = head, K = token)
#pragma unroll
    for (int hs = 0; hs < K::HS; ++hs) {
      const int h = 4 * hs + kg;
      if (h < G) {
        const int kgx = n16 >> 2, ii = n16 & 3;
        const int r0 = 2 * (kgx & 1), d = ii & 1;
        const int tl = 16 * (kgx >> 1) + (ii < 2 ? 4 + r0 + d : r0 + d);
#pragma unroll
        for (int kc2 = 0; kc2 < 2; ++kc2) {
          const int t0 = 32 * kc2 + tl;
          const float p0 = W.z[h][t0], p1 = W.z[h][t0 + 8];
#pragma unroll
          for (int j = 0; j < K::VG; ++j) {
            const uint32_t pk = f16_pair(p0 * (W.u.st.vsig[j][t0] * fs), p1 * (W.u.st.vsig[j][t0 + 8] * fs));
            spart[hs][j] += f16_low(pk) + f16_high(pk);
            W.abuf[4 * ((((kc2 * K::VG + j) * 4 + kgx) * G) + h) + ii] = pk;
          }
        }
      }
    }
    wave_sync();

    // ---- weighted sum of the value codes
#pragma unroll
    for (int kc2 = 0; kc2 < 2; ++kc2) {
      const int blk = 2 * kc2 + (kg >> 1);
      const int r0 = 2 * (kg & 1);
#pragma unroll
      for (int j = 0; j < K::VG; ++j) {
        const u32x4 A = n16 < G ? *reinterpret_cast<const u32x4 *>(&W.abuf[4 * (((kc2 * K::VG + j) * 4 + kg) * G + n16)])
                                : zero4;
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          const int ch = 32 * j + 16 * t2 + n16;
          const uint32_t w = W.u.st.vw[blk][ch];
          const u32x4 bv = {((w >> (2 * r0)) & vmask) | vone, ((w >> (2 * r0 + 2)) & vmask) | vone,
                            ((w << (8 - 2 * r0)) & vmask) | vone, ((w << (6 - 2 * r0)) & vmask) | vone};
          vacc[2 * j + t2] = mfma16(A, bv, vacc[2 * j + t2]);
        }
      }
    }
    wave_sync();
    if (more) commit();
    wave_sync();
  }

  // ---------------------------------------------------------------- merge the wavefronts
  {
    float ssum[K::HS][K::VG];
#pragma unroll
    for (int hs = 0; hs < K::HS; ++hs)
#pragma unroll
      for (int j = 0; j < K::VG; ++j) ssum[hs][j] = row16_sum(spart[hs][j]);
    const float inv_f = f_set ? ldexpf(1.0f, -f_run) : 0.0f;
#pragma unroll
    for (int nt = 0; nt < K::NTT; ++nt) {
      const int ch = 16 * nt + n16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 4 * kg + i;
        const int hh = h < G ? h : 0;
        float sh = 0.0f;
#pragma unroll
        for (int hs = 0; hs < K::HS; ++hs) {
          const float x = __shfl(ssum[hs][nt / 2], 16 * (hh & 3), 64);   // value group of channel 16nt..
          if (hs == hh / 4) sh = x;
        }
        if (h < G) W.u.merge[h][ch] = (8.0f * vacc[nt][i] - 11.0f * sh) * inv_f;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
      if (lane == h) {
        W.mstate[h] = m_run[h];
        W.lstate[h] = l_run[h];
      }
  }
  __syncthreads();
  // Straight-line: every LDS read of an element is issued before any is used, and
  // a wavefront without tokens is dropped by selects, not branches.
  for (int e = tid; e < G * D; e += kThreads) {
    const int h = e / D, ch = e % D;
    float lw[kWaves], mw[kWaves], ow[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      lw[w] = sm.w[w].lstate[h];
      mw[w] = sm.w[w].mstate[h];
      ow[w] = sm.w[w].u.merge[h][ch];
    }
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = lw[w] > 0.0f ? fmaxf(M, mw[w]) : M;
    float o = 0.0f, L = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const bool live = lw[w] > 0.0f;
      const float f = exp2f((live ? mw[w] : M) - M);
      o = live ? fmaf(ow[w], f, o) : o;
      L = live ? fmaf(lw[w], f, L) : L;
    }
    if (outp) {
      const float inv = L > 0.0f ? 1.0f / L : 0.0f;
      outp[h * D + ch] = o * inv;
    } else {
      wsp[h * (D + kPartialHead) + kPartialHead + ch] = o;
      if (ch == 0) {
        wsp[h * (D + kPartialHead) + 0] = M;
        wsp[h * (D + kPartialHead) + 1] = L;
      }
    }
  }
}

template <int D, int G>
hipError_t launch_decode_t(const dqk_cache &c, const float *qp, const int32_t *sel, int shared, int hq,
                           int keep, float scale2, int split, float *out, float *ws,
                           hipStream_t s) {
  const int nsplit = num_splits(c.capacity, split);
  const int items = c.batch * c.num_kv_heads * nsplit;
  // one split per row: the kernel writes the output itself and no combine runs
  hipLaunchKernelGGL((decode_kernel<D, G>), dim3((unsigned)items), dim3(kThreads), 0, s, c, qp,
                     sel, shared, hq, keep, scale2, split, nsplit, ws, nsplit == 1 ? out : nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  return launch_combine(ws, c.batch, hq, c.num_kv_heads, D, nsplit, out, s);
}

template <int D>
hipError_t launch_decode_d(const dqk_cache &c, const float *qp, const int32_t *sel, int shared, int hq,
                           int keep, float scale2, int split, bool even, float *out, float *ws,
                           hipStream_t s) {
  switch (hq / c.num_kv_heads) {
    case 1: return launch_decode_t<D, 1>(c, qp, sel, shared, hq, keep, scale2, split, out, ws, s);
    case 2: return launch_decode_t<D, 2>(c, qp, sel, shared, hq, keep, scale2, split, out, ws, s);
    case 4:
    case 8: {
      // the matrix-core decodes (one workgroup for the four or eight heads of a KV
      // head) need a capacity that is a multiple of 64 tokens
      const bool eight = hq == 8 * c.num_kv_heads;
      if (!(eight ? decode8_supported(c, hq) : decode4_supported(c, hq)))
        return eight ? launch_decode_t<D, 8>(c, qp, sel, shared, hq, keep, scale2, split, out, ws, s)
                     : launch_decode_t<D, 4>(c, qp, sel, shared, hq, keep, scale2, split, out, ws, s);
      const int nsplit = num_splits(c.capacity, split);
      // one split per row: the kernel writes the output itself and no combine runs
      float *o = nsplit == 1 ? out : nullptr;
      const hipError_t e = eight ? launch_decode8(c, qp, sel, shared != 0, hq, keep, scale2, split, even, ws, o, s)
                                 : launch_decode4(c, qp, sel, shared != 0, hq, keep, scale2, split, even, ws, o, s);
      if (e != hipSuccess || nsplit == 1) return e;
      return launch_combine(ws, c.batch, hq, c.num_kv_heads, D, nsplit, out, s);
    }
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const dqk_cache &c, const float *q_prime, const int32_t *sel_idx,
                         bool shared, int hq, int keep, float sm_scale, int split, bool even,
                         float *out, float *ws, hipStream_t s) {
  const float scale2 = sm_scale * 1.4426950408889634f;  // logits in log2 units
  if (c.head_dim == 64)
    return launch_decode_d<64>(c, q_prime, sel_idx, shared ? 1 : 0, hq, keep, scale2, split, even, out, ws, s);
  return launch_decode_d<128>(c, q_prime, sel_idx, shared ? 1 : 0, hq, keep, scale2, split, even, out, ws, s);
}

}  // namespace dqk
