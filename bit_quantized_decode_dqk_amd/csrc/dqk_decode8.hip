// Decode attention over the 2-bit cache for GQA groups of eight query heads
// (hq / hkv == 8), with per-head or group-shared kept sets: one workgroup serves
// all eight heads of a KV head, so each key and value byte is read once and each
// 2-bit code is turned into a matrix-core operand once for the eight heads.
//
// Dual-QK (arXiv abstract; tech.dede.sh summary, "Throughput on SGLang"): keys
// and values are stored in 2 bits and the key channels no head of the group
// keeps are never read.  The operand encodings are those of the four-head
// kernel (dqk_decode4.hip): a 2-bit code masked in place in an fp16 word with a
// zero exponent is the exact subnormal u * 2^(2k-24), shifted to mantissa bits
// 6-9 for the logits; logit weights are split into fp16 high and low parts; the
// numerators times the value scales are single fp16 values; accumulation is fp32.
// What changes is the shape of the work:
//  - a block is 128 tokens, and wavefront w takes the block's key group w
//    (32 tokens).  The logit product of one K chunk has rows (head h, part) for
//    all eight heads and K = 32 union slots of that one group, so that no K
//    position of the product is zero; B holds the group's codes, shared by the
//    eight heads;
//  - the weighted sum runs the four-head product twice per operand, once for
//    heads 0-3 and once for heads 4-7, on the same value-code operands.
// Per chunk of up to ten blocks: pass 1 commits each block's codes and logit
// A operands to LDS (two buffers, loads two blocks ahead, one barrier per
// block) and keeps the logits in registers; pass 2 streams each wavefront's
// value tiles (three in flight) once the chunk's maxima are known.  The
// workgroup leaves its partial (m, l, o) per head for the combine, or, with a
// single split per row, the normalized output.
//
// The capacity must be a multiple of 64 tokens (whole dwords of every key-scale
// row); other shapes use the other decode kernels.
#include "dqk_decode_ops.h"

namespace dqk {
namespace {

using namespace wave;
using namespace dops;

constexpr int kG8 = 8;               // query heads per workgroup: the whole group
constexpr int kThreads8 = 256;
constexpr int kWaves8 = kThreads8 / 64;
constexpr int kTile8 = kGroup;       // tokens per wavefront tile: one key group
constexpr int kBlock8 = kTile8 * kWaves8;   // tokens per workgroup block
constexpr int kChunk8 = kDecodeChunkBlocks; // blocks per chunk: logits of a chunk stay in registers
// one block more than a chunk runs as one chunk: the extra block is committed to
// LDS buffer kChunk8 & 1 and its values use stage kChunk8 % 3

template <int D>
struct Lay8 {
  static constexpr int OCT = D / 8;     // union-slot octets
  static constexpr int NKC = D / 32;    // logit K chunks: four octets (32 slots) of the tile's group
  static constexpr int VG = D / 32;     // value scale groups
  static constexpr int AROW = D + 8;    // fp16 per logit A row (padded against bank conflicts)
  static constexpr int SPJ = D / 2;     // logit A jobs per tile: union-slot pairs
  static constexpr int NH = D / 64;     // 64-channel halves of the weighted sum
  static constexpr int CJ = OCT * (kBlock8 / 16);   // key-code jobs: slot octet x 16-token group
};

// The keys of one 128-token block as staged in LDS.
template <int D>
struct __attribute__((aligned(16))) KBlock8 {
  uint32_t y[kWaves8][Lay8<D>::OCT][kTile8 / 4][2];   // key codes: tile, slot octet, token quad, slots 0-3 | 4-7
  // logit A operands of tile w: rows 2h + part (head h, fp16 high/low part),
  // slots in octet order 0,2,1,3,4,6,5,7; the tiles are 8 dwords apart modulo
  // the 32 LDS banks
  struct {
    uint16_t r[2 * kG8][Lay8<D>::AROW];
    uint16_t pad[16];
  } a[kWaves8];
  uint32_t c0w[kBlock8 / 2];   // key channel 0: fp16 pair of tokens 2i, 2i+1
};

template <int D>
struct __attribute__((aligned(16))) WaveSmem8 {
  u32x4 zero;   // a 16-byte zero operand
  union {
    struct {
      // value A: group j, K chunk kc, then word row w, head h, 8 K positions at
      // ((w * 8 + h) * 8 + k), padded by 4 dwords per (j, kc) slab
      uint16_t pbuf[Lay8<D>::VG][2][2 * kG8 * 8 + 8];
    } t;
    float merge[kG8][D];   // the wavefront's output at the end of the split
  } u;
  float mstate[kG8], lstate[kG8];
};

template <int D>
struct __attribute__((aligned(16))) Smem8 {
  KBlock8<D> kb[2];
  WaveSmem8<D> w[kWaves8];
  float coefc[kG8][D];   // q' * sm * log2(e) by channel (0 where the head drops the channel)
  float coefs[kG8][D];   // coefc in union-slot order * 2^-E_h (0 past |U|)
  float e2[kG8];         // 2^E_h
  float redm[kG8][2];    // largest |coefficient| per head and 64-channel half
  float tailz[kG8][kGroup];   // exact logits of the unfinished last key group
  union {
    uint8_t b[kG8][D];   // kept[h][c]: head h keeps channel c
    uint32_t w[kG8 * D / 4];
  } kept;
  unsigned long long umask[2];   // the union U of kept key channels >= 1
  int32_t ulist[D];              // compact slots: key channel of slot i (-1 past |U|)
};

// Registers of one block of keys in flight.
struct KStage8 {
  uint32_t kc[8];   // key codes: 8 slots x 16 tokens
  uint32_t ks[2];   // key scales of two slots, the job's key group (fp16 in the low half)
  uint32_t c0;      // channel 0: two tokens
};

// Registers of one tile of values in flight (one wavefront).
template <int D>
struct VStage8 {
  uint32_t vw[Lay8<D>::NH][2];   // value words of channel 64 half + 16q + n, word rows 0-1 of the tile
  uint32_t vs[Lay8<D>::VG];      // value scales of tokens t, t+1: [t groups | t+1 groups]
};

// c ? b : a over four values selected by the two low bits of q (no indexed load).
__device__ __forceinline__ float sel4(int q, float a0, float a1, float a2, float a3) {
  return sel2((q & 2) != 0, sel2((q & 1) != 0, a0, a1), sel2((q & 1) != 0, a2, a3));
}

// COMPACT (group-shared kept sets, one per KV head): union slot i holds the
// i-th kept key channel other than 0, and only the nkc K chunks that hold the
// keep - 1 such channels are worked on; otherwise slot i holds channel i + 1 and
// all K chunks run.
template <int D, bool COMPACT>
__global__ __launch_bounds__(kThreads8, 2) void decode8_kernel(dqk_cache c,
                                                               const float *__restrict__ qp,
                                                               const int32_t *__restrict__ sel,
                                                               int hq, int grid3, int keep, float scale2,
                                                               int nsplit, int bps, int ncu_q, int ncu_r,
                                                               int nkc, float *__restrict__ ws,
                                                               float *__restrict__ out) {
  using L = Lay8<D>;
  constexpr int G = kG8;
  __shared__ Smem8<D> sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Work item (unit, split s) in split-major order, as in the four-head kernel:
  // the grid is (KV head, row, split) where it fits, else one-dimensional.
  const int units = c.batch * c.num_kv_heads;
  int b, g, s;
  if (grid3) {
    g = blockIdx.x;
    b = blockIdx.y;
    s = blockIdx.z;
  } else {
    const int item = blockIdx.x;
    if (item >= units * nsplit) return;
    const int unit = item % units;
    s = item / units;
    b = unit / c.num_kv_heads;
    g = unit % c.num_kv_heads;
  }
  const int unit = b * c.num_kv_heads + g;
  const int len = max(0, min(c.lengths[b], c.capacity));
  // q' rows of the group and the kept lists, in flight with the length
  const size_t row0 = (size_t)b * hq + (size_t)g * G;
  constexpr int SJ = (G * D) / kThreads8;   // elements per lane
  float qv[SJ];
  int sv[SJ];
#pragma unroll
  for (int k = 0; k < SJ; ++k) {
    const int e = tid + kThreads8 * k;
    qv[k] = qp[row0 * D + e];
    // the head's kept set: its own row, or its KV head's shared one (position
    // e mod keep, by subtraction: e < G keep)
    if constexpr (COMPACT) {
      int es = e;
#pragma unroll
      for (int h = 1; h < G; ++h) es = es >= keep ? es - keep : es;
      sv[k] = e < G * keep ? sel[(size_t)unit * keep + es] : -1;
    } else {
      sv[k] = e < G * keep ? sel[row0 * keep + e] : -1;
    }
  }
  // compact slots: the shared kept list without channel 0, one slot per lane
  int uch = -1;
  if constexpr (COMPACT) {
    if (tid < D && tid + 1 < keep) uch = sel[(size_t)unit * keep + tid + 1];
  }
  const int nblk_all = (len + kBlock8 - 1) / kBlock8;
  // bps > 0: split s is blocks [s bps, (s + 1) bps).  Else the row's blocks are
  // shared out over the splits evenly, or unevenly when two workgroups share
  // each compute unit (uneven_shares).
  int blo, bhi;
  {
    const int fs = ncu_q + ncu_r > 0 ? min(nsplit, ncu_q + (unit < ncu_r ? 1 : 0)) : 0;
    if (bps > 0) {
      blo = min(s * bps, nblk_all);
      bhi = min(blo + bps, nblk_all);
    } else if (const SplitShares sh = uneven_shares(nblk_all, nsplit, fs, len % kGroup != 0 ? 1 : 0);
               sh.second >= 0) {
      const BlockRange r = uneven_split_range(sh, s, fs, nsplit, nblk_all);
      blo = r.lo;
      bhi = r.hi;
    } else if ((unsigned long long)nblk_all * (unsigned long long)nsplit < (1ull << 32)) {
      blo = (int)(((uint32_t)s * (uint32_t)nblk_all) / (uint32_t)nsplit);
      bhi = (int)(((uint32_t)(s + 1) * (uint32_t)nblk_all) / (uint32_t)nsplit);
    } else {
      blo = (int)(((long long)s * nblk_all) / nsplit);
      bhi = (int)(((long long)(s + 1) * nblk_all) / nsplit);
    }
  }
  const int t_begin = blo * kBlock8;
  const int t_end = min(bhi * kBlock8, len);
  const int nb = bhi - blo;
  float *wsp = ws + ((size_t)unit * nsplit + s) * G * (D + kPartialHead);
  float *outp = out ? out + row0 * D : nullptr;
  if (t_begin >= t_end) {
    if (outp) {
      for (int e = tid; e < G * D; e += kThreads8) outp[e] = 0.0f;
    } else {
      for (int e = tid; e < G * (D + kPartialHead); e += kThreads8)
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
  const uint16_t *vscales = c.v_scales + unit * (size_t)c.capacity * L::VG;
  const int t_body = (len / kGroup) * kGroup;
  const int code_end = min(t_body, t_end);

  // buffer resources moved to the block or tile; an offset past the resource
  // returns zero (kFar), a block past the end gets an empty resource
  const uint32_t kc_bytes = (uint32_t)(D * kc_stride), ks_bytes = (uint32_t)(D * ks_stride * 2);
  const uint32_t c0_bytes = (uint32_t)(c.capacity * 2), vw_bytes = (uint32_t)((c.capacity / 16) * D * 4);
  const uint32_t vs_bytes = (uint32_t)(c.capacity * L::VG * 2);
  auto rsrc = [&](const void *base, uint32_t bytes, uint32_t off, bool live) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)((const char *)base + (live ? off : 0u)), (short)0,
                                             live ? (int)(bytes - off) : 0, kRsrcWord3);
  };

  // rows of the unfinished last key group (only where the split reaches it)
  const bool has_tail = t_body < t_end;
  constexpr int TJ = kGroup * D / (4 * kThreads8);   // float4 per lane
  f32x4 tv[TJ];
  {
    const auto rt = rsrc(tail, (uint32_t)(kGroup * D * 4), 0u, has_tail);
#pragma unroll
    for (int k = 0; k < TJ; ++k)
      tv[k] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rt, 16u * (tid + kThreads8 * k), 0, 0));
  }

  // ---------------------------------------------------------------- key loads (every lane)
  // Union slot i holds key channel i + 1 (the last slot is empty): the first
  // block is issued for every channel as soon as the length is known, later
  // blocks for the union only.  Compact slots hold the shared set's channels:
  // the first block is issued once the set is in LDS, for those channels only.
  auto mul_apart = [](uint32_t a, uint32_t b2) {
    uint32_t p = a * b2;
    asm volatile("" : "+v"(p));
    return p;
  };
  // key-code job: slot octet lo, 16-token group lq of the block (8 slots x 4
  // bytes); lanes past the jobs repeat the first ones (the same bytes to the
  // same place)
  const int cj = tid % L::CJ;
  const int lo = cj / (kBlock8 / 16), lq = cj % (kBlock8 / 16);
  const uint32_t kc_row = (uint32_t)kc_stride, ks_row = 2u * (uint32_t)ks_stride;
  // logit A job: tile at (= key group at of the block), union slots s0 = 8o + a,
  // s1 = s0 + 2 (a = 0, 1, 4, 5), side by side in the octet order of the A rows
  const int aj = tid % (kWaves8 * L::SPJ), at = aj & 3, asp = aj >> 2;
  const int aoct = asp >> 2, am = asp & 3;
  const int as0 = 8 * aoct + (am & 1) + 4 * (am >> 1), as1 = as0 + 2;
  auto slot_channel = [&](int i) -> int {
    if constexpr (COMPACT) return sm.ulist[i];
    else return i + 1 < D ? i + 1 : -1;
  };
  uint32_t kvo[8], ksv[2];
  auto job_offsets = [&]() {
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const int ch = slot_channel(8 * lo + cc);
      kvo[cc] = ch >= 0 ? mul_apart((uint32_t)ch, kc_row) + 4u * (uint32_t)lq : kFar;
    }
    const int c0a = slot_channel(as0), c1a = slot_channel(as1);
    ksv[0] = c0a >= 0 ? mul_apart((uint32_t)c0a, ks_row) + 2u * (uint32_t)at : kFar;
    ksv[1] = c1a >= 0 ? mul_apart((uint32_t)c1a, ks_row) + 2u * (uint32_t)at : kFar;
  };
  if constexpr (!COMPACT) job_offsets();
  const uint32_t c0o = tid < kBlock8 / 2 ? 4u * tid : kFar;

  auto kissue = [&](KStage8 &S, int p0, bool live) {
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t u0 = (uint32_t)p0;
    const auto rk = rsrc(kcodes, kc_bytes, u0 >> 2, live);
    const auto rks = rsrc(kscales, ks_bytes, (u0 / kGroup) * 2u, live);
    const auto rc0 = rsrc(c0row, c0_bytes, u0 * 2u, live);
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) S.kc[cc] = __builtin_amdgcn_raw_buffer_load_b32(rk, kvo[cc], 0, 0);
#pragma unroll
    for (int k = 0; k < 2; ++k) S.ks[k] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rks, ksv[k], 0, 0);
    S.c0 = __builtin_amdgcn_raw_buffer_load_b32(rc0, c0o, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  const int nbc0 = nb == kChunk8 + 1 ? kChunk8 + 1 : min(kChunk8, nb);
  KStage8 S0, S1;
  if constexpr (!COMPACT) kissue(S0, t_begin, 0 < nbc0);

  // ---------------------------------------------------------------- setup (whole workgroup)
  for (int e = tid; e < G * D / 4; e += kThreads8) sm.kept.w[e] = 0u;
  if constexpr (COMPACT) {
    if (tid < D) sm.ulist[tid] = uch >= 1 && uch < D ? uch : -1;
  }
  block_barrier();
  if constexpr (COMPACT) {   // the first block once the compact slots are known
    job_offsets();
    kissue(S0, t_begin, 0 < nbc0);
  }
#pragma unroll
  for (int k = 0; k < SJ; ++k) {
    const int e = tid + kThreads8 * k;
    if (e < G * keep && sv[k] >= 0 && sv[k] < D) sm.kept.b[e / keep][sv[k]] = 1;
  }
  block_barrier();
#pragma unroll
  for (int k = 0; k < SJ; ++k) {
    // head h and half of element e are the same for the whole wavefront
    const int e = tid + kThreads8 * k, h = e / D, ch = e % D;
    const float cv = sm.kept.b[h][ch] ? qv[k] * scale2 : 0.0f;
    sm.coefc[h][ch] = cv;
    const float mx = wave_max(ch >= 1 ? fabsf(cv) : 0.0f);
    if (lane == 0) sm.redm[h][ch / 64] = mx;
  }
  {
    bool f = false;
    if (tid >= 1 && tid < D) {
#pragma unroll
      for (int h = 0; h < G; ++h) f = f || sm.kept.b[h][tid] != 0;
    }
    const unsigned long long m = __ballot(f);
    if (lane == 0 && wave < 2) sm.umask[wave] = m;
  }
  // tail rows to LDS (the key block buffers are free until the first block)
  constexpr int TS = D + 4;
  static_assert(sizeof(sm.kb[0]) >= sizeof(float) * kGroup * TS, "tail rows fit a key block buffer");
  float *trow = reinterpret_cast<float *>(&sm.kb[0]);
  if (has_tail) {
#pragma unroll
    for (int k = 0; k < TJ; ++k) {
      const int e = 4 * (tid + kThreads8 * k);
      *reinterpret_cast<f32x4 *>(trow + (e / D) * TS + e % D) = tv[k];
    }
  }
  block_barrier();
  // exact logits of the unfinished last key group, one per (head, token)
  if (has_tail && tid < G * kGroup) {
    const int h = tid / kGroup, r = tid % kGroup, t = t_body + r;
    float zz = -INFINITY;
    if (t < t_end) {
      zz = sm.coefc[h][0] * f16_value(c0row[t]);
#pragma unroll
      for (int c4 = 0; c4 < D; c4 += 4) {
        const f32x4 cf = *reinterpret_cast<const f32x4 *>(&sm.coefc[h][c4]);
        const f32x4 x = *reinterpret_cast<const f32x4 *>(&trow[r * TS + c4]);
        if (c4 > 0) zz = fmaf(cf.x, x.x, zz);
        zz = fmaf(cf.y, x.y, zz);
        zz = fmaf(cf.z, x.z, zz);
        zz = fmaf(cf.w, x.w, zz);
      }
    }
    sm.tailz[h][r] = zz;
  }
  // coefficients in slot order, scaled by 2^-E_h
  for (int e = tid; e < G * D; e += kThreads8) {
    const int h = e / D, i = e % D;
    const float mx = D > 64 ? fmaxf(sm.redm[h][0], sm.redm[h][1]) : sm.redm[h][0];
    int ex = 0;
    if (mx > 0.0f) frexpf(mx, &ex);
    const int ch = slot_channel(i);
    sm.coefs[h][i] = ch >= 0 ? sm.coefc[h][ch] * ldexpf(1.0f, -ex) : 0.0f;
    if (i == 0) sm.e2[h] = ldexpf(1.0f, ex);
  }
  block_barrier();
  float ca[G], cb[G];   // coefficients of the job's two slots per head (0 outside U)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    ca[h] = sm.coefs[h][as0];
    cb[h] = sm.coefs[h][as1];
  }
  // key scales of the A-building slots outside U count as zero; later blocks
  // read the union's channels only
  uint32_t ksm[2];
  {
    const unsigned long long m0 = sm.umask[0], m1 = sm.umask[1];
    auto member = [&](int slot) {
      const int ch = slot_channel(slot);
      if (ch < 1) return false;
      return ((ch < 64 ? m0 >> ch : m1 >> (ch & 63)) & 1ull) != 0ull;
    };
#pragma unroll
    for (int cc = 0; cc < 8; ++cc)
      if (!member(8 * lo + cc)) kvo[cc] = kFar;
    ksm[0] = member(as0) ? 0xffffffffu : 0u;
    ksm[1] = member(as1) ? 0xffffffffu : 0u;
    if (!ksm[0]) ksv[0] = kFar;
    if (!ksm[1]) ksv[1] = kFar;
  }
  kissue(S1, t_begin + kBlock8, 1 < nbc0);

  auto kcommit = [&](KStage8 &S, KBlock8<D> &B, int p0) {
    {
      uint32_t y0[4], y1[4];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const uint32_t *x = S.kc + 4 * half;
        const uint32_t t0 = __builtin_amdgcn_perm(x[1], x[0], 0x05010400u);   // s0.b0 s1.b0 s0.b1 s1.b1
        const uint32_t t1 = __builtin_amdgcn_perm(x[3], x[2], 0x05010400u);   // s2.b0 s3.b0 s2.b1 s3.b1
        const uint32_t t2 = __builtin_amdgcn_perm(x[1], x[0], 0x07030602u);   // s0.b2 s1.b2 s0.b3 s1.b3
        const uint32_t t3 = __builtin_amdgcn_perm(x[3], x[2], 0x07030602u);
        uint32_t *yy = half ? y1 : y0;
        yy[0] = __builtin_amdgcn_perm(t1, t0, 0x05040100u);   // quad 0: s0 s1 s2 s3
        yy[1] = __builtin_amdgcn_perm(t1, t0, 0x07060302u);   // quad 1
        yy[2] = __builtin_amdgcn_perm(t3, t2, 0x05040100u);   // quad 2
        yy[3] = __builtin_amdgcn_perm(t3, t2, 0x07060302u);   // quad 3
      }
      u32x4 *dst = reinterpret_cast<u32x4 *>(&B.y[lq >> 1][lo][4 * (lq & 1)][0]);
      dst[0] = u32x4{y0[0], y1[0], y0[1], y1[1]};
      dst[1] = u32x4{y0[2], y1[2], y0[3], y1[3]};
    }
    // logit A operands of tile at: scales of a key group past the coded range
    // count as zero; high part = fp16 of the product, low part = fp16 of what the
    // high part leaves out
    uint32_t v = (S.ks[0] & 0xffffu & ksm[0]) | ((S.ks[1] << 16) & ksm[1]);
    if (p0 + kBlock8 > code_end) {   // workgroup-uniform
      if ((p0 / kGroup + at) * kGroup >= code_end) v = 0u;
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const uint32_t hi = mixhi<1>(mixlo<0>(ca[h], v), cb[h], v);
      const uint32_t lw = reshi<1, 1>(reslo<0, 0>(ca[h], v, hi), cb[h], v, hi);
      uint16_t (*ar)[L::AROW] = B.a[at].r;
      *reinterpret_cast<uint32_t *>(&ar[2 * h][8 * aoct + 2 * am]) = hi;
      *reinterpret_cast<uint32_t *>(&ar[2 * h + 1][8 * aoct + 2 * am]) = lw;
    }
    if (tid < kBlock8 / 2) B.c0w[tid] = S.c0;
  };

  // ---------------------------------------------------------------- per-wavefront state
  WaveSmem8<D> &W = sm.w[wave];
  const int q = lane >> 4, n = lane & 15;   // logit lanes: heads 2q, 2q + 1; tokens 2n, 2n + 1
  const uint32_t shl2 = (uint32_t)(6 - 4 * (n & 1)) * 0x00010001u;
  const uint32_t shr2 = (uint32_t)(2 + 4 * (n & 1)) * 0x00010001u;
  float ez[2][2], n3e[2], c0c[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int h = 2 * q + hh;
    const float e = sm.e2[h];
    n3e[hh] = -3.0f * e;
    c0c[hh] = sm.coefc[h][0];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) ez[hh][nt] = ldexpf(e, 25 - 2 * (3 + nt));
  }
  u32x4 ones = {kOneF16x2, kOneF16x2, kOneF16x2, kOneF16x2};

  // Logits (log2 units) of this wavefront's tile: z[hh][nt] for head 2q + hh and
  // token tile0 + 2n + nt; -inf past the end of the split.
  auto logits = [&](const KBlock8<D> &B, int tile0, float (&z)[2][2]) {
    f32x4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = acc0, accs = acc0;
    asm volatile("" : "+v"(ones));
#pragma unroll
    for (int kc = 0; kc < L::NKC; ++kc) {
      if constexpr (COMPACT) {
        if (kc >= nkc) break;   // wavefront-uniform
      }
      const u32x4 al = *reinterpret_cast<const u32x4 *>(&B.a[wave].r[n][8 * (4 * kc + q)]);
      const u32x2 dk = *reinterpret_cast<const u32x2 *>(&B.y[wave][4 * kc + q][n >> 1][0]);
      const uint32_t l0 = pk_shl16(dk.x, shl2), h0 = pk_shr16(dk.x, shr2);
      const uint32_t l1 = pk_shl16(dk.y, shl2), h1 = pk_shr16(dk.y, shr2);
      constexpr uint32_t M3 = 0x00C000C0u, M4 = 0x03000300u;
      const u32x4 b0 = {l0 & M3, h0 & M3, l1 & M3, h1 & M3};   // token 2n: u 2^-18
      const u32x4 b1 = {l0 & M4, h0 & M4, l1 & M4, h1 & M4};   // token 2n+1: u 2^-16
      acc0 = mfma16(al, b0, acc0);
      acc1 = mfma16(al, b1, acc1);
      accs = mfma16(al, ones, accs);
    }
    const uint32_t cx0 = B.c0w[kTile8 / 2 * wave + n];
    const float x0f[2] = {h2f(cx0 & 0xffffu), h2f(cx0 >> 16)};
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const float cs = accs[2 * hh] + accs[2 * hh + 1];
      const float bb = n3e[hh] * cs;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const f32x4 &a = nt == 0 ? acc0 : acc1;
        const float u = a[2 * hh] + a[2 * hh + 1];
        z[hh][nt] = fmaf(ez[hh][nt], u, fmaf(c0c[hh], x0f[nt], bb));
      }
    }
    const int tl0 = tile0 + 2 * n;
    if (tile0 + kTile8 > t_end) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        if (tl0 + nt >= t_end) z[0][nt] = z[1][nt] = -INFINITY;
    }
    if (tile0 + kTile8 > t_body && t_body < t_end) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int t = tl0 + nt;
        if (t >= t_body && t < t_end) {
          z[0][nt] = sm.tailz[2 * q][t - t_body];
          z[1][nt] = sm.tailz[2 * q + 1][t - t_body];
        }
      }
    }
  };

  // ---------------------------------------------------------------- value loads (per wavefront)
  // value A producer: my tokens are c = 2(n&7), c+1 of word row n >> 3
  const int pw = n >> 3, pkc = (n >> 1) & 1, pi0 = 4 * (n & 1) + ((n >> 2) & 1);
  const int pk[2] = {value_k(2 * (n & 3)), value_k(2 * (n & 3) + 1)};
  const uint32_t vwv = (uint32_t)(16 * q + n) * 4u;                 // word row 0, channel 16q + n
  const uint32_t vsv = (uint32_t)(2 * n) * (uint32_t)(L::VG * 2);   // scales of my two tokens

  // Values are read once: their loads carry the non-temporal hint, so that they
  // do not push the key lines out of L2 (a key block uses a quarter of each
  // 128-byte line of its channels' codes; the next blocks use the rest).
  constexpr int kNT = 2;
  auto vissue = [&](VStage8<D> &V, int tile0, bool live) {
    __builtin_amdgcn_sched_barrier(0);
    live = live && tile0 < t_end;
    const uint32_t u0 = (uint32_t)tile0;
    const auto rvw = rsrc(vwords, vw_bytes, (u0 >> 4) * (uint32_t)(D * 4), live);
    const auto rvs = rsrc(vscales, vs_bytes, u0 * (uint32_t)(L::VG * 2), live);
#pragma unroll
    for (int hf = 0; hf < L::NH; ++hf)
#pragma unroll
      for (int wr = 0; wr < 2; ++wr)
        V.vw[hf][wr] = __builtin_amdgcn_raw_buffer_load_b32(rvw, vwv + (uint32_t)(wr * D + 64 * hf) * 4u, 0, kNT);
    if constexpr (L::VG == 4) {
      const u32x4 x = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rvs, vsv, 0, kNT));
      V.vs[0] = x.x; V.vs[1] = x.y; V.vs[2] = x.z; V.vs[3] = x.w;
    } else {
      const u32x2 x = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rvs, vsv, 0, kNT));
      V.vs[0] = x.x; V.vs[1] = x.y;
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---------------------------------------------------------------- running state
  float m_run[G];
#pragma unroll
  for (int h = 0; h < G; ++h) m_run[h] = -INFINITY;
  int f_run = 0, es_run = -24;
  uint32_t sbound = 0u;
  bool firstv = true;
  float fp[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) fp[nt] = (float)(f_run + 24 - 2 * pk[nt]);
  float lacc[2][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}};
  // weighted sum, per half of the heads (heads 4 hq2 .. 4 hq2 + 3): lane (n, q)
  // accumulates those heads of channel 64 half + 16q + n
  f32x4 vacc[2][L::NH];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int hf = 0; hf < L::NH; ++hf) vacc[h2][hf] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float sacc[2][L::VG];   // S = 2^F sum p scale per (head 2q + hh, value group j), partial per lane
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int j = 0; j < L::VG; ++j) sacc[hh][j] = 0.0f;
  const float kback[2] = {ldexpf(1.0f, 2 * pk[0] - 24), ldexpf(1.0f, 2 * pk[1] - 24)};
  if (lane == 0) W.zero = u32x4{0u, 0u, 0u, 0u};

  auto values = [&](const VStage8<D> &V, int tile0, const float (&z)[2][2], const float (&mr)[2]) {
    const int t0 = tile0 + 2 * n;
    const uint32_t m0 = t0 < t_end ? 0xffffffffu : 0u, m1 = t0 + 1 < t_end ? 0xffffffffu : 0u;
    uint32_t cvs[L::VG];
#pragma unroll
    for (int i = 0; i < L::VG; ++i) cvs[i] = V.vs[i] & (i < L::VG / 2 ? m0 : m1);

    // value exponent F: moves only when a value scale outgrows 2^es_run
    uint32_t smax = 0;
#pragma unroll
    for (int i = 0; i < L::VG; ++i) smax = max(smax, max(cvs[i] & 0xffffu, cvs[i] >> 16));
    if (firstv || __ballot(smax >= sbound) != 0ull) {
      const float sv2 = wave_max(h2f(smax));
      int es_t = -24;
      if (sv2 > 0.0f) frexpf(sv2, &es_t);
      const int es_new = firstv ? es_t : max(es_run, es_t);
      const int f_new = 15 - 24 - es_new;
      if (!firstv) {
        const float beta = ldexpf(1.0f, f_new - f_run);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int hf = 0; hf < L::NH; ++hf) vacc[h2][hf] *= beta;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
          for (int j = 0; j < L::VG; ++j) sacc[hh][j] *= beta;
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) lacc[hh][nt] *= beta;
        }
      }
      f_run = f_new;
      es_run = es_new;
      sbound = pow2_bits(es_new);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) fp[nt] = (float)(f_run + 24 - 2 * pk[nt]);
      firstv = false;
    }

    // numerators -> value A operands (row = head, K = token)
    float p[2][2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        p[hh][nt] = __builtin_amdgcn_exp2f(z[hh][nt] - mr[hh] + fp[nt]);
        lacc[hh][nt] += p[hh][nt];
      }
#pragma unroll
    for (int j = 0; j < L::VG; ++j) {
      const uint32_t s0 = cvs[j >> 1], s1 = cvs[L::VG / 2 + (j >> 1)];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        uint16_t *dst = &W.u.t.pbuf[j][pkc][(pw * kG8 + 2 * q + hh) * 8 + pi0];
        const uint32_t a0 = (j & 1) ? mixlo<1>(p[hh][0], s0) : mixlo<0>(p[hh][0], s0);
        const uint32_t a1 = (j & 1) ? mixlo<1>(p[hh][1], s1) : mixlo<0>(p[hh][1], s1);
        dst[0] = (uint16_t)a0;
        dst[2] = (uint16_t)a1;
        sacc[hh][j] = mix_acc(sacc[hh][j], a0, kback[0]);
        sacc[hh][j] = mix_acc(sacc[hh][j], a1, kback[1]);
      }
    }
    wave_sync();

    // weighted sum of the value codes, the operand of each code word shared by
    // both halves of the heads: A of lane (row 4jj + h, K group q) is head
    // 4 h2 + h's 8 numerators of value group 2 half + jj/2 when q == jj, else zero
    const int jj = n >> 2, ah = n & 3;
#pragma unroll
    for (int hf = 0; hf < L::NH; ++hf)
#pragma unroll
      for (int wr = 0; wr < 2; ++wr)
#pragma unroll
        for (int kc2 = 0; kc2 < 2; ++kc2) {
          const u32x4 bv = value_operand(V.vw[hf][wr], kc2);
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const u32x4 *src =
                q == jj ? reinterpret_cast<const u32x4 *>(&W.u.t.pbuf[2 * hf + (jj >> 1)][kc2][(wr * kG8 + 4 * h2 + ah) * 8])
                        : &W.zero;
            vacc[h2][hf] = mfma16(*src, bv, vacc[h2][hf]);
          }
        }
    wave_sync();
  };

  // ---------------------------------------------------------------- chunks
  for (int cb = 0; cb < nb;) {
    if (cb > 0) block_barrier();
    const int nbc = nb - cb == kChunk8 + 1 ? kChunk8 + 1 : min(kChunk8, nb - cb);
    const int c_t0 = t_begin + kBlock8 * cb;
    float zs[kChunk8][2][2];
    float zl[2] = {-INFINITY, -INFINITY};

    // pass 1: keys (block i in LDS buffer i & 1, loads two blocks ahead)
    if (cb > 0) {
      kissue(S0, c_t0, 0 < nbc);
      kissue(S1, c_t0 + kBlock8, 1 < nbc);
    }
    __builtin_amdgcn_s_setprio(1);
    kcommit(S0, sm.kb[0], c_t0);
    kissue(S0, c_t0 + 2 * kBlock8, 2 < nbc);
    block_barrier();
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int i = 0; i < kChunk8; ++i) {
      if (i >= nbc) break;
      const int p0 = c_t0 + kBlock8 * i;
      logits(sm.kb[i & 1], p0 + kTile8 * wave, zs[i]);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) zl[hh] = fmaxf(zl[hh], fmaxf(zs[i][hh][0], zs[i][hh][1]));
      KStage8 &S = (i & 1) ? S0 : S1;   // holds block i + 1
      __builtin_amdgcn_s_setprio(1);
      kcommit(S, sm.kb[(i + 1) & 1], p0 + kBlock8);
      kissue(S, p0 + 3 * kBlock8, i + 3 < nbc);
      block_barrier();
      __builtin_amdgcn_s_setprio(0);
    }
    float z9[2][2];
    if (nbc > kChunk8) {
      logits(sm.kb[kChunk8 & 1], c_t0 + kBlock8 * kChunk8 + kTile8 * wave, z9);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) zl[hh] = fmaxf(zl[hh], fmaxf(z9[hh][0], z9[hh][1]));
    }

    // pass 2: values; the first three tiles are on their way during the maximum
    VStage8<D> V0, V1, V2;
    vissue(V0, c_t0 + kTile8 * wave, true);
    vissue(V1, c_t0 + kBlock8 + kTile8 * wave, 1 < nbc);
    vissue(V2, c_t0 + 2 * kBlock8 + kTile8 * wave, 2 < nbc);

    // exact maximum of each head's logits in the chunk (wavefront-uniform):
    // row q of the lanes holds heads 2q and 2q + 1
    float d[G];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const float zm = row16_max(zl[hh]);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        d[2 * r + hh] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, zm), 16 * r));
    }
    bool rise = false;
    float al[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mn = fmaxf(m_run[h], d[h]);
      al[h] = (m_run[h] == -INFINITY || mn == m_run[h]) ? 1.0f : exp2f(m_run[h] - mn);
      rise = rise || (m_run[h] != -INFINITY && mn > m_run[h]);
      m_run[h] = mn;
    }
    if (rise) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int hf = 0; hf < L::NH; ++hf)
#pragma unroll
          for (int i = 0; i < 4; ++i) vacc[h2][hf][i] *= al[4 * h2 + i];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const float a = sel4(q, al[hh], al[2 + hh], al[4 + hh], al[6 + hh]);
#pragma unroll
        for (int j = 0; j < L::VG; ++j) sacc[hh][j] *= a;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) lacc[hh][nt] *= a;
      }
    }
    float mr[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const float m = sel4(q, m_run[hh], m_run[2 + hh], m_run[4 + hh], m_run[6 + hh]);
      mr[hh] = m == -INFINITY ? 0.0f : m;
    }

#pragma unroll
    for (int i = 0; i < kChunk8; ++i) {
      if (i >= nbc) break;
      VStage8<D> &V = (i % 3 == 0) ? V0 : (i % 3 == 1) ? V1 : V2;
      const int tile0 = c_t0 + kBlock8 * i + kTile8 * wave;
      if (tile0 < t_end) values(V, tile0, zs[i], mr);
      __builtin_amdgcn_s_setprio(1);
      vissue(V, tile0 + 3 * kBlock8, i + 3 < nbc);
      __builtin_amdgcn_s_setprio(0);
    }
    if (nbc > kChunk8) {
      const int tile0 = c_t0 + kBlock8 * kChunk8 + kTile8 * wave;
      VStage8<D> &VX = kChunk8 % 3 == 0 ? V0 : kChunk8 % 3 == 1 ? V1 : V2;
      if (tile0 < t_end) values(VX, tile0, z9, mr);
    }
    cb += nbc;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---------------------------------------------------------------- merge the wavefronts
  const bool had = t_begin + kTile8 * wave < t_end;
  {
    float lh[G];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      float ll = fmaf(lacc[hh][0], ldexpf(1.0f, -(int)fp[0]), lacc[hh][1] * ldexpf(1.0f, -(int)fp[1]));
      ll = row16_sum(ll);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        lh[2 * r + hh] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ll), 16 * r));
    }
    float sh[G][L::VG];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int j = 0; j < L::VG; ++j) {
        const float v = row16_sum(sacc[hh][j]);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sh[2 * r + hh][j] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16 * r));
      }
    const float inv_f = ldexpf(1.0f, -f_run);
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int hf = 0; hf < L::NH; ++hf) {
        const int ch = 64 * hf + 16 * q + n;   // value group 2 hf + (q >> 1)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int h = 4 * h2 + i;
          const float si = sel2((q >> 1) != 0, sh[h][2 * hf], sh[h][2 * hf + 1]);
          W.u.merge[h][ch] = (2.0f * vacc[h2][hf][i] - 3.0f * si) * inv_f;
        }
      }
#pragma unroll
    for (int h = 0; h < G; ++h)
      if (lane == h) {
        W.mstate[h] = m_run[h];
        W.lstate[h] = had ? lh[h] : 0.0f;
      }
  }
  __syncthreads();
  static_assert((G * D) % kThreads8 == 0, "whole rounds of elements");
#pragma unroll
  for (int k = 0; k < (G * D) / kThreads8; ++k) {
    const int e = tid + kThreads8 * k, h = e / D, ch = e % D;
    float lw[kWaves8], mw[kWaves8], ow[kWaves8];
#pragma unroll
    for (int w = 0; w < kWaves8; ++w) {
      lw[w] = sm.w[w].lstate[h];
      mw[w] = sm.w[w].mstate[h];
      ow[w] = sm.w[w].u.merge[h][ch];
    }
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves8; ++w) M = lw[w] > 0.0f ? fmaxf(M, mw[w]) : M;
    float o = 0.0f, Lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves8; ++w) {
      const bool live = lw[w] > 0.0f;
      const float f = exp2f((live ? mw[w] : M) - M);
      o = live ? fmaf(ow[w], f, o) : o;
      Lsum = live ? fmaf(lw[w], f, Lsum) : Lsum;
    }
    if (outp) {
      const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
      outp[h * D + ch] = o * inv;
    } else {
      wsp[h * (D + kPartialHead) + kPartialHead + ch] = o;
      if (ch == 0) {
        wsp[h * (D + kPartialHead) + 0] = M;
        wsp[h * (D + kPartialHead) + 1] = Lsum;
      }
    }
  }
}

}  // namespace

bool decode8_supported(const dqk_cache &c, int hq) {
  return c.capacity % 64 == 0 && hq == kG8 * c.num_kv_heads;
}

hipError_t launch_decode8(const dqk_cache &c, const float *q_prime, const int32_t *sel_idx, bool shared,
                          int hq, int keep, float scale2, int split, bool even, float *ws, float *out,
                          hipStream_t s) {
  const int nsplit = num_splits(c.capacity, split);
  // a caller's split of whole 128-token blocks covers exactly its tokens of
  // every row; otherwise each split takes a share of its row's current blocks
  const int bps = !even && split % kBlock8 == 0 ? split / kBlock8 : 0;
  const int units = c.batch * c.num_kv_heads;
  const int items = units * nsplit;
  const int grid3 = c.batch <= 65535 && nsplit <= 65535 ? 1 : 0;
  const dim3 grid = grid3 ? dim3((unsigned)c.num_kv_heads, (unsigned)c.batch, (unsigned)nsplit)
                          : dim3((unsigned)items);
  int ncu = 0;
  if (even && bps == 0) {
    const int n = compute_units();
    if (n > 0 && n < 4096 && items > n && items <= 2 * n) ncu = n;
  }
  const int ncu_q = ncu / units, ncu_r = ncu % units;
  // group-shared kept sets use compact slots: only the K chunks (32 slots each)
  // that hold the keep - 1 kept channels other than 0 are worked on
  const int nkc = shared ? (keep - 1 + 31) / 32 : c.head_dim / 32;
  const dim3 block(kThreads8);
  if (c.head_dim == 64) {
    if (shared)
      hipLaunchKernelGGL((decode8_kernel<64, true>), grid, block, 0, s, c, q_prime, sel_idx, hq, grid3, keep,
                         scale2, nsplit, bps, ncu_q, ncu_r, nkc, ws, out);
    else
      hipLaunchKernelGGL((decode8_kernel<64, false>), grid, block, 0, s, c, q_prime, sel_idx, hq, grid3, keep,
                         scale2, nsplit, bps, ncu_q, ncu_r, nkc, ws, out);
  } else {
    if (shared)
      hipLaunchKernelGGL((decode8_kernel<128, true>), grid, block, 0, s, c, q_prime, sel_idx, hq, grid3, keep,
                         scale2, nsplit, bps, ncu_q, ncu_r, nkc, ws, out);
    else
      hipLaunchKernelGGL((decode8_kernel<128, false>), grid, block, 0, s, c, q_prime, sel_idx, hq, grid3, keep,
                         scale2, nsplit, bps, ncu_q, ncu_r, nkc, ws, out);
  }
  return hipGetLastError();
}

}  // namespace dqk
