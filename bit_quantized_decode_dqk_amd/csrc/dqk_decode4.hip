// Decode attention over the 2-bit cache for GQA groups of four query heads
// (hq / hkv == 4), both contractions on the matrix cores.
//
// Dual-QK (arXiv abstract; tech.dede.sh summary, "Throughput on SGLang"): keys
// and values are stored in 2 bits and the key channels a query head does not
// keep are never read, which is where the decode speedup comes from.  One
// workgroup serves the four query heads of one KV head over an equal share of
// the sequence's 64-token tiles; only the union U of the group's kept key
// channels is read (their 2-bit rows are channel-major, so a dropped channel
// costs no bytes), together with channel 0's fp16 row and, for the unfinished
// last group, the exact tail.  Each head's logit uses only its own channels (its
// coefficient is zero on the others).  Values are never pruned.
//
// Decoding.  A 2-bit code u whose bit pair sits at bits 2k, 2k+1 of an fp16 word
// with a zero exponent field is the subnormal u * 2^(2k-24), exact; masking a
// packed code word therefore yields two operands per instruction with no shift
// and no offset, and the power 2^(2k-24) is compensated in the other operand or
// in the output.  The matrix cores take fp16 subnormals as they are.  With the
// level 2u - 3 of a code:
//  - logits, per 64-token tile with key groups g = 0, 1: A[(g, h, limb)][(g, s)]
//    is the fp16 high or low part of q'_{h,U[s]} * sm * log2(e) * scale_{U[s],g}
//    * 2^-E_h, block diagonal over g (rows 8g + 2h + limb, K = 16 union slots of
//    each group); B[(g, s)][t] = u_{s,t} 2^(2r-24) with r = t mod 4; a product
//    with B = 1 gives C1 = sum A.  Then
//      z = 2^(E_h + 25 - 2r) (C_high + C_low) - 3 2^E_h (C1_high + C1_low) + ch0 term.
//  - values, per 32 tokens and 16 channels of value group j: A[h][t] =
//    p_{h,t} scale_{t,j} 2^(F + 24 - 2k(t)) in fp16 (p the softmax numerator, F a
//    power of two that keeps A finite), B[t][c] = u 2^(2k-24); a product with
//    B = 2^(2k-24) gives S = 2^F sum p scale, and out = 2^-F (2 C - 3 S).
// Softmax: each wavefront keeps a running maximum per head that may trail the
// largest logit seen by up to 8 (log2 units); it moves, and the running sums
// are rescaled, only when a logit exceeds it by more than that or a value scale
// outgrows the range that 2^F allows.
#include "dqk_internal.h"
#include "dqk_wave.h"

namespace dqk {
namespace {

using namespace wave;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half2 __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));

constexpr int kG4 = 4;              // query heads per KV head
constexpr int kThreads4 = 256;
constexpr int kWaves4 = kThreads4 / 64;
constexpr int kTile4 = 64;          // tokens per wavefront tile: two key groups
constexpr float kSlack = 8.0f;      // log2 headroom of the running maximum
constexpr uint32_t kOneF16x2 = 0x3C003C00u;
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit elements, range-checked (gfx9)
constexpr uint32_t kFar = 0x40000000u;   // offset past every plane: the load returns zero

template <int D>
struct Lay4 {
  static constexpr int OCT = D / 8;     // union-slot octets
  static constexpr int NKC = D / 16;    // logit K chunks (16 slots of each key group)
  static constexpr int VG = D / 32;     // value scale groups
  static constexpr int SPL = D / 8;     // union slots per lane in the logit A build
  static constexpr int AROW = D + 8;    // fp16 per logit A row (padded against bank conflicts)
  static constexpr int KSL = D / 64;    // key-scale slots loaded per lane
};

template <int D>
struct __attribute__((aligned(16))) WaveSmem4 {
  union {
    struct {
      uint32_t y[Lay4<D>::OCT][16][2];           // key codes: slot octet, token quad, slots 0-3 | 4-7
      uint16_t ksig[2][D];                        // key scales (fp16 bits): key group, slot
      uint16_t abuf[16][Lay4<D>::AROW];           // logit A rows 8g+2h+limb, slots in octet order 0,2,1,3,4,6,5,7
      uint16_t pbuf[Lay4<D>::VG][2][kG4][4][8];   // value A: group j, K chunk, head, word, K position
    } t;
    float merge[kG4][D];                          // the wavefront's output at the end of the split
  } u;
  float mstate[kG4], lstate[kG4];
};

template <int D>
struct __attribute__((aligned(16))) Smem4 {
  WaveSmem4<D> w[kWaves4];
  float coefc[kG4][D];     // q' * sm * log2(e) by channel (0 where the head drops the channel)
  float coefs[kG4][D];     // coefc in union-slot order * 2^-E_h (0 past |U|)
  float e2[kG4];           // 2^E_h
  float redm[kG4][kWaves4];
  int hmask[D];
  int16_t ulist[D];
  int wcount[2];
};

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
__device__ __forceinline__ uint16_t f2h(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// c ? b : a on two values the compiler may not fold into an indexed load
// (an array indexed by a lane-dependent value would go to scratch memory).
__device__ __forceinline__ float sel2(bool c, float a, float b) {
  asm volatile("" : "+v"(a), "+v"(b));
  return c ? b : a;
}

// a * (fp16 in the low or high half of h), one mixed-precision FMA (exact product,
// one rounding), register operands only.
template <int HALF>
__device__ __forceinline__ float mul_f16(float a, uint32_t h) {
  float d;
  if constexpr (HALF == 0)
    asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "=v"(d) : "v"(a), "v"(h));
  else
    asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "=v"(d) : "v"(a), "v"(h));
  return d;
}

// a * (fp16 half SH of s) - (fp16 half HH of h): the part of the product that
// the fp16 number in h leaves out, in one mixed-precision FMA.
template <int SH, int HH>
__device__ __forceinline__ float fma_res(float a, uint32_t s, uint32_t h) {
  float d;
  if constexpr (SH == 0 && HH == 0)
    asm("v_fma_mix_f32 %0, %1, %2, -%3 op_sel:[0,0,0] op_sel_hi:[0,1,1]" : "=v"(d) : "v"(a), "v"(s), "v"(h));
  else if constexpr (SH == 0 && HH == 1)
    asm("v_fma_mix_f32 %0, %1, %2, -%3 op_sel:[0,0,1] op_sel_hi:[0,1,1]" : "=v"(d) : "v"(a), "v"(s), "v"(h));
  else if constexpr (SH == 1 && HH == 0)
    asm("v_fma_mix_f32 %0, %1, %2, -%3 op_sel:[0,1,0] op_sel_hi:[0,1,1]" : "=v"(d) : "v"(a), "v"(s), "v"(h));
  else
    asm("v_fma_mix_f32 %0, %1, %2, -%3 op_sel:[0,1,1] op_sel_hi:[0,1,1]" : "=v"(d) : "v"(a), "v"(s), "v"(h));
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

// KSP: the capacity is a multiple of 64, so the two key-group scales of a tile
// are one aligned dword of every scale row.
template <int D, bool KSP>
__global__ __launch_bounds__(kThreads4, 2) void decode4_kernel(dqk_cache c,
                                                               const float *__restrict__ qp,
                                                               const int32_t *__restrict__ sel,
                                                               int hq, int keep, float scale2,
                                                               int nsplit, float *__restrict__ ws) {
  using L = Lay4<D>;
  constexpr int G = kG4;
  __shared__ Smem4<D> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Split-major order: workgroups of one split index run together.
  const int units = c.batch * c.num_kv_heads;
  const int unit = blockIdx.x % units, s = blockIdx.x / units;
  const int b = unit / c.num_kv_heads, g = unit % c.num_kv_heads;
  const int len = max(0, min(c.lengths[b], c.capacity));
  const int ntot = (len + kTile4 - 1) / kTile4;
  const int tlo = (int)(((long long)s * ntot) / nsplit);
  const int thi = (int)(((long long)(s + 1) * ntot) / nsplit);
  const int t_begin = tlo * kTile4;
  const int t_end = min(thi * kTile4, len);
  float *wsp = ws + ((size_t)unit * nsplit + s) * G * (D + kPartialHead);
  if (t_begin >= t_end) {
    for (int e = tid; e < G * (D + kPartialHead); e += kThreads4)
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
  const uint16_t *vscales = c.v_scales + unit * (size_t)c.capacity * L::VG;
  const int t_body = (len / kGroup) * kGroup;
  const int code_end = min(t_body, t_end);

  // ---------------------------------------------------------------- setup (whole workgroup)
  for (int e = tid; e < G * D; e += kThreads4) sm.coefc[e / D][e % D] = 0.0f;
  for (int e = tid; e < D; e += kThreads4) sm.hmask[e] = 0;
  __syncthreads();
  const size_t row0 = (size_t)b * hq + (size_t)g * G;
  for (int e = tid; e < G * keep; e += kThreads4) {
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
  const int nkc = (nu + 15) / 16;
  for (int e = tid; e < G * D; e += kThreads4) {
    const int h = e / D, i = e % D;
    float mx = sm.redm[h][0];
#pragma unroll
    for (int w = 1; w < kWaves4; ++w) mx = fmaxf(mx, sm.redm[h][w]);
    int ex = 0;
    if (mx > 0.0f) frexpf(mx, &ex);
    sm.coefs[h][i] = i < nu ? sm.coefc[h][sm.ulist[i]] * ldexpf(1.0f, -ex) : 0.0f;
    if (i == 0) sm.e2[h] = ldexpf(1.0f, ex);
  }
  __syncthreads();

  // ---------------------------------------------------------------- per-wavefront state
  WaveSmem4<D> &W = sm.w[wave];
  const int q = lane >> 4, n = lane & 15;
  const int lg = q >> 1, hp = q & 1;   // logit lanes: key group of the tile, head pair (2hp, 2hp+1)

  // logit A build: (group ab_g, head ab_h, slots ab_s .. ab_s+SPL-1)
  const int ab_g = lane >> 5, ab_h = (lane >> 3) & 3, ab_s = L::SPL * (lane & 7);
  float cf[L::SPL];
#pragma unroll
  for (int i = 0; i < L::SPL; ++i) cf[i] = sm.coefs[ab_h][ab_s + i];
  const bool arow = (n >> 3) == (q >> 1);   // my A row belongs to my K block's key group

  // Loads go through buffer resources of the unit's planes: an offset past the
  // plane returns zero, so absent slots simply point past the end (kFar).
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      (void *)kcodes, (short)0, (int)(D * kc_stride), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rks = __builtin_amdgcn_make_buffer_rsrc(
      (void *)kscales, (short)0, (int)(D * ks_stride * 2), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rc0 = __builtin_amdgcn_make_buffer_rsrc(
      (void *)c0row, (short)0, (int)(c.capacity * 2), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rvw = __builtin_amdgcn_make_buffer_rsrc(
      (void *)vwords, (short)0, (int)((c.capacity / 16) * D * 4), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rvs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)vscales, (short)0, (int)(c.capacity * L::VG * 2), kRsrcWord3);

  // key-code loads: slot octet so, 16-token block tb of the tile
  const int so = lane >> 2, tb = lane & 3;
  uint32_t kvo[8];
#pragma unroll
  for (int cc = 0; cc < 8; ++cc) {
    const int i = 8 * so + cc;
    kvo[cc] = (so < L::OCT && i < nu) ? (uint32_t)(sm.ulist[i] * kc_stride) + 4u * tb : kFar;
  }
  uint32_t ksv[L::KSL];
#pragma unroll
  for (int cs = 0; cs < L::KSL; ++cs) {
    const int i = lane + 64 * cs;
    ksv[cs] = i < nu ? (uint32_t)(sm.ulist[i] * ks_stride * 2) : kFar;
  }
  const uint32_t c0v = (uint32_t)(32 * lg + 2 * n) * 2u;
  const uint32_t vwv = (uint32_t)(q * D + 2 * n) * 4u;
  const uint32_t vsv = (uint32_t)(32 * lg + 2 * n) * (uint32_t)(L::VG * 2);

  // logit output: tokens 32lg + 2n + nt (nt = 0, 1), token position r = 2(n&1) + nt in its quad
  const uint32_t mk0 = 0x00030003u << (4 * (n & 1)), mk1 = mk0 << 2;
  float ez[2][2], n3e[2], c0c[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int h = 2 * hp + hh;
    const float e = sm.e2[h];
    n3e[hh] = -3.0f * e;
    c0c[hh] = sm.coefc[h][0];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) ez[hh][nt] = ldexpf(e, 25 - 2 * (2 * (n & 1) + nt));
  }
  // value A producer: my tokens are c = 2(n&7), c+1 of word 2lg + (n>>3)
  const int pw = 2 * lg + (n >> 3), pkc = (n >> 1) & 1, pi0 = 4 * (n & 1) + ((n >> 2) & 1);
  const int pk[2] = {value_k(2 * (n & 3)), value_k(2 * (n & 3) + 1)};

  // running state
  float m_run[G];
#pragma unroll
  for (int h = 0; h < G; ++h) m_run[h] = 0.0f;
  float mr[2] = {0.0f, 0.0f};
  int f_run = 0, es_run = -24;
  uint32_t sbound = 0x7C00u;
  float fp[2], thr[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    fp[nt] = (float)(f_run + 24 - 2 * pk[nt]);
    thr[nt] = kSlack + fp[nt];
  }
  bool first = true;
  float lacc[2][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}};
  f32x4 vacc[L::VG][2], sacc[L::VG];
#pragma unroll
  for (int j = 0; j < L::VG; ++j) {
    vacc[j][0] = vacc[j][1] = sacc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  u32x4 alog[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};   // logit A operands: zero in off-diagonal lanes
  u32x4 aval[2];   // value A operands
  u32x4 ones = {kOneF16x2, kOneF16x2, kOneF16x2, kOneF16x2};
  const u32x4 unit_k[2] = {{0x00010001u, 0x00040004u, 0x00100010u, 0x00400040u},
                           {0x01000100u, 0x00100010u, 0x00400040u, 0x01000100u}};

  const int ntiles = thi - tlo;

  // prefetch registers (next tile) and the current tile's value operands
  uint32_t px[8];
  uint32_t pks[L::KSL][2];   // fp16 scale bits of the tile's two key groups (one or two loads)
  uint32_t nx0, cx0 = 0;
  u32x2 nvw[L::VG], cvw[L::VG];
  uint32_t nvs[L::VG], cvs[L::VG];   // fp16 scales: [j/2] of token 0 then of token 1 (packed pairs)

  auto issue = [&](int tk) {
    const uint32_t p0 = (uint32_t)(t_begin + kTile4 * tk);
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) px[cc] = __builtin_amdgcn_raw_buffer_load_b32(rk, kvo[cc] + (p0 >> 2), 0, 0);
#pragma unroll
    for (int cs = 0; cs < L::KSL; ++cs) {
      const uint32_t off = ksv[cs] + (p0 / kGroup) * 2u;
      if constexpr (KSP) {
        pks[cs][0] = __builtin_amdgcn_raw_buffer_load_b32(rks, off, 0, 0);
      } else {
        pks[cs][0] = __builtin_amdgcn_raw_buffer_load_b16(rks, off, 0, 0);
        pks[cs][1] = __builtin_amdgcn_raw_buffer_load_b16(rks, off + 2u, 0, 0);
      }
    }
    nx0 = __builtin_amdgcn_raw_buffer_load_b32(rc0, c0v + p0 * 2u, 0, 0);
#pragma unroll
    for (int j = 0; j < L::VG; ++j)
      nvw[j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rvw, vwv + (p0 >> 4) * (uint32_t)(D * 4) + 128u * j, 0, 0));
    if constexpr (L::VG == 4) {
      const u32x4 x = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rvs, vsv + p0 * (uint32_t)(L::VG * 2), 0, 0));
      nvs[0] = x.x; nvs[1] = x.y; nvs[2] = x.z; nvs[3] = x.w;
    } else {
      const u32x2 x = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rvs, vsv + p0 * (uint32_t)(L::VG * 2), 0, 0));
      nvs[0] = x.x; nvs[1] = x.y;
    }
  };

  auto commit = [&](int tk_next) {
    if (so < L::OCT) {
      uint32_t y0[4], y1[4];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const uint32_t *x = px + 4 * half;
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
      u32x4 *dst = reinterpret_cast<u32x4 *>(&W.u.t.y[so][4 * tb][0]);
      dst[0] = u32x4{y0[0], y1[0], y0[1], y1[1]};
      dst[1] = u32x4{y0[2], y1[2], y0[3], y1[3]};
    }
    {
      // scales of a key group past the coded range (the exact tail or beyond) stay zero
      const int grp0 = (t_begin + kTile4 * tk_next) / kGroup;
      const uint32_t keep0 = grp0 * kGroup < code_end ? 0xffffu : 0u;
      const uint32_t keep1 = (grp0 + 1) * kGroup < code_end ? 0xffff0000u : 0u;
#pragma unroll
      for (int cs = 0; cs < L::KSL; ++cs) {
        const uint32_t raw = KSP ? pks[cs][0] : (pks[cs][0] & 0xffffu) | (pks[cs][1] << 16);
        const uint32_t v = raw & (keep0 | keep1);
        W.u.t.ksig[0][lane + 64 * cs] = (uint16_t)v;
        W.u.t.ksig[1][lane + 64 * cs] = (uint16_t)(v >> 16);
      }
    }
    cx0 = nx0;
    {
      // value scales of tokens past the split end are zero (their numerators are zero too)
      const int t0 = t_begin + kTile4 * tk_next + 32 * lg + 2 * n;
      const uint32_t m0 = t0 < t_end ? 0xffffffffu : 0u, m1 = t0 + 1 < t_end ? 0xffffffffu : 0u;
#pragma unroll
      for (int j = 0; j < L::VG; ++j) {
        cvw[j] = nvw[j];
        cvs[j] = nvs[j] & (j < L::VG / 2 ? m0 : m1);
      }
    }
  };

  if (wave < ntiles) {
    issue(wave);
    commit(wave);
  }
  wave_sync();

  for (int tk = wave; tk < ntiles; tk += kWaves4) {
    const int tile0 = t_begin + kTile4 * tk;
    const bool more = tk + kWaves4 < ntiles;
    if (more) issue(tk + kWaves4);   // in flight during this tile's compute

    // ---- logit A operands of the tile's two key groups (compact build)
    {
      const u32x4 *src = reinterpret_cast<const u32x4 *>(&W.u.t.ksig[ab_g][ab_s]);
#pragma unroll
      for (int o = 0; o < L::SPL / 8; ++o) {
        const u32x4 sg = src[o];
        // pairs in octet order (0,2) (1,3) (4,6) (5,7): high part = fp16 of the
        // product, low part = fp16 of what the high part leaves out
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int pr = 0; pr < 4; ++pr) {
          // slots ta and ta+2: the same half (ta & 1) of sigma dwords ta>>1 and ta>>1 + 1
          const int ta = (pr & 2) * 2 + (pr & 1);
          const float ca = cf[8 * o + ta], cb = cf[8 * o + ta + 2];
          const uint32_t sa = sg[ta >> 1], sb = sg[(ta >> 1) + 1];
          float xa, xb, ra, rb;
          if (ta & 1) {
            xa = mul_f16<1>(ca, sa);
            xb = mul_f16<1>(cb, sb);
          } else {
            xa = mul_f16<0>(ca, sa);
            xb = mul_f16<0>(cb, sb);
          }
          const uint32_t hh = __builtin_bit_cast(uint32_t, __builtin_convertvector((float2v){xa, xb}, half2));
          if (ta & 1) {
            ra = fma_res<1, 0>(ca, sa, hh);
            rb = fma_res<1, 1>(cb, sb, hh);
          } else {
            ra = fma_res<0, 0>(ca, sa, hh);
            rb = fma_res<0, 1>(cb, sb, hh);
          }
          hw[pr] = hh;
          lw[pr] = __builtin_bit_cast(uint32_t, __builtin_convertvector((float2v){ra, rb}, half2));
        }
        u32x4 *dh = reinterpret_cast<u32x4 *>(&W.u.t.abuf[8 * ab_g + 2 * ab_h][ab_s + 8 * o]);
        u32x4 *dl = reinterpret_cast<u32x4 *>(&W.u.t.abuf[8 * ab_g + 2 * ab_h + 1][ab_s + 8 * o]);
        *dh = u32x4{hw[0], hw[1], hw[2], hw[3]};
        *dl = u32x4{lw[0], lw[1], lw[2], lw[3]};
      }
    }
    wave_sync();

    // ---- logits: C rows (group lg, heads 2hp, 2hp+1, high/low), columns tokens 32lg + 2n + nt
    f32x4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = acc0, accs = acc0;
    asm volatile("" : "+v"(ones));
    {
      u32x2 dd[2];
      if (nkc > 0) {
        if (arow) alog[0] = *reinterpret_cast<const u32x4 *>(&W.u.t.abuf[n][8 * (q & 1)]);
        dd[0] = *reinterpret_cast<const u32x2 *>(&W.u.t.y[q & 1][8 * lg + (n >> 1)][0]);
      }
#pragma unroll
      for (int kc = 0; kc < L::NKC; ++kc) {
        if (kc < nkc) {
          const int cur = kc & 1, nxt = cur ^ 1;
          if (kc + 1 < L::NKC && kc + 1 < nkc) {
            if (arow) alog[nxt] = *reinterpret_cast<const u32x4 *>(&W.u.t.abuf[n][16 * (kc + 1) + 8 * (q & 1)]);
            dd[nxt] = *reinterpret_cast<const u32x2 *>(&W.u.t.y[2 * (kc + 1) + (q & 1)][8 * lg + (n >> 1)][0]);
          }
          const uint32_t d0 = dd[cur].x, d1 = dd[cur].y, d0s = d0 >> 8, d1s = d1 >> 8;
          const u32x4 b0 = {d0 & mk0, d0s & mk0, d1 & mk0, d1s & mk0};
          const u32x4 b1 = {d0 & mk1, d0s & mk1, d1 & mk1, d1s & mk1};
          acc0 = mfma16(alog[cur], b0, acc0);
          acc1 = mfma16(alog[cur], b1, acc1);
          accs = mfma16(alog[cur], ones, accs);
        }
      }
    }

    // ---- logits (log2 units) relative to the running max, plus the value exponent
    float zp[2][2];
    const float x0f[2] = {h2f(cx0 & 0xffffu), h2f(cx0 >> 16)};
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const float cs = accs[2 * hh] + accs[2 * hh + 1];
      const float bb = fmaf(n3e[hh], cs, -mr[hh]);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const f32x4 &a = nt == 0 ? acc0 : acc1;
        const float u = a[2 * hh] + a[2 * hh + 1];
        const float w = fmaf(c0c[hh], x0f[nt], bb + fp[nt]);
        zp[hh][nt] = fmaf(ez[hh][nt], u, w);
      }
    }
    const int tl0 = tile0 + 32 * lg + 2 * n;   // my first token
    if (tile0 + kTile4 > t_end) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        if (tl0 + nt >= t_end) zp[0][nt] = zp[1][nt] = -INFINITY;
    }
    // tokens of the unfinished last group: exact fp32 tail keys
    if (tile0 + kTile4 > t_body && t_body < t_end) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int t = tl0 + nt;
        if (t >= t_body && t < t_end) {
          const float *row = tail + (size_t)(t & 31) * D;
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int h = 2 * hp + hh;
            float zz = sm.coefc[h][0] * x0f[nt];
            for (int i = 0; i < nu; ++i) {
              const int ch = sm.ulist[i];
              zz = fmaf(sm.coefc[h][ch], row[ch], zz);
            }
            zp[hh][nt] = zz - mr[hh] + fp[nt];
          }
        }
      }
    }

    // ---- running maximum / value exponent: move only when needed (wavefront-uniform)
    uint32_t smax = 0;
#pragma unroll
    for (int i = 0; i < L::VG; ++i) smax = max(smax, max(cvs[i] & 0xffffu, cvs[i] >> 16));
    const bool over = zp[0][0] > thr[0] || zp[1][0] > thr[0] || zp[0][1] > thr[1] ||
                      zp[1][1] > thr[1] || smax >= sbound;
    if (first || __ballot(over) != 0ull) {
      float d[G];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float zm = fmaxf(zp[hh][0] - fp[0], zp[hh][1] - fp[1]);
        zm = row16_max(zm);
        const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, zm), 0));
        const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, zm), 16));
        const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, zm), 32));
        const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, zm), 48));
        d[hh] = fmaxf(r0, r2);        // head hh   (rows q = 0, 2)
        d[2 + hh] = fmaxf(r1, r3);    // head 2+hh (rows q = 1, 3)
      }
      const float sv = wave_max(h2f(smax));
      int es_t = -24;
      if (sv > 0.0f) frexpf(sv, &es_t);
      const int es_new = first ? es_t : max(es_run, es_t);
      const int f_new = 15 - (int)kSlack - 24 - es_new;
      const float beta = first ? 1.0f : ldexpf(1.0f, f_new - f_run);
      float al[G], dm[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        dm[h] = first ? d[h] : fmaxf(d[h], 0.0f);
        m_run[h] += dm[h];
        al[h] = first ? 1.0f : exp2f(-dm[h]) * beta;
      }
#pragma unroll
      for (int j = 0; j < L::VG; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          vacc[j][0][i] *= al[i];
          vacc[j][1][i] *= al[i];
          sacc[j][i] *= al[i];
        }
      const float df = (float)(f_new - f_run);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const float a = sel2(hp, al[hh], al[2 + hh]);
        const float dmh = sel2(hp, dm[hh], dm[2 + hh]);
        mr[hh] = sel2(hp, m_run[hh], m_run[2 + hh]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          lacc[hh][nt] *= a;
          zp[hh][nt] += df - dmh;
        }
      }
      f_run = f_new;
      es_run = es_new;
      sbound = pow2_bits(es_new);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        fp[nt] = (float)(f_run + 24 - 2 * pk[nt]);
        thr[nt] = kSlack + fp[nt];
      }
      first = false;
    }

    // ---- numerators -> value A operands (row = head, K = token)
    float p[2][2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        p[hh][nt] = __builtin_amdgcn_exp2f(zp[hh][nt]);
        lacc[hh][nt] += p[hh][nt];
      }
#pragma unroll
    for (int j = 0; j < L::VG; ++j) {
      const uint32_t s0 = (cvs[j >> 1] >> (16 * (j & 1))) & 0xffffu;
      const uint32_t s1 = (cvs[L::VG / 2 + (j >> 1)] >> (16 * (j & 1))) & 0xffffu;
      const float f0 = h2f(s0), f1 = h2f(s1);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        uint16_t *dst = &W.u.t.pbuf[j][pkc][2 * hp + hh][pw][pi0];
        dst[0] = f2h(p[hh][0] * f0);
        dst[2] = f2h(p[hh][1] * f1);
      }
    }
    wave_sync();

    // ---- weighted sum of the value codes
    // rows 4..15 of the value A operand are never read: every lane loads (head n mod 4)
    aval[0] = *reinterpret_cast<const u32x4 *>(&W.u.t.pbuf[0][0][n & 3][q][0]);
#pragma unroll
    for (int kc2 = 0; kc2 < 2; ++kc2) {
#pragma unroll
      for (int j = 0; j < L::VG; ++j) {
        const int step = kc2 * L::VG + j, cur = step & 1;
        if (step + 1 < 2 * L::VG) {
          const int j2 = (step + 1) % L::VG, k2 = (step + 1) / L::VG;
          aval[cur ^ 1] = *reinterpret_cast<const u32x4 *>(&W.u.t.pbuf[j2][k2][n & 3][q][0]);
        }
        sacc[j] = mfma16(aval[cur], unit_k[kc2], sacc[j]);
        vacc[j][0] = mfma16(aval[cur], value_operand(cvw[j].x, kc2), vacc[j][0]);
        vacc[j][1] = mfma16(aval[cur], value_operand(cvw[j].y, kc2), vacc[j][1]);
      }
    }
    wave_sync();
    if (more) commit(tk + kWaves4);
    wave_sync();
  }

  // ---------------------------------------------------------------- merge the wavefronts
  {
    float lh[G];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      float ll = fmaf(lacc[hh][0], ldexpf(1.0f, -(int)fp[0]), lacc[hh][1] * ldexpf(1.0f, -(int)fp[1]));
      ll = row16_sum(ll);
      const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ll), 0));
      const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ll), 16));
      const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ll), 32));
      const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ll), 48));
      lh[hh] = r0 + r2;
      lh[2 + hh] = r1 + r3;
    }
    const float inv_f = ldexpf(1.0f, -f_run);
    if (q == 0) {
#pragma unroll
      for (int j = 0; j < L::VG; ++j)
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            W.u.merge[i][32 * j + 2 * n + e] = (2.0f * vacc[j][e][i] - 3.0f * sacc[j][i]) * inv_f;
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
      if (lane == h) {
        W.mstate[h] = m_run[h];
        W.lstate[h] = ntiles > wave ? lh[h] : 0.0f;
      }
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += kThreads4) {
    const int h = e / D, ch = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves4; ++w)
      if (sm.w[w].lstate[h] > 0.0f) M = fmaxf(M, sm.w[w].mstate[h]);
    float o = 0.0f, Lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves4; ++w) {
      if (sm.w[w].lstate[h] > 0.0f) {
        const float f = exp2f(sm.w[w].mstate[h] - M);
        o = fmaf(sm.w[w].u.merge[h][ch], f, o);
        Lsum = fmaf(sm.w[w].lstate[h], f, Lsum);
      }
    }
    wsp[h * (D + kPartialHead) + kPartialHead + ch] = o;
    if (ch == 0) {
      wsp[h * (D + kPartialHead) + 0] = M;
      wsp[h * (D + kPartialHead) + 1] = Lsum;
    }
  }
}

}  // namespace

hipError_t launch_decode4(const dqk_cache &c, const float *q_prime, const int32_t *sel_idx, int hq,
                          int keep, float scale2, int nsplit, float *ws, hipStream_t s) {
  const int items = c.batch * c.num_kv_heads * nsplit;
  const dim3 grid((unsigned)items), block(kThreads4);
  const bool ksp = c.capacity % 64 == 0;
  if (c.head_dim == 64) {
    if (ksp)
      hipLaunchKernelGGL((decode4_kernel<64, true>), grid, block, 0, s, c, q_prime, sel_idx, hq, keep, scale2, nsplit, ws);
    else
      hipLaunchKernelGGL((decode4_kernel<64, false>), grid, block, 0, s, c, q_prime, sel_idx, hq, keep, scale2, nsplit, ws);
  } else {
    if (ksp)
      hipLaunchKernelGGL((decode4_kernel<128, true>), grid, block, 0, s, c, q_prime, sel_idx, hq, keep, scale2, nsplit, ws);
    else
      hipLaunchKernelGGL((decode4_kernel<128, false>), grid, block, 0, s, c, q_prime, sel_idx, hq, keep, scale2, nsplit, ws);
  }
  return hipGetLastError();
}

}  // namespace dqk
