// Decode attention over the 2-bit cache for GQA groups of four query heads
// (hq / hkv == 4), both contractions on the matrix cores.
//
// Dual-QK (arXiv abstract; tech.dede.sh summary, "Throughput on SGLang"): keys
// and values are stored in 2 bits and the key channels a query head does not
// keep are never read, which is where the decode speedup comes from.  One
// workgroup serves the four query heads of one KV head over an equal share of
// the sequence's 256-token blocks; only the union U of the group's kept key
// channels is read (their 2-bit rows are channel-major, so a dropped channel
// costs no bytes), together with channel 0's fp16 row and, for the unfinished
// last group, the exact tail.  Each head's logit uses only its own channels (its
// coefficient is zero on the others).  Values are never pruned.
//
// Memory pipeline.  A block is 256 tokens of one (batch row, KV head): the key
// code rows of U, their scales, channel 0, the value words and the value
// scales, about 20 KB at head_dim 128.  Every lane of the workgroup issues the
// same fixed set of buffer loads for a block (lanes without a part of it point
// past the plane, which returns zero and moves no bytes); two blocks are in
// flight in registers while a third is computed from LDS.  A block's registers
// are written to one of two LDS buffers (key codes transposed into the operand
// order of the logit product) and one workgroup barrier per block publishes it.
// Wavefront w then computes the block's 64-token tile w.
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
//    each group); B[(g, s)][t] = u_{s,t} 2^(2k-24) with k = 3 or 4 (the codes are
//    shifted to mantissa bits 6-9 first); a product with B = 1 gives C1 = sum A.
//    Then z = 2^(E_h + 25 - 2k) (C_high + C_low) - 3 2^E_h (C1_high + C1_low) + ch0 term.
//  - values, per 32 tokens and 16 channels of value group j: A[h][t] =
//    p_{h,t} scale_{t,j} 2^(F + 24 - 2k(t)) in fp16 (p the softmax numerator, F a
//    power of two that keeps A finite), B[t][c] = u 2^(2k-24); a product with
//    B = 2^(2k-24) gives S = 2^F sum p scale, and out = 2^-F (2 C - 3 S).
// Softmax: each wavefront keeps a running maximum per head that may trail the
// largest logit seen by up to 8 (log2 units); it moves, and the running sums
// are rescaled, only when a logit exceeds it by more than that or a value scale
// outgrows the range that 2^F allows.
//
// The capacity must be a multiple of 64 tokens (the key scales of a block are
// then whole dwords of every scale row); other capacities use the general
// decode kernel.
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
constexpr int kBlock4 = kTile4 * kWaves4;   // tokens per workgroup block
constexpr int kKsPerBlock = kBlock4 / kGroup;   // key groups per block
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
  static constexpr int VCH = 4 * D;     // 16-byte value chunks per block (16 rows of D words)
  static constexpr int SCH = D;         // 16-byte value-scale chunks per block
  static constexpr int KSD = D / 64;    // key-scale dwords per lane per block (4 per slot)
};

// One 256-token block as staged in LDS.
template <int D>
struct __attribute__((aligned(16))) Block4 {
  uint32_t y[kWaves4][Lay4<D>::OCT][16][2];   // key codes: tile, slot octet, token quad, slots 0-3 | 4-7
  uint16_t ksig[kKsPerBlock][D];              // key scales (fp16 bits): key group of the block, slot
  uint32_t vw[16][D];                         // value words: 16-token row of the block, channel
  // 16-byte chunk i of this region is written by lane i: the value scales (fp16
  // bits, [token][value group]), then key channel 0 (fp16 bits), then chunks no
  // part of the block needs (lanes without such a part write there)
  union {
    u32x4 chunk[kThreads4];
    struct {
      uint16_t vs[kBlock4][Lay4<D>::VG];
      uint16_t c0[kBlock4];
    } m;
  } misc;
};

template <int D>
struct __attribute__((aligned(16))) WaveSmem4 {
  union {
    struct {
      uint16_t abuf[16][Lay4<D>::AROW];           // logit A rows 8g+2h+limb, slots in octet order 0,2,1,3,4,6,5,7
      uint16_t pbuf[Lay4<D>::VG][2][kG4][4][8];   // value A: group j, K chunk, head, word, K position
    } t;
    float merge[kG4][D];                          // the wavefront's output at the end of the split
  } u;
  float mstate[kG4], lstate[kG4];
};

template <int D>
struct __attribute__((aligned(16))) Smem4 {
  Block4<D> blk[2];
  WaveSmem4<D> w[kWaves4];
  float coefc[kG4][D];     // q' * sm * log2(e) by channel (0 where the head drops the channel)
  float coefs[kG4][D];     // coefc in union-slot order * 2^-E_h (0 past |U|)
  float e2[kG4];           // 2^E_h
  float redm[kG4][kWaves4];
  int hmask[D];
  int16_t ulist[D];
  int wcount[2];
};

// Registers of one block in flight.
template <int D>
struct Stage4 {
  uint32_t kc[8];          // key codes: 8 slots x 16 tokens
  u32x4 vw[2];             // value words: two 16-byte chunks
  u32x4 vs;                // value scales: one 16-byte chunk
  uint32_t ks[Lay4<D>::KSD];       // key scales: dwords (two groups of one slot each)
  u32x4 c0;                // channel 0: one 16-byte chunk
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

// KSP: 2-byte loads are not needed for the key scales of a block (a key scale row
// starts on a dword boundary).  The kernel is only launched with capacity % 64 == 0,
// where this holds; KSP=false loads the scales as 16-bit halves.
template <int D>
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
  const int nblk_all = (len + kBlock4 - 1) / kBlock4;
  const int blo = (int)(((long long)s * nblk_all) / nsplit);
  const int bhi = (int)(((long long)(s + 1) * nblk_all) / nsplit);
  const int t_begin = blo * kBlock4;
  const int t_end = min(bhi * kBlock4, len);
  const int nb = bhi - blo;
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

  // ---------------------------------------------------------------- block loads (every lane)
  // Loads go through buffer resources of the unit's planes whose base is moved
  // to the block (scalar arithmetic; the per-lane offsets stay fixed): an offset
  // past the resource returns zero, so absent parts point past the end (kFar)
  // and a block past the end gets an empty resource.
  const uint32_t kc_bytes = (uint32_t)(D * kc_stride), ks_bytes = (uint32_t)(D * ks_stride * 2);
  const uint32_t c0_bytes = (uint32_t)(c.capacity * 2), vw_bytes = (uint32_t)((c.capacity / 16) * D * 4);
  const uint32_t vs_bytes = (uint32_t)(c.capacity * L::VG * 2);

  // Every lane has one job of each kind, so that no write to LDS depends on the
  // lane; at head_dim 64 the upper lanes repeat the key-code and value jobs of
  // the lower ones (the same bytes to the same place).
  // key codes: slot octet lo, 16-token quarter lq of the block; 8 slots x 4 bytes
  const int lo = (tid >> 4) % L::OCT, lq = tid & 15;
  uint32_t kvo[8];
#pragma unroll
  for (int cc = 0; cc < 8; ++cc) {
    const int i = 8 * lo + cc;
    kvo[cc] = i < nu ? (uint32_t)(sm.ulist[i] * kc_stride) + 4u * lq : kFar;
  }
  // key scales: dword jobs j = tid (+ 256): slot j / 4, groups 2(j % 4), +1 of the block
  constexpr int KSD = L::KSD;
  uint32_t ksv[KSD];
#pragma unroll
  for (int k = 0; k < KSD; ++k) {
    const int j = tid + kThreads4 * k;
    const int sl = j >> 2;
    ksv[k] = sl < nu ? (uint32_t)(sm.ulist[sl] * ks_stride * 2) + 4u * (j & 3) : kFar;
  }
  // value words: 16-byte chunks tid, tid + 256 of the block's 16 rows of D words
  int vch[2];
  uint32_t vwo[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    vch[k] = (tid + kThreads4 * k) % L::VCH;
    vwo[k] = (uint32_t)((vch[k] / (D / 4)) * D * 4 + (vch[k] % (D / 4)) * 16);
  }
  // value scales (lanes below SCH) or channel 0 (the next 32 lanes): chunk tid of misc
  constexpr int C0CH = kBlock4 * 2 / 16;
  const uint32_t vso = tid < L::SCH ? 16u * tid : kFar;
  const uint32_t c0o = (tid >= L::SCH && tid < L::SCH + C0CH) ? 16u * (tid - L::SCH) : kFar;

  // Every call issues the same loads, also for blocks past the end (they point
  // past the planes): the count of loads in flight is then the same on every
  // path, and the waits before a block's registers are used stay partial.
  auto rsrc = [&](const void *base, uint32_t bytes, uint32_t off, bool live) {
    // off < bytes for every live block (p0 < len <= capacity)
    return __builtin_amdgcn_make_buffer_rsrc((void *)((const char *)base + (live ? off : 0u)), (short)0,
                                             live ? (int)(bytes - off) : 0, kRsrcWord3);
  };
  auto issue = [&](Stage4<D> &S, int bk) {
    __builtin_amdgcn_sched_barrier(0);
    const bool live = bk < nb;
    const uint32_t p0 = (uint32_t)(t_begin + kBlock4 * bk);
    const auto rk = rsrc(kcodes, kc_bytes, p0 >> 2, live);
    const auto rks = rsrc(kscales, ks_bytes, (p0 / kGroup) * 2u, live);
    const auto rc0 = rsrc(c0row, c0_bytes, p0 * 2u, live);
    const auto rvw = rsrc(vwords, vw_bytes, (p0 >> 4) * (uint32_t)(D * 4), live);
    const auto rvs = rsrc(vscales, vs_bytes, p0 * (uint32_t)(L::VG * 2), live);
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) S.kc[cc] = __builtin_amdgcn_raw_buffer_load_b32(rk, kvo[cc], 0, 0);
#pragma unroll
    for (int k = 0; k < 2; ++k)
      S.vw[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rvw, vwo[k], 0, 0));
    S.vs = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rvs, vso, 0, 0));  // zero past the plane
#pragma unroll
    for (int k = 0; k < KSD; ++k) S.ks[k] = __builtin_amdgcn_raw_buffer_load_b32(rks, ksv[k], 0, 0);
    S.c0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc0, c0o, 0, 0));
    // keep the blocks' loads in issue order: a block's loads must all be older
    // than the next block's for the partial waits above to apply
    __builtin_amdgcn_sched_barrier(0);
  };

  auto commit = [&](Stage4<D> &S, Block4<D> &B, int bk) {
    const int p0 = t_begin + kBlock4 * bk;
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
      u32x4 *dst = reinterpret_cast<u32x4 *>(&B.y[lq >> 2][lo][4 * (lq & 3)][0]);
      dst[0] = u32x4{y0[0], y1[0], y0[1], y1[1]};
      dst[1] = u32x4{y0[2], y1[2], y0[3], y1[3]};
    }
    // key scales of a key group past the coded range (the exact tail or beyond) stay zero
#pragma unroll
    for (int k = 0; k < KSD; ++k) {
      const int j = tid + kThreads4 * k;
      const int sl = j >> 2, gp = 2 * (j & 3);
      const int g0 = p0 / kGroup + gp;
      const uint32_t v = S.ks[k];
      B.ksig[gp][sl] = g0 * kGroup < code_end ? (uint16_t)v : (uint16_t)0;
      B.ksig[gp + 1][sl] = (g0 + 1) * kGroup < code_end ? (uint16_t)(v >> 16) : (uint16_t)0;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k)
      *reinterpret_cast<u32x4 *>(&B.vw[vch[k] / (D / 4)][(vch[k] % (D / 4)) * 4]) = S.vw[k];
    // at most one of the two is not zero (the other load pointed past its plane)
    B.misc.chunk[tid] = S.vs | S.c0;
  };

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

  // logit output: tokens 32lg + 2n + nt (nt = 0, 1), token position r0 + nt in its quad with
  // r0 = 2(n&1).  Both codes of a lane are first shifted inside each fp16 half so
  // that token r0 sits at bits 6-7 and token r0+1 at bits 8-9: the matrix cores
  // accumulate products whose fp16 operand is a deep subnormal (codes at bits 0-5)
  // with visibly less than fp32 accuracy, while from 2^-18 upward they do not.
  const uint32_t shl2 = (uint32_t)(6 - 4 * (n & 1)) * 0x00010001u;   // low byte of each half
  const uint32_t shr2 = (uint32_t)(2 + 4 * (n & 1)) * 0x00010001u;   // high byte of each half
  float ez[2][2], n3e[2], c0c[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int h = 2 * hp + hh;
    const float e = sm.e2[h];
    n3e[hh] = -3.0f * e;
    c0c[hh] = sm.coefc[h][0];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) ez[hh][nt] = ldexpf(e, 25 - 2 * (3 + nt));
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

  // ---------------------------------------------------------------- one tile of one block
  auto compute = [&](const Block4<D> &B, int bk) {
    const int tile0 = t_begin + kBlock4 * bk + kTile4 * wave;
    if (tile0 >= t_end) return;

    // ---- logit A operands of the tile's two key groups (compact build)
    {
      const u32x4 *src = reinterpret_cast<const u32x4 *>(&B.ksig[2 * wave + ab_g][ab_s]);
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
          uint32_t hh, ll;
          if (ta & 1) {
            hh = mixhi<1>(mixlo<1>(ca, sa), cb, sb);
            ll = reshi<1, 1>(reslo<1, 0>(ca, sa, hh), cb, sb, hh);
          } else {
            hh = mixhi<0>(mixlo<0>(ca, sa), cb, sb);
            ll = reshi<0, 1>(reslo<0, 0>(ca, sa, hh), cb, sb, hh);
          }
          hw[pr] = hh;
          lw[pr] = ll;
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
        dd[0] = *reinterpret_cast<const u32x2 *>(&B.y[wave][q & 1][8 * lg + (n >> 1)][0]);
      }
#pragma unroll
      for (int kc = 0; kc < L::NKC; ++kc) {
        if (kc < nkc) {
          const int cur = kc & 1, nxt = cur ^ 1;
          if (kc + 1 < L::NKC && kc + 1 < nkc) {
            if (arow) alog[nxt] = *reinterpret_cast<const u32x4 *>(&W.u.t.abuf[n][16 * (kc + 1) + 8 * (q & 1)]);
            dd[nxt] = *reinterpret_cast<const u32x2 *>(&B.y[wave][2 * (kc + 1) + (q & 1)][8 * lg + (n >> 1)][0]);
          }
          const uint32_t l0 = pk_shl16(dd[cur].x, shl2), h0 = pk_shr16(dd[cur].x, shr2);
          const uint32_t l1 = pk_shl16(dd[cur].y, shl2), h1 = pk_shr16(dd[cur].y, shr2);
          constexpr uint32_t M3 = 0x00C000C0u, M4 = 0x03000300u;
          const u32x4 b0 = {l0 & M3, h0 & M3, l1 & M3, h1 & M3};   // token r0: u 2^-18
          const u32x4 b1 = {l0 & M4, h0 & M4, l1 & M4, h1 & M4};   // token r0+1: u 2^-16
          acc0 = mfma16(alog[cur], b0, acc0);
          acc1 = mfma16(alog[cur], b1, acc1);
          accs = mfma16(alog[cur], ones, accs);
        }
      }
    }

    // ---- this tile's channel 0, value scales and value words from the block
    const int tt = kTile4 * wave + 32 * lg + 2 * n;   // my first token within the block
    const uint32_t cx0 = *reinterpret_cast<const uint32_t *>(&B.misc.m.c0[tt]);
    uint32_t cvs[L::VG];
    {
      // value scales of tokens past the split end are zero (their numerators are zero too)
      const int t0 = tile0 + 32 * lg + 2 * n;
      const uint32_t m0 = t0 < t_end ? 0xffffffffu : 0u, m1 = t0 + 1 < t_end ? 0xffffffffu : 0u;
      if constexpr (L::VG == 4) {
        const u32x4 x = *reinterpret_cast<const u32x4 *>(&B.misc.m.vs[tt][0]);
        cvs[0] = x.x & m0; cvs[1] = x.y & m0; cvs[2] = x.z & m1; cvs[3] = x.w & m1;
      } else {
        const u32x2 x = *reinterpret_cast<const u32x2 *>(&B.misc.m.vs[tt][0]);
        cvs[0] = x.x & m0; cvs[1] = x.y & m1;
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
      // the value scale of token nt, group j is half (j & 1) of cvs[nt * VG/2 + j/2]
      const uint32_t s0 = cvs[j >> 1], s1 = cvs[L::VG / 2 + (j >> 1)];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        uint16_t *dst = &W.u.t.pbuf[j][pkc][2 * hp + hh][pw][pi0];
        if (j & 1) {
          dst[0] = (uint16_t)mixlo<1>(p[hh][0], s0);
          dst[2] = (uint16_t)mixlo<1>(p[hh][1], s1);
        } else {
          dst[0] = (uint16_t)mixlo<0>(p[hh][0], s0);
          dst[2] = (uint16_t)mixlo<0>(p[hh][1], s1);
        }
      }
    }
    wave_sync();

    // ---- weighted sum of the value codes
    // rows 4..15 of the value A operand are never read: every lane loads (head n mod 4)
    u32x2 cvw[L::VG];
#pragma unroll
    for (int j = 0; j < L::VG; ++j)
      cvw[j] = *reinterpret_cast<const u32x2 *>(&B.vw[4 * wave + q][32 * j + 2 * n]);
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
  };

  // ---------------------------------------------------------------- block pipeline
  // Two blocks in flight in registers; block bk is written to LDS buffer bk & 1
  // once its loads have landed, published by one barrier, then computed.  The
  // barrier of block bk also tells every wavefront that block bk - 1, which
  // used the other buffer, has been computed by all of them.
  // Blocks go in pairs; a block past the end is all zeros and computes nothing.
  Stage4<D> S0, S1;
  issue(S0, 0);
  issue(S1, 1);
  for (int bk = 0; bk < nb; bk += 2) {
    commit(S0, sm.blk[0], bk);
    issue(S0, bk + 2);
    block_barrier();
    compute(sm.blk[0], bk);
    commit(S1, sm.blk[1], bk + 1);
    issue(S1, bk + 3);
    block_barrier();
    compute(sm.blk[1], bk + 1);
  }
  // the loads of the two blocks past the end (they return zeros) land before the merge
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---------------------------------------------------------------- merge the wavefronts
  const bool had = t_begin + kTile4 * wave < t_end;   // this wavefront computed a tile
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
        W.lstate[h] = had ? lh[h] : 0.0f;
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

bool decode4_supported(const dqk_cache &c) { return c.capacity % 64 == 0; }

hipError_t launch_decode4(const dqk_cache &c, const float *q_prime, const int32_t *sel_idx, int hq,
                          int keep, float scale2, int nsplit, float *ws, hipStream_t s) {
  const int items = c.batch * c.num_kv_heads * nsplit;
  const dim3 grid((unsigned)items), block(kThreads4);
  if (c.head_dim == 64)
    hipLaunchKernelGGL((decode4_kernel<64>), grid, block, 0, s, c, q_prime, sel_idx, hq, keep, scale2, nsplit, ws);
  else
    hipLaunchKernelGGL((decode4_kernel<128>), grid, block, 0, s, c, q_prime, sel_idx, hq, keep, scale2, nsplit, ws);
  return hipGetLastError();
}

}  // namespace dqk
