// Decode attention over the 2-bit cache for GQA groups of four query heads
// (hq / hkv == 4), both contractions on the matrix cores.
//
// Dual-QK (arXiv abstract; tech.dede.sh summary, "Throughput on SGLang"): keys
// and values are stored in 2 bits and the key channels a query head does not
// keep are never read, which is where the decode speedup comes from.  One
// workgroup serves the four query heads of one KV head over a share of the
// sequence's 256-token blocks; only the union U of the group's kept key channels
// is read (their 2-bit rows are channel-major, so a dropped channel costs no
// bytes; with per-head kept sets the workgroup's first block, issued before U is
// known, reads every channel, while a group-shared set is read first and packed
// into the first slots), together with channel 0's fp16 row and, for the
// unfinished last group, the exact tail.  Each head's logit uses only its own
// channels (its coefficient is zero on the others).  Values are never pruned.
// The workgroup leaves its partial (m, l, o) per head for the combine, or, when
// a row has a single split, the normalized output itself.
//
// Two passes per chunk of up to ten blocks (2560 tokens):
//  1. keys.  Every lane of the workgroup issues the same fixed set of buffer
//     loads for a block (lanes without a part of it point past the plane, which
//     returns zero and moves no bytes); two blocks are in flight in registers
//     while a third is worked on.  A block's key codes are written to one of two
//     LDS buffers, transposed into the operand order of the logit product, and
//     one workgroup barrier per block publishes them.  Wavefront w computes the
//     logits of the block's 64-token tile w and keeps them in registers.
//  2. values.  With the exact maximum of its logits in the chunk known, every
//     wavefront streams the value words and scales of its own tiles straight
//     into registers (three tiles in flight, no barrier) and accumulates the
//     weighted sum.  Only a later chunk with a larger maximum rescales what was
//     accumulated.
//
// Decoding.  A 2-bit code u whose bit pair sits at bits 2k, 2k+1 of an fp16 word
// with a zero exponent field is the subnormal u * 2^(2k-24), exact; masking a
// packed code word therefore yields two operands per instruction, and the power
// 2^(2k-24) is compensated in the other operand or in the output.  The matrix
// cores take fp16 subnormals as they are.  With the level 2u - 3 of a code:
//  - logits, per 64-token tile with key groups g = 0, 1: A[(g, h, limb)][(g, s)]
//    is the fp16 high or low part of q'_{h,U[s]} * sm * log2(e) * scale_{U[s],g}
//    * 2^-E_h, block diagonal over g (rows 8g + 2h + limb, K = 16 union slots of
//    each group); B[(g, s)][t] = u_{s,t} 2^(2k-24) with k = 3 or 4 (the codes are
//    shifted to mantissa bits 6-9 first); a product with B = 1 gives C1 = sum A.
//    Then z = 2^(E_h + 25 - 2k) (C_high + C_low) - 3 2^E_h (C1_high + C1_low) + ch0 term.
//  - values, per 32 tokens and 16 channels of value group j: A[h][t] =
//    p_{h,t} scale_{t,j} 2^(F + 24 - 2k(t)) in fp16 (p = 2^(z - max) <= 1, F a
//    power of two that keeps A below 2^15), B[t][c] = u 2^(2k-24); beside the
//    product, mixed-precision FMAs sum S = 2^F sum p scale from the same fp16
//    operands, and out = 2^-F (2 C - 3 S).
//    F moves (and what was accumulated is rescaled by a power of two) only when
//    a value scale outgrows the range it allows.
//
// The capacity must be a multiple of 64 tokens (the key scales of a block are
// then whole dwords of every scale row); other capacities use the general
// decode kernel.
#include <atomic>

#include "dqk_decode_ops.h"

namespace dqk {
namespace {

using namespace wave;
using namespace dops;

constexpr int kG4 = 4;              // query heads per workgroup: the KV head's group
constexpr int kThreads4 = 256;
constexpr int kWaves4 = kThreads4 / 64;
constexpr int kTile4 = 64;          // tokens per wavefront tile: two key groups
constexpr int kBlock4 = kTile4 * kWaves4;   // tokens per workgroup block
constexpr int kChunk4 = kDecodeChunkBlocks;   // blocks per chunk: logits of a chunk stay in registers
// one block more than a chunk runs as one chunk: the extra block is committed to
// LDS buffer kChunk4 & 1 and its values use stage kChunk4 % 3 (blocks alternate
// over the two buffers and the value tiles over three stages)

template <int D>
struct Lay4 {
  static constexpr int OCT = D / 8;     // union-slot octets
  static constexpr int NKC = D / 16;    // logit K chunks (16 slots of each key group)
  static constexpr int VG = D / 32;     // value scale groups
  static constexpr int AROW = D + 8;    // fp16 per logit A row (padded against bank conflicts)
  static constexpr int SPJ = D / 2;     // logit A jobs (union-slot pair, key-group pair) per block / 4
  static constexpr int NH = D / 64;     // 64-channel halves of the weighted sum
};

// The keys of one 256-token block as staged in LDS.
template <int D>
struct __attribute__((aligned(16))) KBlock4 {
  uint32_t y[kWaves4][Lay4<D>::OCT][16][2];   // key codes: tile, slot octet, token quad, slots 0-3 | 4-7
  // logit A operands of tile w: rows 8g + 2h + limb (key group g of the tile,
  // head h, fp16 high/low part), slots in octet order 0,2,1,3,4,6,5,7.  The
  // tiles are 8 dwords apart modulo the 32 LDS banks, so that the four tiles
  // of one A-building write land in different banks.
  struct {
    uint16_t r[16][Lay4<D>::AROW];
    uint16_t pad[16];
  } a[kWaves4];
  uint32_t c0w[kThreads4];                    // key channel 0: fp16 pair of tokens 2i, 2i+1 (i < 128)
};

template <int D>
struct __attribute__((aligned(16))) WaveSmem4 {
  u32x4 zero;   // a 16-byte zero operand
  union {
    struct {
      // value A: group j, K chunk kc, then word w, head h, 8 K positions at
      // ((w * 4 + h) * 8 + k); each (j, kc) slab is padded by 4 dwords so that
      // neither the 2-byte writes nor the 16-byte reads meet in an LDS bank
      uint16_t pbuf[Lay4<D>::VG][2][4 * kG4 * 8 + 8];
    } t;
    float merge[kG4][D];                          // the wavefront's output at the end of the split
  } u;
  float mstate[kG4], lstate[kG4];
};

template <int D>
struct __attribute__((aligned(16))) Smem4 {
  KBlock4<D> kb[2];
  WaveSmem4<D> w[kWaves4];
  float coefc[kG4][D];     // q' * sm * log2(e) by channel (0 where the head drops the channel)
  float coefs[kG4][D];     // coefc in union-slot order * 2^-E_h (0 past |U|)
  float e2[kG4];           // 2^E_h
  float redm[kG4][2];         // largest |coefficient| per head and 64-channel half
  float tailz[kG4][kGroup];   // exact logits of the unfinished last key group
  union {
    uint8_t b[kG4][D];        // kept[h][c]: head h keeps channel c
    uint32_t w[kG4 * D / 4];
  } kept;
  unsigned long long umask[2];   // the union U of kept key channels >= 1: bit c of word c / 64
  int32_t ulist[D];              // compact slots: key channel of slot i (-1 past |U|)
};

// Registers of one block of keys in flight.
template <int D>
struct KStage4 {
  uint32_t kc[8];              // key codes: 8 slots x 16 tokens
  uint32_t ks[2];              // key scales of two slots: dwords (two groups each)
  uint32_t c0;                 // channel 0: two tokens
};

// Registers of one tile of values in flight (one wavefront).
template <int D>
struct VStage4 {
  uint32_t vw[Lay4<D>::NH][4];   // value words of channel 64 half + 16q + n, word rows 0-3 of the tile
  uint32_t vs[Lay4<D>::VG];      // value scales of tokens t, t+1: [t groups | t+1 groups]
};

// COMPACT (group-shared kept sets, one per KV head): union slot i holds the
// i-th kept key channel other than 0, so the slots past |U| = keep - 1 fill
// only the last of the nkc K chunks that are worked on; otherwise slot i holds
// channel i + 1 and all K chunks run.
template <int D, bool COMPACT>
__global__ __launch_bounds__(kThreads4, 2) void decode4_kernel(dqk_cache c,
                                                               const float *__restrict__ qp,
                                                               const int32_t *__restrict__ sel,
                                                               int shared, int hq, int grid3, int keep,
                                                               float scale2, int nsplit, int bps, int ncu_q,
                                                               int ncu_r, int nkc, float *__restrict__ ws,
                                                               float *__restrict__ out) {
  using L = Lay4<D>;
  constexpr int G = kG4;
  __shared__ Smem4<D> sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: block and tile offsets stay scalar
  // Work item (unit, split s) in split-major order: workgroups of one split index
  // run together.  The grid is (KV head, row, split) where it fits (grid3), so
  // that the linear workgroup id is the item s * units + unit and no division
  // stands between the start and the length load; otherwise it is
  // one-dimensional over the items.
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
  // The group's q' rows (all channels) and kept-channel lists are loaded before
  // anything waits, in parallel with the length: one round trip for the setup.
  const size_t row0 = (size_t)b * hq + (size_t)g * G;
  constexpr int SJ = (G * D) / kThreads4;   // elements per lane
  float qv[SJ];
  int sv[SJ];
#pragma unroll
  for (int k = 0; k < SJ; ++k) {
    const int e = tid + kThreads4 * k;
    qv[k] = qp[row0 * D + e];
    // the head's kept set: its own row, or its KV head's shared one (position
    // e mod keep, by subtraction: e < G keep)
    int es = e;
#pragma unroll
    for (int h = 1; h < G; ++h) es = es >= keep ? es - keep : es;
    sv[k] = e < G * keep ? (shared ? sel[(size_t)unit * keep + es] : sel[row0 * keep + e]) : -1;
  }
  // compact slots: the shared kept list without channel 0, one slot per lane
  int uch = -1;
  if constexpr (COMPACT) {
    if (tid < D && tid + 1 < keep) uch = sel[(size_t)unit * keep + tid + 1];
  }
  const int nblk_all = (len + kBlock4 - 1) / kBlock4;
  // bps > 0: split s is blocks [s bps, (s + 1) bps) of the row.  Else the row's
  // blocks are shared out over the nsplit splits: evenly, or, when two workgroups
  // share each compute unit (ncu = ncu_q * units + ncu_r > 0: the number of
  // compute units, workgroup ids below it being the first on their unit),
  // unevenly (uneven_shares).
  int blo, bhi;
  {
    // first-slot splits: items s * units + unit below ncu
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
  const int t_begin = blo * kBlock4;
  const int t_end = min(bhi * kBlock4, len);
  const int nb = bhi - blo;
  float *wsp = ws + ((size_t)unit * nsplit + s) * G * (D + kPartialHead);
  // out != nullptr: a single split per row, whose normalized output is written
  // directly (what the combine makes of one partial); an empty row gives zeros
  float *outp = out ? out + row0 * D : nullptr;
  if (t_begin >= t_end) {
    if (outp) {
      for (int e = tid; e < G * D; e += kThreads4) outp[e] = 0.0f;
    } else {
      for (int e = tid; e < G * (D + kPartialHead); e += kThreads4)
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

  // Loads go through buffer resources of the unit's planes whose base is moved
  // to the block or tile (scalar arithmetic; the per-lane offsets stay fixed):
  // an offset past the resource returns zero, so absent parts point past the
  // end (kFar) and a block past the end gets an empty resource.
  const uint32_t kc_bytes = (uint32_t)(D * kc_stride), ks_bytes = (uint32_t)(D * ks_stride * 2);
  const uint32_t c0_bytes = (uint32_t)(c.capacity * 2), vw_bytes = (uint32_t)((c.capacity / 16) * D * 4);
  const uint32_t vs_bytes = (uint32_t)(c.capacity * L::VG * 2);
  auto rsrc = [&](const void *base, uint32_t bytes, uint32_t off, bool live) {
    // off < bytes for every live block or tile (its first token is below len <= capacity)
    return __builtin_amdgcn_make_buffer_rsrc((void *)((const char *)base + (live ? off : 0u)), (short)0,
                                             live ? (int)(bytes - off) : 0, kRsrcWord3);
  };

  // Rows of the unfinished last key group, only in the workgroup that reaches it
  // (elsewhere the resource is empty and the loads move no bytes): issued before
  // the key blocks, so that staging them waits for nothing else.
  const bool has_tail = t_body < t_end;
  constexpr int TJ = kGroup * D / (4 * kThreads4);   // float4 per lane
  f32x4 tv[TJ];
  {
    const auto rt = rsrc(tail, (uint32_t)(kGroup * D * 4), 0u, has_tail);
#pragma unroll
    for (int k = 0; k < TJ; ++k)
      tv[k] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rt, 16u * (tid + kThreads4 * k), 0, 0));
  }

  // ---------------------------------------------------------------- key loads (every lane)
  // Union slot i holds key channel i + 1 (the last slot is empty), so the layout
  // of a block does not depend on the selection: the first block is issued for
  // every channel as soon as the length is known, and its latency overlaps the
  // setup below.  Once the union U of the group's kept channels is known, the
  // channels outside it point past the plane (zero codes, no bytes) for the later
  // blocks; their coefficients are zero, so the extra bytes of the first block
  // change no result.
  // Every lane has one job of each kind, so that no write to LDS depends on the
  // lane; at head_dim 64 the upper lanes repeat the key-code jobs of the lower
  // ones (the same bytes to the same place).
  // key codes: slot octet lo, 16-token quarter lq of the block; 8 slots x 4 bytes
  // Offsets in 32-bit arithmetic (a plane of a unit is below 4 GiB).  The products
  // are kept apart from the additions: fused, they become a 64-bit multiply-add
  // whose unused high addend may be any register, also one a setup load is still
  // writing, and the key loads would then wait for that load.
  auto mul_apart = [](uint32_t a, uint32_t b) {
    uint32_t p = a * b;
    asm volatile("" : "+v"(p));
    return p;
  };
  const int lo = (tid >> 4) % L::OCT, lq = tid & 15;
  const uint32_t kc_row = (uint32_t)kc_stride, ks_row = 2u * (uint32_t)ks_stride;
  // logit A operands, built here from the key scales: job j (one per lane; the
  // upper lanes repeat the lower ones at head_dim 64) is key-group pair gp = tile
  // j % 4 of the block and union slots s0 = 8o + a, s1 = s0 + 2 (a = 0, 1, 4, 5),
  // which sit side by side in the octet order of the A rows
  const int aj = tid % (4 * L::SPJ), agp = aj & 3, asp = aj >> 2;
  const int aoct = asp >> 2, am = asp & 3;
  const int as0 = 8 * aoct + (am & 1) + 4 * (am >> 1), as1 = as0 + 2;
  // a wavefront's key-code and A jobs are the 32 slots from 32 (wave mod OCT/4) on:
  // with compact slots, a wavefront whose slots all lie past the nkc chunks has
  // none to read or build (workgroup- and wavefront-uniform)
  const bool slots_live = !COMPACT || 32 * (wave % (L::OCT / 4)) < 16 * nkc;
  // channel of a slot: i + 1, or the compact list (LDS, filled in the setup)
  auto slot_channel = [&](int i) -> int {
    if constexpr (COMPACT) return sm.ulist[i];
    else return i + 1 < D ? i + 1 : -1;
  };
  uint32_t kvo[8], ksv[2];
  auto job_offsets = [&]() {
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const int ch = slot_channel(8 * lo + cc);
      kvo[cc] = ch >= 0 && slots_live ? mul_apart((uint32_t)ch, kc_row) + 4u * (uint32_t)lq : kFar;
    }
    const int c0a = slot_channel(as0), c1a = slot_channel(as1);
    ksv[0] = c0a >= 0 && slots_live ? mul_apart((uint32_t)c0a, ks_row) + 4u * (uint32_t)agp : kFar;
    ksv[1] = c1a >= 0 && slots_live ? mul_apart((uint32_t)c1a, ks_row) + 4u * (uint32_t)agp : kFar;
  };
  if constexpr (!COMPACT) job_offsets();
  // channel 0: dword tid (tokens 2 tid, 2 tid + 1) for the lower 128 lanes
  const uint32_t c0o = tid < kBlock4 / 2 ? 4u * tid : kFar;

  // Every call issues the same loads, also for blocks past the end: the count of
  // loads in flight is then the same on every path, and the waits before a
  // block's registers are used stay partial.
  auto kissue = [&](KStage4<D> &S, int p0, bool live) {
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t u0 = (uint32_t)p0;
    const auto rk = rsrc(kcodes, kc_bytes, u0 >> 2, live);
    const auto rks = rsrc(kscales, ks_bytes, (u0 / kGroup) * 2u, live);
    const auto rc0 = rsrc(c0row, c0_bytes, u0 * 2u, live);
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) S.kc[cc] = __builtin_amdgcn_raw_buffer_load_b32(rk, kvo[cc], 0, 0);
#pragma unroll
    for (int k = 0; k < 2; ++k) S.ks[k] = __builtin_amdgcn_raw_buffer_load_b32(rks, ksv[k], 0, 0);
    S.c0 = __builtin_amdgcn_raw_buffer_load_b32(rc0, c0o, 0, 0);
    // keep the blocks' loads in issue order: a block's loads must all be older
    // than the next block's for the partial waits to apply
    __builtin_amdgcn_sched_barrier(0);
  };

  const int nbc0 = nb == kChunk4 + 1 ? kChunk4 + 1 : min(kChunk4, nb);
  KStage4<D> S0, S1;
  if constexpr (!COMPACT) kissue(S0, t_begin, 0 < nbc0);

  // ---------------------------------------------------------------- setup (whole workgroup)
  // Barriers here order LDS only (block_barrier): a full __syncthreads would also
  // wait for the blocks just issued.
  for (int e = tid; e < G * D / 4; e += kThreads4) sm.kept.w[e] = 0u;
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
    const int e = tid + kThreads4 * k;
    if (e < G * keep && sv[k] >= 0 && sv[k] < D) sm.kept.b[e / keep][sv[k]] = 1;
  }
  block_barrier();
#pragma unroll
  for (int k = 0; k < SJ; ++k) {
    // head h and half of element e are the same for the whole wavefront
    const int e = tid + kThreads4 * k, h = e / D, ch = e % D;
    const float cv = sm.kept.b[h][ch] ? qv[k] * scale2 : 0.0f;
    sm.coefc[h][ch] = cv;
    const float mx = wave_max(ch >= 1 ? fabsf(cv) : 0.0f);   // largest |coefficient| over channels >= 1
    if (lane == 0) sm.redm[h][ch / 64] = mx;
  }
  {
    // the union U: bit c of umask for key channel c >= 1 kept by some head of the group
    const bool f = tid >= 1 && tid < D &&
                   (sm.kept.b[0][tid % D] | sm.kept.b[1][tid % D] | sm.kept.b[2][tid % D] | sm.kept.b[3][tid % D]);
    const unsigned long long m = __ballot(f);
    if (lane == 0 && wave < 2) sm.umask[wave] = m;
  }
  // Tail rows to LDS (the key block buffers are free until the first block),
  // padded to D + 4 floats so that the rows of a wavefront's lanes fall in
  // different banks.
  constexpr int TS = D + 4;
  static_assert(sizeof(sm.kb[0]) >= sizeof(float) * kGroup * TS, "tail rows fit a key block buffer");
  float *trow = reinterpret_cast<float *>(&sm.kb[0]);
  if (has_tail) {
#pragma unroll
    for (int k = 0; k < TJ; ++k) {
      const int e = 4 * (tid + kThreads4 * k);
      *reinterpret_cast<f32x4 *>(trow + (e / D) * TS + e % D) = tv[k];
    }
  }
  block_barrier();
  // Tokens of the unfinished last key group: exact logits from the fp32 tail
  // keys, one per (head, token).  Every channel is summed in ascending order: a
  // channel the head drops has coefficient 0 and adds exactly nothing.
  if (has_tail && tid < G * kGroup) {
    const int h = tid / kGroup, r = tid % kGroup, t = t_body + r;
    float zz = -INFINITY;
    if (t < t_end) {
      zz = sm.coefc[h][0] * f16_value(c0row[t]);   // channel 0: its fp16 value, as in the blocks
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
  // coefficients in slot order, scaled by 2^-E_h (E_h: exponent of the head's
  // largest |coefficient| over channels >= 1)
  for (int e = tid; e < G * D; e += kThreads4) {
    const int h = e / D, i = e % D;
    const float mx = D > 64 ? fmaxf(sm.redm[h][0], sm.redm[h][1]) : sm.redm[h][0];
    int ex = 0;
    if (mx > 0.0f) frexpf(mx, &ex);
    const int ch = slot_channel(i);
    sm.coefs[h][i] = ch >= 0 ? sm.coefc[h][ch] * ldexpf(1.0f, -ex) : 0.0f;
    if (i == 0) sm.e2[h] = ldexpf(1.0f, ex);
  }
  block_barrier();
  float ca[G], cb[G];   // coefficients of the two slots per head (0 outside U)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    ca[h] = sm.coefs[h][as0];
    cb[h] = sm.coefs[h][as1];
  }
  // Key scales of the A-building slots outside U count as zero: the first block
  // read them (their coefficients are zero, but a scale that is not finite would
  // still poison the products), later blocks do not read them.
  uint32_t ksm[2];
  {
    // later blocks read the union's channels only
    // (compact slots hold union channels only; past |U| they read nothing)
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
  // the second block once the union is known (a smaller first burst of loads: the
  // first blocks of every workgroup arrive sooner)
  kissue(S1, t_begin + kBlock4, 1 < nbc0);

  auto kcommit = [&](KStage4<D> &S, KBlock4<D> &B, int p0) {
    if (slots_live) {
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
    // logit A operands: key scales of a key group past the coded range (the exact
    // tail or beyond) count as zero.  High part = fp16 of the product, low part =
    // fp16 of what the high part leaves out (about 22 significant bits together).
    uint32_t v0 = S.ks[0] & ksm[0], v1 = S.ks[1] & ksm[1];
    if (slots_live) {
    if (p0 + kBlock4 > code_end) {   // workgroup-uniform
      const int g0 = p0 / kGroup + 2 * agp;
      const uint32_t km = (g0 * kGroup < code_end ? 0xffffu : 0u) | ((g0 + 1) * kGroup < code_end ? 0xffff0000u : 0u);
      v0 &= km;
      v1 &= km;
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      uint32_t hi0 = mixhi<0>(mixlo<0>(ca[h], v0), cb[h], v1);
      uint32_t lo0 = reshi<0, 1>(reslo<0, 0>(ca[h], v0, hi0), cb[h], v1, hi0);
      uint32_t hi1 = mixhi<1>(mixlo<1>(ca[h], v0), cb[h], v1);
      uint32_t lo1 = reshi<1, 1>(reslo<1, 0>(ca[h], v0, hi1), cb[h], v1, hi1);
      uint16_t (*ar)[L::AROW] = B.a[agp].r;
      *reinterpret_cast<uint32_t *>(&ar[2 * h][8 * aoct + 2 * am]) = hi0;
      *reinterpret_cast<uint32_t *>(&ar[2 * h + 1][8 * aoct + 2 * am]) = lo0;
      *reinterpret_cast<uint32_t *>(&ar[8 + 2 * h][8 * aoct + 2 * am]) = hi1;
      *reinterpret_cast<uint32_t *>(&ar[8 + 2 * h + 1][8 * aoct + 2 * am]) = lo1;
    }
    }
    B.c0w[tid] = S.c0;
  };

  // ---------------------------------------------------------------- per-wavefront state
  WaveSmem4<D> &W = sm.w[wave];
  const int q = lane >> 4, n = lane & 15;
  const int lg = q >> 1, hp = q & 1;   // logit lanes: key group of the tile, head pair (2hp, 2hp+1)

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
  u32x4 ones = {kOneF16x2, kOneF16x2, kOneF16x2, kOneF16x2};

  // Logits (log2 units) of this wavefront's tile of one block: z[hh][nt] for head
  // 2hp + hh and token tile0 + 32lg + 2n + nt; -inf past the end of the split.
  auto logits = [&](const KBlock4<D> &B, int tile0, float (&z)[2][2]) {
    // ---- C rows (group lg, heads 2hp, 2hp+1, high/low), columns tokens 32lg + 2n + nt
    f32x4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = acc0, accs = acc0;
    asm volatile("" : "+v"(ones));
    {
      // every K chunk is worked on (slots past |U| have zero codes and zero
      // coefficients): straight-line code without branches between the products
      const uint16_t *arow_base = arow ? &B.a[wave].r[n][8 * (q & 1)] : reinterpret_cast<const uint16_t *>(&W.zero);
      const int astep = arow ? 16 : 0;
#pragma unroll
      for (int kc = 0; kc < L::NKC; ++kc) {
        if constexpr (COMPACT) {
          if (kc >= nkc) break;   // wavefront-uniform
        }
        const u32x4 al = *reinterpret_cast<const u32x4 *>(arow_base + astep * kc);
        const u32x2 dk = *reinterpret_cast<const u32x2 *>(&B.y[wave][2 * kc + (q & 1)][8 * lg + (n >> 1)][0]);
        const uint32_t l0 = pk_shl16(dk.x, shl2), h0 = pk_shr16(dk.x, shr2);
        const uint32_t l1 = pk_shl16(dk.y, shl2), h1 = pk_shr16(dk.y, shr2);
        constexpr uint32_t M3 = 0x00C000C0u, M4 = 0x03000300u;
        const u32x4 b0 = {l0 & M3, h0 & M3, l1 & M3, h1 & M3};   // token r0: u 2^-18
        const u32x4 b1 = {l0 & M4, h0 & M4, l1 & M4, h1 & M4};   // token r0+1: u 2^-16
        acc0 = mfma16(al, b0, acc0);
        acc1 = mfma16(al, b1, acc1);
        accs = mfma16(al, ones, accs);
      }
    }
    const int tt = kTile4 * wave + 32 * lg + 2 * n;   // my first token within the block
    const uint32_t cx0 = B.c0w[tt >> 1];
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
    const int tl0 = tile0 + 32 * lg + 2 * n;   // my first token
    if (tile0 + kTile4 > t_end) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        if (tl0 + nt >= t_end) z[0][nt] = z[1][nt] = -INFINITY;
    }
    // tokens of the unfinished last group: the exact logits computed up front
    if (tile0 + kTile4 > t_body && t_body < t_end) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int t = tl0 + nt;
        if (t >= t_body && t < t_end) {
          z[0][nt] = sm.tailz[2 * hp][t - t_body];
          z[1][nt] = sm.tailz[2 * hp + 1][t - t_body];
        }
      }
    }
  };

  // ---------------------------------------------------------------- value loads (per wavefront)
  // value A producer: my tokens are c = 2(n&7), c+1 of word 2lg + (n>>3)
  const int pw = 2 * lg + (n >> 3), pkc = (n >> 1) & 1, pi0 = 4 * (n & 1) + ((n >> 2) & 1);
  const int pk[2] = {value_k(2 * (n & 3)), value_k(2 * (n & 3) + 1)};
  const uint32_t vwv = (uint32_t)(16 * q + n) * 4u;                   // word row 0, channel 16q + n of the tile
  const uint32_t vsv = (uint32_t)(32 * lg + 2 * n) * (uint32_t)(L::VG * 2);   // scales of my two tokens

  // Values are read once: their loads carry the non-temporal hint, so that they
  // do not push out of L2 the key lines a block shares with the next one (a key
  // block uses half of each 128-byte line of its channels' codes).
  constexpr int kNT = 2;
  auto vissue = [&](VStage4<D> &V, int tile0, bool live) {
    __builtin_amdgcn_sched_barrier(0);
    live = live && tile0 < t_end;
    const uint32_t u0 = (uint32_t)tile0;
    const auto rvw = rsrc(vwords, vw_bytes, (u0 >> 4) * (uint32_t)(D * 4), live);
    const auto rvs = rsrc(vscales, vs_bytes, u0 * (uint32_t)(L::VG * 2), live);
#pragma unroll
    for (int hf = 0; hf < L::NH; ++hf)
#pragma unroll
      for (int wr = 0; wr < 4; ++wr)
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
  float m_run[G];      // per head: the maximum logit so far (-inf before any)
#pragma unroll
  for (int h = 0; h < G; ++h) m_run[h] = -INFINITY;
  int f_run = 0, es_run = -24;
  uint32_t sbound = 0u;   // fp16 bits of 2^es_run: a larger value scale moves F
  bool firstv = true;
  float fp[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) fp[nt] = (float)(f_run + 24 - 2 * pk[nt]);
  float lacc[2][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}};
  // Weighted sum: one product per 8 tokens and 64 channels, block diagonal in K:
  // C[4jj + h][n] = sum over the 8 tokens of A[h][t] B[t][16jj + n], K = (jj, t),
  // so lane (n, q) accumulates heads 0-3 of channel 64 half + 16q + n.
  f32x4 vacc[L::NH];
#pragma unroll
  for (int hf = 0; hf < L::NH; ++hf) vacc[hf] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // S = 2^F sum p scale per (head 2hp + hh, value group j), from the same fp16
  // operands (each scaled back by the 2^(2k-24) of its token), partial per lane.
  float sacc[2][L::VG];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int j = 0; j < L::VG; ++j) sacc[hh][j] = 0.0f;
  const float kback[2] = {ldexpf(1.0f, 2 * pk[0] - 24), ldexpf(1.0f, 2 * pk[1] - 24)};
  if (lane == 0) W.zero = u32x4{0u, 0u, 0u, 0u};

  // One tile of values: numerators from the stored logits, weighted sum of the codes.
  auto values = [&](const VStage4<D> &V, int tile0, const float (&z)[2][2], const float (&mr)[2]) {
    // value scales of tokens past the split end are zero (their numerators are zero too)
    const int t0 = tile0 + 32 * lg + 2 * n;
    const uint32_t m0 = t0 < t_end ? 0xffffffffu : 0u, m1 = t0 + 1 < t_end ? 0xffffffffu : 0u;
    uint32_t cvs[L::VG];
#pragma unroll
    for (int i = 0; i < L::VG; ++i) cvs[i] = V.vs[i] & (i < L::VG / 2 ? m0 : m1);

    // ---- value exponent F: moves only when a value scale outgrows 2^es_run
    uint32_t smax = 0;
#pragma unroll
    for (int i = 0; i < L::VG; ++i) smax = max(smax, max(cvs[i] & 0xffffu, cvs[i] >> 16));
    if (firstv || __ballot(smax >= sbound) != 0ull) {
      const float sv = wave_max(h2f(smax));
      int es_t = -24;
      if (sv > 0.0f) frexpf(sv, &es_t);
      const int es_new = firstv ? es_t : max(es_run, es_t);
      const int f_new = 15 - 24 - es_new;
      if (!firstv) {
        const float beta = ldexpf(1.0f, f_new - f_run);
#pragma unroll
        for (int hf = 0; hf < L::NH; ++hf) vacc[hf] *= beta;
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

    // ---- numerators -> value A operands (row = head, K = token)
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
      // the value scale of token nt, group j is half (j & 1) of cvs[nt * VG/2 + j/2]
      const uint32_t s0 = cvs[j >> 1], s1 = cvs[L::VG / 2 + (j >> 1)];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        uint16_t *dst = &W.u.t.pbuf[j][pkc][(pw * 4 + 2 * hp + hh) * 8 + pi0];
        const uint32_t a0 = (j & 1) ? mixlo<1>(p[hh][0], s0) : mixlo<0>(p[hh][0], s0);
        const uint32_t a1 = (j & 1) ? mixlo<1>(p[hh][1], s1) : mixlo<0>(p[hh][1], s1);
        dst[0] = (uint16_t)a0;
        dst[2] = (uint16_t)a1;
        sacc[hh][j] = mix_acc(sacc[hh][j], a0, kback[0]);
        sacc[hh][j] = mix_acc(sacc[hh][j], a1, kback[1]);
      }
    }
    wave_sync();

    // ---- weighted sum of the value codes: A of lane (row 4jj + h, K group q) is
    // head h's 8 numerators of value group 2 half + jj/2 when q == jj, else zero
    const int jj = n >> 2, ah = n & 3;
#pragma unroll
    for (int hf = 0; hf < L::NH; ++hf)
#pragma unroll
      for (int wr = 0; wr < 4; ++wr)
#pragma unroll
        for (int kc2 = 0; kc2 < 2; ++kc2) {
          const u32x4 *src = q == jj ? reinterpret_cast<const u32x4 *>(&W.u.t.pbuf[2 * hf + (jj >> 1)][kc2][(wr * 4 + ah) * 8])
                                     : &W.zero;
          vacc[hf] = mfma16(*src, value_operand(V.vw[hf][wr], kc2), vacc[hf]);
        }
    wave_sync();
  };

  // ---------------------------------------------------------------- chunks
  for (int cb = 0; cb < nb;) {
    // a wavefront that is through with the previous chunk waits here until the
    // others have also read the key blocks of its last two blocks
    if (cb > 0) block_barrier();
    // blocks in this chunk: up to kChunk4, or kChunk4 + 1 when that many are left
    // (the extra block takes the same steps after the others, with logits of its
    // own), so that a share of one block more costs one block, not one chunk
    const int nbc = nb - cb == kChunk4 + 1 ? kChunk4 + 1 : min(kChunk4, nb - cb);
    const int c_t0 = t_begin + kBlock4 * cb;         // first token of the chunk
    float zs[kChunk4][2][2];                         // this wavefront's logits of the chunk
    float zl[2] = {-INFINITY, -INFINITY};            // and their maximum per head of the pair

    // ---- pass 1: keys.  Block i is written to LDS buffer i & 1 once its loads
    // have landed and is published by a barrier.  The body for block i works
    // out its logits and, in the same straight-line code, writes block i + 1 to
    // the other buffer (so the matrix products of one block overlap the vector
    // work of the next), issues the loads of block i + 3 into the registers
    // block i + 1 came in, and ends with the barrier that publishes block i + 1
    // and tells every wavefront that block i is done with.  Loads run two
    // blocks ahead of their commit.  Blocks past the chunk are committed as
    // zeros (their loads are empty) and never read.
    if (cb > 0) {   // the first chunk's were issued during the setup
      kissue(S0, c_t0, 0 < nbc);
      kissue(S1, c_t0 + kBlock4, 1 < nbc);
    }
    // A block's commit and the loads issued with it gate the barrier every
    // wavefront of the workgroup waits on: they run at raised wave priority, so
    // they win the issue arbitration against the logits and value work of the
    // other workgroup on the compute unit (which otherwise, being older or not,
    // decides who waits).
    __builtin_amdgcn_s_setprio(1);
    kcommit(S0, sm.kb[0], c_t0);
    kissue(S0, c_t0 + 2 * kBlock4, 2 < nbc);
    block_barrier();
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int i = 0; i < kChunk4; ++i) {
      if (i >= nbc) break;
      const int p0 = c_t0 + kBlock4 * i;
      // every tile is worked on: tokens past the end get -inf inside logits()
      logits(sm.kb[i & 1], p0 + kTile4 * wave, zs[i]);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) zl[hh] = fmaxf(zl[hh], fmaxf(zs[i][hh][0], zs[i][hh][1]));
      KStage4<D> &S = (i & 1) ? S0 : S1;   // holds block i + 1
      __builtin_amdgcn_s_setprio(1);   // commit, issue and barrier: raised, as above
      kcommit(S, sm.kb[(i + 1) & 1], p0 + kBlock4);
      kissue(S, p0 + 3 * kBlock4, i + 3 < nbc);
      block_barrier();
      __builtin_amdgcn_s_setprio(0);
    }
    float z9[2][2];   // the extra block: committed to buffer kChunk4 & 1 by the last body
    if (nbc > kChunk4) {
      logits(sm.kb[kChunk4 & 1], c_t0 + kBlock4 * kChunk4 + kTile4 * wave, z9);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) zl[hh] = fmaxf(zl[hh], fmaxf(z9[hh][0], z9[hh][1]));
    }

    // ---- pass 2: values; the first three tiles are on their way during the maximum
    VStage4<D> V0, V1, V2;
    vissue(V0, c_t0 + kTile4 * wave, true);
    vissue(V1, c_t0 + kBlock4 + kTile4 * wave, 1 < nbc);
    vissue(V2, c_t0 + 2 * kBlock4 + kTile4 * wave, 2 < nbc);

    // exact maximum of each head's logits in the chunk (wavefront-uniform)
    float d[G];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const float zm = row16_max(zl[hh]);
      const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, zm), 0));
      const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, zm), 16));
      const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, zm), 32));
      const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, zm), 48));
      d[hh] = fmaxf(r0, r2);        // head hh   (rows q = 0, 2)
      d[2 + hh] = fmaxf(r1, r3);    // head 2+hh (rows q = 1, 3)
    }
    // a head whose maximum rises rescales what was accumulated before this chunk
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
      for (int hf = 0; hf < L::NH; ++hf)
#pragma unroll
        for (int i = 0; i < 4; ++i) vacc[hf][i] *= al[i];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const float a = sel2(hp, al[hh], al[2 + hh]);
#pragma unroll
        for (int j = 0; j < L::VG; ++j) sacc[hh][j] *= a;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) lacc[hh][nt] *= a;
      }
    }
    // subtracted from my heads' logits (0 for a head with no logit yet: its numerators are 0)
    float mr[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const float m = sel2(hp, m_run[hh], m_run[2 + hh]);
      mr[hh] = m == -INFINITY ? 0.0f : m;
    }

#pragma unroll
    for (int i = 0; i < kChunk4; ++i) {
      if (i >= nbc) break;
      VStage4<D> &V = (i % 3 == 0) ? V0 : (i % 3 == 1) ? V1 : V2;
      const int tile0 = c_t0 + kBlock4 * i + kTile4 * wave;
      if (tile0 < t_end) values(V, tile0, zs[i], mr);
      __builtin_amdgcn_s_setprio(1);   // value loads are issued at raised priority too
      vissue(V, tile0 + 3 * kBlock4, i + 3 < nbc);
      __builtin_amdgcn_s_setprio(0);
    }
    if (nbc > kChunk4) {   // the extra block's values are in stage kChunk4 % 3
      const int tile0 = c_t0 + kBlock4 * kChunk4 + kTile4 * wave;
      VStage4<D> &VX = kChunk4 % 3 == 0 ? V0 : kChunk4 % 3 == 1 ? V1 : V2;
      if (tile0 < t_end) values(VX, tile0, z9, mr);
    }
    cb += nbc;
  }
  // loads of tiles past the end (they return zeros) land before the merge
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---------------------------------------------------------------- merge the wavefronts
  const bool had = t_begin + kTile4 * wave < t_end;   // this wavefront had tokens
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
    // S per (head, value group): sum over the 32 lanes of each head pair
    float sh[G][L::VG];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int j = 0; j < L::VG; ++j) {
        const float v = row16_sum(sacc[hh][j]);
        const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
        const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
        const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
        const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
        sh[hh][j] = r0 + r2;
        sh[2 + hh][j] = r1 + r3;
      }
    const float inv_f = ldexpf(1.0f, -f_run);
#pragma unroll
    for (int hf = 0; hf < L::NH; ++hf) {
      const int ch = 64 * hf + 16 * q + n;   // value group 2 hf + (q >> 1)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float si = sel2((q >> 1) != 0, sh[i][2 * hf], sh[i][2 * hf + 1]);
        W.u.merge[i][ch] = (2.0f * vacc[hf][i] - 3.0f * si) * inv_f;
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
  // Straight-line: every LDS read of an element is issued before any is used, and
  // a wavefront without tokens is dropped by selects, not branches.
  static_assert((G * D) % kThreads4 == 0, "whole rounds of elements");
#pragma unroll
  for (int k = 0; k < (G * D) / kThreads4; ++k) {
    const int e = tid + kThreads4 * k, h = e / D, ch = e % D;
    float lw[kWaves4], mw[kWaves4], ow[kWaves4];
#pragma unroll
    for (int w = 0; w < kWaves4; ++w) {
      lw[w] = sm.w[w].lstate[h];
      mw[w] = sm.w[w].mstate[h];
      ow[w] = sm.w[w].u.merge[h][ch];
    }
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves4; ++w) M = lw[w] > 0.0f ? fmaxf(M, mw[w]) : M;
    float o = 0.0f, Lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves4; ++w) {
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

int compute_units() {
  static std::atomic<int> cache[64];   // per device: 0 = not yet queried
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

bool decode4_supported(const dqk_cache &c, int hq) {
  return c.capacity % 64 == 0 && hq == kG4 * c.num_kv_heads;
}

hipError_t launch_decode4(const dqk_cache &c, const float *q_prime, const int32_t *sel_idx,
                          bool shared, int hq, int keep, float scale2, int split, bool even,
                          float *ws, float *out, hipStream_t s) {
  const int nsplit = num_splits(c.capacity, split);
  // a caller's split of whole blocks covers exactly its split tokens of every row;
  // otherwise (and always for the library's own split count) each split takes an
  // equal share of its row's current blocks
  const int bps = !even && split % kBlock4 == 0 ? split / kBlock4 : 0;
  const int units = c.batch * c.num_kv_heads;
  const int items = units * nsplit;
  // (KV head, row, split), whose linear order is the item order, if rows and
  // splits fit the grid's second and third dimensions; else one-dimensional
  const int grid3 = c.batch <= 65535 && nsplit <= 65535 ? 1 : 0;
  const dim3 grid = grid3 ? dim3((unsigned)c.num_kv_heads, (unsigned)c.batch, (unsigned)nsplit)
                          : dim3((unsigned)items);
  const dim3 block(kThreads4);
  // uneven shares for two workgroups per compute unit (the library's own split
  // only; the kernel's share arithmetic is 32-bit for fewer than 4096 compute units)
  int ncu = 0;
  if (even && bps == 0) {
    const int n = compute_units();
    if (n > 0 && n < 4096 && items > n && items <= 2 * n) ncu = n;
  }
  const int ncu_q = ncu / units, ncu_r = ncu % units;
  // group-shared kept sets use compact slots: only the K chunks that hold the
  // keep - 1 kept channels other than 0 are worked on
  const int nkc = shared ? (keep - 1 + 15) / 16 : c.head_dim / 16;
  const int sh = shared ? 1 : 0;
  if (c.head_dim == 64) {
    if (shared)
      hipLaunchKernelGGL((decode4_kernel<64, true>), grid, block, 0, s, c, q_prime, sel_idx, sh, hq, grid3, keep,
                         scale2, nsplit, bps, ncu_q, ncu_r, nkc, ws, out);
    else
      hipLaunchKernelGGL((decode4_kernel<64, false>), grid, block, 0, s, c, q_prime, sel_idx, sh, hq, grid3, keep,
                         scale2, nsplit, bps, ncu_q, ncu_r, nkc, ws, out);
  } else {
    if (shared)
      hipLaunchKernelGGL((decode4_kernel<128, true>), grid, block, 0, s, c, q_prime, sel_idx, sh, hq, grid3, keep,
                         scale2, nsplit, bps, ncu_q, ncu_r, nkc, ws, out);
    else
      hipLaunchKernelGGL((decode4_kernel<128, false>), grid, block, 0, s, c, q_prime, sel_idx, sh, hq, grid3, keep,
                         scale2, nsplit, bps, ncu_q, ncu_r, nkc, ws, out);
  }
  return hipGetLastError();
}

}  // namespace dqk
