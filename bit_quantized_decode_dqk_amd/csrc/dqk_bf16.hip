// Unpruned BF16 decode attention: the baseline the pages compare against
// ("relative to unpruned BF16", tech.dede.sh summary, "Results at 128K context"
// and "Throughput on SGLang").  Raw bf16 keys and values, token-major
// [batch][hkv][ld_t][d], no transforms, no quantization, fp32 accumulation.
//
// A work item is one (batch row, KV head, split); it serves every query head of
// the GQA group, so each key and value byte is read once.  Each wavefront takes
// its own 32-token tiles of the split (tiles w, w + 4, ... for wavefront w) with
// its own online softmax, so the tile loop has no workgroup barrier:
//  - logits on the matrix cores (v_mfma_f32_16x16x32_bf16): A = the group's q
//    rows (head m in row m, rows past G zero), B = the tile's keys, each lane
//    loading 16 contiguous bytes of one token's row straight into operand order;
//  - the weighted sum on the vector units: lane (channel group, token subset)
//    loads 8 channels of its tokens' value rows and accumulates all heads; the
//    tile's numerators go through LDS (a wavefront-private buffer).
// The four wavefronts merge their (m, l, o) at the end.  The split partials use
// the same workspace format and combine kernel as the 2-bit decode.
#include "dqk_decode_ops.h"

namespace dqk {
namespace {

using namespace wave;
using dops::kRsrcWord3;

constexpr int kThreads = 256;
constexpr int kWavesB = kThreads / 64;
constexpr int kTileB = 32;                 // tokens per wavefront tile

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <int D, int G>
struct Bf16Smem {
  float p[kWavesB][kTileB][G];   // each wavefront's tile numerators, token-major
  float o[kWavesB][G][D];        // each wavefront's output at the end of the split
  float m[kWavesB][G], l[kWavesB][G];
};

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <int D, int G>
__global__ __launch_bounds__(kThreads, G <= 4 ? 3 : 2) void bf16_decode_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ lengths, int hq, int hkv, int ld_t, float scale2, int split,
    int nsplit, float *__restrict__ ws) {
  __shared__ Bf16Smem<D, G> sm;
  constexpr int KC = D / 32;          // logit K chunks of 32 channels
  constexpr int CG = D / 8;           // weighted-sum channel groups of 8 channels
  constexpr int TS = 64 / CG;         // token subsets (lanes per channel group)
  constexpr int TPL = kTileB / TS;    // tokens per lane and tile in the weighted sum
  constexpr int PH = D + kPartialHead;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int item = blockIdx.x;
  const int unit = item / nsplit, s = item % nsplit;
  const int b = unit / hkv, g = unit % hkv;
  const int len = max(0, min(lengths[b], ld_t));
  const int t_begin = s * split;
  const int t_end = min(t_begin + split, len);
  float *wsp = ws + (size_t)item * G * PH;
  if (t_begin >= t_end) {
    for (int e = tid; e < G * PH; e += kThreads) wsp[e] = (e % PH == 0) ? -INFINITY : 0.0f;
    return;
  }
  const int n = lane & 15, kq = lane >> 4;     // matrix lanes: column / row n, K group kq
  const int cgr = lane % CG, ts = lane / CG;   // weighted-sum lanes: channels 8 cgr.., tokens TPL ts..
  // A operand: q row of head n (zero past G), channels 32 kc + 8 kq .. + 7
  u32x4 qa[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    qa[kc] = u32x4{0u, 0u, 0u, 0u};
    if (n < G)
      qa[kc] = *reinterpret_cast<const u32x4 *>(q + ((size_t)b * hq + (size_t)g * G + n) * D + 32 * kc + 8 * kq);
  }
  const uint16_t *kunit = k + (size_t)unit * ld_t * D;
  const uint16_t *vunit = v + (size_t)unit * ld_t * D;

  float m_run[G], l_run[G];   // wavefront-uniform
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.0f;
  }
  float o[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int c = 0; c < 8; ++c) o[h][c] = 0.0f;

  for (int tile0 = t_begin + kTileB * wave; tile0 < t_end; tile0 += kTileB * kWavesB) {
    // the tile's rows as range-checked buffers: rows at or past t_end read zeros
    const int rows = min(kTileB, t_end - tile0);
    const auto rk = __builtin_amdgcn_make_buffer_rsrc((void *)(kunit + (size_t)tile0 * D), (short)0,
                                                      rows * D * 2, kRsrcWord3);
    const auto rv = __builtin_amdgcn_make_buffer_rsrc((void *)(vunit + (size_t)tile0 * D), (short)0,
                                                      rows * D * 2, kRsrcWord3);
    u32x4 kk[2][KC], vv[TPL];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        kk[ct][kc] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   rk, (uint32_t)(((16 * ct + n) * D + 32 * kc + 8 * kq) * 2), 0, 0));
#pragma unroll
    for (int j = 0; j < TPL; ++j)
      vv[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rv, (uint32_t)(((TPL * ts + j) * D + 8 * cgr) * 2), 0, 0));
    // logits: lane (n, kq) holds heads 4 kq + i of token tile0 + 16 ct + n
    float z[2][4];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) acc = mfma_bf16(qa[kc], kk[ct][kc], acc);
      const bool live = tile0 + 16 * ct + n < t_end;
#pragma unroll
      for (int i = 0; i < 4; ++i) z[ct][i] = live && 4 * kq + i < G ? acc[i] * scale2 : -INFINITY;
    }
    // online softmax per head: the tile maximum, then the new reference
    float rm[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) rm[i] = row16_max(fmaxf(z[0][i], z[1][i]));
    float mn[G], al[G];
    bool rise = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rm[h % 4]), 16 * (h / 4)));
      mn[h] = fmaxf(m_run[h], mt);
      al[h] = exp2f(m_run[h] - mn[h]);   // 0 before the first tile (m_run = -inf)
      rise = rise || mn[h] != m_run[h];
    }
    float mrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) mrow[i] = kq == 0 || G <= 4 ? mn[i % G] : mn[(4 + i) % G];
    float ls[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p0 = exp2f(z[0][i] - mrow[i]), p1 = exp2f(z[1][i] - mrow[i]);
      ls[i] = row16_sum(p0 + p1);
      if (4 * kq + i < G) {
        sm.p[wave][n][4 * kq + i] = p0;
        sm.p[wave][16 + n][4 * kq + i] = p1;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float lt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ls[h % 4]), 16 * (h / 4)));
      l_run[h] = fmaf(l_run[h], al[h], lt);
      m_run[h] = mn[h];
    }
    if (rise) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int c = 0; c < 8; ++c) o[h][c] *= al[h];
    }
    wave_sync();
    // weighted sum: my TPL tokens, 8 channels, every head
#pragma unroll
    for (int j = 0; j < TPL; ++j) {
      const float *pt = sm.p[wave][TPL * ts + j];
      float pv[G];
#pragma unroll
      for (int h = 0; h < G; ++h) pv[h] = pt[h];
      const u32x4 w = vv[j];
      const float vf[8] = {lo_bf16(w.x), hi_bf16(w.x), lo_bf16(w.y), hi_bf16(w.y),
                           lo_bf16(w.z), hi_bf16(w.z), lo_bf16(w.w), hi_bf16(w.w)};
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int c = 0; c < 8; ++c) o[h][c] = fmaf(pv[h], vf[c], o[h][c]);
    }
    wave_sync();   // the next tile's numerators overwrite these
  }
  // the wavefront's output: sum over the token subsets, then to LDS
#pragma unroll
  for (int off = CG; off < 64; off <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int c = 0; c < 8; ++c) o[h][c] += __shfl_xor(o[h][c], off, 64);
  if (ts == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int c = 0; c < 8; ++c) sm.o[wave][h][8 * cgr + c] = o[h][c];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      sm.m[wave][h] = m_run[h];
      sm.l[wave][h] = l_run[h];
    }
  }
  __syncthreads();
  // merge the wavefronts (one without tokens has l = 0) into the split's partial
  for (int e = tid; e < G * D; e += kThreads) {
    const int h = e / D, c = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWavesB; ++w) M = sm.l[w][h] > 0.0f ? fmaxf(M, sm.m[w][h]) : M;
    float oo = 0.0f, L = 0.0f;
#pragma unroll
    for (int w = 0; w < kWavesB; ++w) {
      if (sm.l[w][h] > 0.0f) {
        const float f = exp2f(sm.m[w][h] - M);
        oo = fmaf(sm.o[w][h][c], f, oo);
        L = fmaf(sm.l[w][h], f, L);
      }
    }
    wsp[h * PH + kPartialHead + c] = oo;
    if (c == 0) {
      wsp[h * PH + 0] = M;
      wsp[h * PH + 1] = L;
    }
  }
}

template <int D, int G>
hipError_t launch_t(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *lengths,
                    int batch, int hq, int hkv, int ld_t, float scale2, int split, float *out,
                    float *ws, hipStream_t s) {
  const int nsplit = num_splits(ld_t, split);
  const int items = batch * hkv * nsplit;
  hipLaunchKernelGGL((bf16_decode_kernel<D, G>), dim3((unsigned)items), dim3(kThreads), 0, s, q, k,
                     v, lengths, hq, hkv, ld_t, scale2, split, nsplit, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_combine(ws, batch, hq, hkv, D, nsplit, out, s);
}

template <int D>
hipError_t launch_d(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *lengths,
                    int batch, int hq, int hkv, int ld_t, float scale2, int split, float *out,
                    float *ws, hipStream_t s) {
  switch (hq / hkv) {
    case 1: return launch_t<D, 1>(q, k, v, lengths, batch, hq, hkv, ld_t, scale2, split, out, ws, s);
    case 2: return launch_t<D, 2>(q, k, v, lengths, batch, hq, hkv, ld_t, scale2, split, out, ws, s);
    case 4: return launch_t<D, 4>(q, k, v, lengths, batch, hq, hkv, ld_t, scale2, split, out, ws, s);
    default: return launch_t<D, 8>(q, k, v, lengths, batch, hq, hkv, ld_t, scale2, split, out, ws, s);
  }
}

}  // namespace

hipError_t launch_bf16_decode(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const int32_t *lengths, int batch, int hq, int hkv, int d, int ld_t,
                              float sm_scale, int split, float *out, float *ws, hipStream_t s) {
  const float scale2 = sm_scale * 1.4426950408889634f;
  if (d == 64) return launch_d<64>(q, k, v, lengths, batch, hq, hkv, ld_t, scale2, split, out, ws, s);
  return launch_d<128>(q, k, v, lengths, batch, hq, hkv, ld_t, scale2, split, out, ws, s);
}

}  // namespace dqk
