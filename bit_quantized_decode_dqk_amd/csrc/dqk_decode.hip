// Decode attention over the 2-bit cache with pruned query channels, split over
// the sequence, plus the online-max combine of the splits.
//
// Dual-QK (arXiv abstract; tech.dede.sh summary, "Throughput on SGLang"):
// pruning removes key channels from reads and keys/values are stored in 2 bits,
// which is where the decode speedup comes from.  A work item is one
// (batch row, KV head, split of the sequence); it serves every query head of
// the GQA group.  Only the union of the group's kept key channels is read:
// their 2-bit rows (channel-major, so a dropped channel costs no bytes), their
// per-group scales, channel 0's fp16 row and, for the unfinished last group,
// the exact tail.  Each head's logit uses only its own kept channels.  Values
// are never pruned: every value word of the split is read once.
//
// Layout of the work: 256 lanes, chunks of 1024 tokens.  Logits: lane i owns
// tokens 4i..4i+3 of the chunk (one code byte per kept channel).  Softmax runs
// in the log2 domain with a running max per head.  Values: lane i owns channel
// i % d for a contiguous part of the chunk and accumulates all heads of the
// group.  The partial (max, sum, output) of every head goes to the workspace;
// the combine kernel merges the splits.
#include "dqk_internal.h"

namespace dqk {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 1024;
constexpr int kWaves = kThreads / 64;

template <int D, int G>
struct DecodeSmem {
  float coef[G][D];         // q'_{h,c} * sm * log2(e) (0 if head h drops c)
  int hmask[D];             // bit h: head h keeps channel c
  int16_t ulist[D];         // channels >= 1 kept by some head, ascending
  int wcount[2];
  float red[G][kWaves];
  float p[G][kChunk];       // exp2(z - m) of the chunk; reused for the final reduction
  float vs[kChunk][D / kGroup];
};

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

template <int D, int G>
__global__ __launch_bounds__(kThreads) void decode_kernel(dqk_cache c, const float *__restrict__ qp,
                                                          const int32_t *__restrict__ sel, int hq,
                                                          int keep, float scale2, int split,
                                                          int nsplit, float *__restrict__ ws) {
  __shared__ DecodeSmem<D, G> sm;
  constexpr int VG = D / kGroup;
  constexpr int PARTS = kThreads / D;
  constexpr int TPP = kChunk / PARTS;  // tokens per part in the value pass
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int item = blockIdx.x;
  const int unit = item / nsplit, s = item % nsplit;
  const int b = unit / c.num_kv_heads, g = unit % c.num_kv_heads;
  const int len = max(0, min(c.lengths[b], c.capacity));
  const int t_begin = s * split;
  const int t_end = min(t_begin + split, len);
  float *wsp = ws + (size_t)item * G * (D + 2);
  if (t_begin >= t_end) {
    for (int e = tid; e < G * (D + 2); e += kThreads) wsp[e] = (e % (D + 2) == 0) ? -INFINITY : 0.0f;
    return;
  }

  // ---- selection masks and coefficients of the group's heads
  for (int e = tid; e < G * D; e += kThreads) sm.coef[e / D][e % D] = 0.0f;
  for (int e = tid; e < D; e += kThreads) sm.hmask[e] = 0;
  __syncthreads();
  const size_t row0 = (size_t)b * hq + (size_t)g * G;
  for (int e = tid; e < G * keep; e += kThreads) {
    const int h = e / keep;
    const int ch = sel[(row0 + h) * keep + e % keep];
    if (ch >= 0 && ch < D) {
      atomicOr(&sm.hmask[ch], 1 << h);
      sm.coef[h][ch] = qp[(row0 + h) * D + ch] * scale2;
    }
  }
  __syncthreads();
  {  // ascending union list by ballot over channels (D <= 128: waves 0 and 1)
    const bool f = tid < D && tid >= 1 && sm.hmask[tid] != 0;
    const unsigned long long m = __ballot(f);
    if (lane == 0 && wave < 2) sm.wcount[wave] = __popcll(m);
    __syncthreads();
    if (f) sm.ulist[__popcll(m & ((1ull << lane) - 1ull)) + (wave == 1 ? sm.wcount[0] : 0)] = (int16_t)tid;
  }
  __syncthreads();
  const int nu = sm.wcount[0] + sm.wcount[1];
  const int m0 = sm.hmask[0];

  const size_t kc_stride = (size_t)(c.capacity / 4);
  const size_t ks_stride = (size_t)(c.capacity / kGroup);
  const uint8_t *kc = c.k_codes + unit * (size_t)D * kc_stride;
  const uint16_t *ks = c.k_scales + unit * (size_t)D * ks_stride;
  const uint16_t *c0 = c.k_ch0 + unit * (size_t)c.capacity;
  const float *tail = c.k_tail + unit * (size_t)kGroup * D;
  const uint32_t *vw = c.v_codes + unit * (size_t)(c.capacity / 16) * D;
  const uint16_t *vsc = c.v_scales + unit * (size_t)c.capacity * VG;
  const int t_body = (len / kGroup) * kGroup;

  float m_run[G], l_run[G], o_acc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.0f;
    o_acc[h] = 0.0f;
  }
  const int vch = tid % D, part = tid / D;

  for (int tc = t_begin; tc < t_end; tc += kChunk) {
    const int n_ch = min(kChunk, t_end - tc);
    for (int e = tid; e < n_ch * VG; e += kThreads) sm.vs[e / VG][e % VG] = f16_value(vsc[(size_t)tc * VG + e]);

    // ---- logits of my 4 tokens
    const int tt = tc + 4 * tid;
    const bool live = tt < t_end;
    const bool coded = live && tt < t_body;   // t_body % 4 == 0: all four coded or none
    float z[G][4];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int k = 0; k < 4; ++k) z[h][k] = 0.0f;
    for (int i = 0; i < nu; ++i) {
      const int ch = sm.ulist[i];
      const int hm = sm.hmask[ch];
      uint32_t byte = 0;
      float sc = 0.0f;
      if (coded) {
        byte = kc[(size_t)ch * kc_stride + (tt >> 2)];
        sc = f16_value(ks[(size_t)ch * ks_stride + (tt >> 5)]);
      }
      float w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) w[k] = level_of((byte >> (2 * k)) & 3u);
#pragma unroll
      for (int h = 0; h < G; ++h)
        if (hm & (1 << h)) {
          const float cf = sm.coef[h][ch] * sc;
#pragma unroll
          for (int k = 0; k < 4; ++k) z[h][k] = fmaf(cf, w[k], z[h][k]);
        }
    }
    if (live && !coded) {  // the unfinished last group: exact tail values
      for (int i = 0; i < nu; ++i) {
        const int ch = sm.ulist[i];
        const int hm = sm.hmask[ch];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int t = tt + k;
          if (t >= t_end) break;
          const float x = tail[(size_t)(t & 31) * D + ch];
#pragma unroll
          for (int h = 0; h < G; ++h)
            if (hm & (1 << h)) z[h][k] = fmaf(sm.coef[h][ch], x, z[h][k]);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int t = tt + k;
      if (t < t_end) {
        const float x0 = f16_value(c0[t]);
#pragma unroll
        for (int h = 0; h < G; ++h)
          if (m0 & (1 << h)) z[h][k] = fmaf(sm.coef[h][0], x0, z[h][k]);
      } else {
#pragma unroll
        for (int h = 0; h < G; ++h) z[h][k] = -INFINITY;
      }
    }

    // ---- running max and exponentials
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = fmaxf(fmaxf(z[h][0], z[h][1]), fmaxf(z[h][2], z[h][3]));
      mx = wave_max(mx);
      if (lane == 0) sm.red[h][wave] = mx;
    }
    __syncthreads();
    float alpha[G], m_new[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = sm.red[h][0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, sm.red[h][w]);
      m_new[h] = fmaxf(m_run[h], mx);
      alpha[h] = exp2f(m_run[h] - m_new[h]);
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float ls = 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float p = exp2f(z[h][k] - m_new[h]);
        sm.p[h][4 * tid + k] = p;
        ls += p;
      }
      ls = wave_sum(ls);
      if (lane == 0) sm.red[h][wave] = ls;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float ls = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) ls += sm.red[h][w];
      l_run[h] = l_run[h] * alpha[h] + ls;
      m_run[h] = m_new[h];
      o_acc[h] *= alpha[h];
    }

    // ---- values: channel vch, tokens [part*TPP, part*TPP + TPP) of the chunk
    const int lt0 = part * TPP;
    const int lt1 = min(lt0 + TPP, n_ch);
    for (int w16 = lt0; w16 < lt1; w16 += 16) {
      const uint32_t word = vw[(size_t)((tc + w16) >> 4) * D + vch];
      const int kmax = min(16, lt1 - w16);
      for (int k = 0; k < kmax; ++k) {
        const int lt = w16 + k;
        const float val = sm.vs[lt][vch / kGroup] * level_of((word >> (2 * k)) & 3u);
#pragma unroll
        for (int h = 0; h < G; ++h) o_acc[h] = fmaf(sm.p[h][lt], val, o_acc[h]);
      }
    }
    __syncthreads();
  }

  // ---- merge the value parts and write the partial of every head
  float *red = &sm.p[0][0];  // [PARTS][G][D]
#pragma unroll
  for (int h = 0; h < G; ++h) red[((size_t)part * G + h) * D + vch] = o_acc[h];
  __syncthreads();
  if (tid < D) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float o = 0.0f;
#pragma unroll
      for (int pp = 0; pp < PARTS; ++pp) o += red[((size_t)pp * G + h) * D + tid];
      wsp[h * (D + 2) + 2 + tid] = o;
      if (tid == 0) {
        wsp[h * (D + 2) + 0] = m_run[h];
        wsp[h * (D + 2) + 1] = l_run[h];
      }
    }
  }
}

// Online-max combine of the split partials: M = max m_i, L = sum l_i 2^(m_i-M),
// o = sum o_i 2^(m_i-M) / L.  One workgroup per (batch row, query head).
template <int D>
__global__ __launch_bounds__(D) void combine_kernel(const float *__restrict__ ws, int hq, int hkv,
                                                    int nsplit, float *__restrict__ out) {
  const int row = blockIdx.x;
  const int b = row / hq, h = row % hq;
  const int G = hq / hkv;
  const int unit = b * hkv + h / G, hi = h % G;
  const int c = threadIdx.x;
  const float *base = ws + ((size_t)unit * nsplit * G + hi) * (D + 2);
  const size_t stride = (size_t)G * (D + 2);
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) {
    const float *p = base + s * stride;
    if (p[1] > 0.0f) M = fmaxf(M, p[0]);
  }
  float den = 0.0f, acc = 0.0f;
  for (int s = 0; s < nsplit; ++s) {
    const float *p = base + s * stride;
    if (p[1] > 0.0f) {
      const float f = exp2f(p[0] - M);
      den = fmaf(p[1], f, den);
      acc = fmaf(p[2 + c], f, acc);
    }
  }
  out[(size_t)row * D + c] = den > 0.0f ? acc / den : 0.0f;
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
  hipLaunchKernelGGL(combine_kernel<D>, dim3((unsigned)(c.batch * hq)), dim3(D), 0, s, ws, hq,
                     c.num_kv_heads, nsplit, out);
  return hipGetLastError();
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
