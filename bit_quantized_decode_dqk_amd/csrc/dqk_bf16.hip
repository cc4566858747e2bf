// Unpruned BF16 decode attention: the baseline the pages compare against
// ("relative to unpruned BF16", tech.dede.sh summary, "Results at 128K context"
// and "Throughput on SGLang").  Raw bf16 keys and values, token-major
// [batch][hkv][ld_t][d], no transforms, no quantization, fp32 accumulation.
//
// A work item is one (batch row, KV head, split); it serves every query head of
// the GQA group so each key/value byte is read once.  64-token tiles of K and V
// are staged through LDS with coalesced 16-byte loads (rows padded by one dword
// against bank conflicts); the next tile's loads are in flight in registers
// while the current one is worked on.  Lanes own (token, head) pairs for the
// logits and (channel, part) pairs for the weighted sum.  The split partials use the same
// workspace format and combine kernel as the 2-bit decode.
#include "dqk_internal.h"

namespace dqk {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;

template <int D, int G>
struct Bf16Smem {
  float q[G][D];
  uint32_t kt[kTile][D / 2 + 1];
  uint32_t vt[kTile][D / 2 + 1];
  float p[G][kTile];
  float mrun[G], lrun[G], alpha[G];
};

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <int D, int G>
__global__ __launch_bounds__(kThreads) void bf16_decode_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ lengths, int hq, int hkv, int ld_t, float scale2, int split,
    int nsplit, float *__restrict__ ws) {
  __shared__ Bf16Smem<D, G> sm;
  constexpr int PARTS = kThreads / D;
  constexpr int TPP = kTile / PARTS;
  constexpr int DW = D / 2;  // dwords per row
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int item = blockIdx.x;
  const int unit = item / nsplit, s = item % nsplit;
  const int b = unit / hkv, g = unit % hkv;
  const int len = max(0, min(lengths[b], ld_t));
  const int t_begin = s * split;
  const int t_end = min(t_begin + split, len);
  float *wsp = ws + (size_t)item * G * (D + kPartialHead);
  if (t_begin >= t_end) {
    for (int e = tid; e < G * (D + kPartialHead); e += kThreads) wsp[e] = (e % (D + kPartialHead) == 0) ? -INFINITY : 0.0f;
    return;
  }
  for (int e = tid; e < G * D; e += kThreads)
    sm.q[e / D][e % D] = bf16_value(q[((size_t)b * hq + (size_t)g * G + e / D) * D + e % D]) * scale2;
  if (tid < G) {
    sm.mrun[tid] = -INFINITY;
    sm.lrun[tid] = 0.0f;
  }
  const uint4 *k4 = reinterpret_cast<const uint4 *>(k + (size_t)unit * ld_t * D);
  const uint4 *v4 = reinterpret_cast<const uint4 *>(v + (size_t)unit * ld_t * D);
  const int vch = tid % D, part = tid / D;
  float o_acc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) o_acc[h] = 0.0f;

  // K and V rows tc..tc+kTile-1 as 16-byte pieces (D/8 per row), PPT per thread;
  // rows at or past t_end are zeros
  constexpr int PPT = kTile * (D / 8) / kThreads;
  static_assert(PPT * kThreads == kTile * (D / 8), "whole pieces per thread");
  uint4 pk[PPT], pv[PPT];
  auto fetch = [&](int tc) {
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int e = tid + kThreads * j, r = e / (D / 8), piece = e % (D / 8);
      pk[j] = pv[j] = make_uint4(0, 0, 0, 0);
      if (tc + r < t_end) {
        pk[j] = k4[(size_t)(tc + r) * (D / 8) + piece];
        pv[j] = v4[(size_t)(tc + r) * (D / 8) + piece];
      }
    }
  };
  fetch(t_begin);
  for (int tc = t_begin; tc < t_end; tc += kTile) {
    const int n = min(kTile, t_end - tc);
    // stage this tile (the previous one is no longer read: the loop ends with a
    // barrier), then put the next tile's loads in flight
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int e = tid + kThreads * j, r = e / (D / 8), piece = e % (D / 8);
      uint32_t *kr = &sm.kt[r][piece * 4];
      uint32_t *vr = &sm.vt[r][piece * 4];
      kr[0] = pk[j].x; kr[1] = pk[j].y; kr[2] = pk[j].z; kr[3] = pk[j].w;
      vr[0] = pv[j].x; vr[1] = pv[j].y; vr[2] = pv[j].z; vr[3] = pv[j].w;
    }
    __syncthreads();
    if (tc + kTile < t_end) fetch(tc + kTile);
    // logits: lane pair (token r, head h)
    for (int e = tid; e < kTile * G; e += kThreads) {
      const int r = e % kTile, h = e / kTile;
      float acc = 0.0f;
#pragma unroll 8
      for (int w = 0; w < DW; ++w) {
        const uint32_t x = sm.kt[r][w];
        acc = fmaf(sm.q[h][2 * w], lo_bf16(x), acc);
        acc = fmaf(sm.q[h][2 * w + 1], hi_bf16(x), acc);
      }
      sm.p[h][r] = r < n ? acc : -INFINITY;
    }
    __syncthreads();
    // softmax update of each head by one wave (64 tokens = 64 lanes)
    for (int h = wave; h < G; h += kThreads / 64) {
      const float z = sm.p[h][lane];
      float mx = z;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
      const float mnew = fmaxf(sm.mrun[h], mx);
      const float p = exp2f(z - mnew);
      float ls = p;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) ls += __shfl_xor(ls, o, 64);
      sm.p[h][lane] = p;
      if (lane == 0) {
        const float a = exp2f(sm.mrun[h] - mnew);
        sm.alpha[h] = a;
        sm.lrun[h] = sm.lrun[h] * a + ls;
        sm.mrun[h] = mnew;
      }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) o_acc[h] *= sm.alpha[h];
    for (int r = part * TPP; r < min(part * TPP + TPP, n); ++r) {
      const uint32_t x = sm.vt[r][vch >> 1];
      const float val = (vch & 1) ? hi_bf16(x) : lo_bf16(x);
#pragma unroll
      for (int h = 0; h < G; ++h) o_acc[h] = fmaf(sm.p[h][r], val, o_acc[h]);
    }
    __syncthreads();
  }
  // merge parts through the (now free) K tile
  float *red = reinterpret_cast<float *>(&sm.kt[0][0]);  // [PARTS][G][D] <= 256*G floats
#pragma unroll
  for (int h = 0; h < G; ++h) red[((size_t)part * G + h) * D + vch] = o_acc[h];
  __syncthreads();
  if (tid < D) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float o = 0.0f;
#pragma unroll
      for (int pp = 0; pp < PARTS; ++pp) o += red[((size_t)pp * G + h) * D + tid];
      wsp[h * (D + kPartialHead) + kPartialHead + tid] = o;
      if (tid == 0) {
        wsp[h * (D + kPartialHead) + 0] = sm.mrun[h];
        wsp[h * (D + kPartialHead) + 1] = sm.lrun[h];
      }
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
