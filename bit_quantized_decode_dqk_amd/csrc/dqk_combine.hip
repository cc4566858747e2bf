// Online-max combine of split partials (shared by the 2-bit and the bf16 decode).
//
// A decode split leaves, per query head, the running max m (log2 units), the sum
// l of 2^(z - m) and the unnormalized output o.  The combine forms
// M = max m_i, L = sum l_i 2^(m_i - M), out = sum o_i 2^(m_i - M) / L; splits
// with l = 0 (past the sequence end) drop out, and an empty sequence gives 0.
#include "dqk_internal.h"

namespace dqk {
namespace {

// One wavefront per (batch row, query head, 32-channel slice).  Lane s merges
// splits s, s+64, ... on its own (all of its loads are issued before any is
// used), then the 64 lane results are merged: the maximum and the denominator
// with cross-lane shuffles, the 32 outputs through LDS.
constexpr int kSlice = 32;
constexpr int kCombineLanes = 64;

template <int D>
__global__ __launch_bounds__(kCombineLanes) void combine_kernel(const float *__restrict__ ws,
                                                                int hq, int hkv, int nsplit,
                                                                float *__restrict__ out) {
  constexpr int NSL = D / kSlice;
  __shared__ float part[kCombineLanes][kSlice + 1];
  const int row = blockIdx.x / NSL, sl = blockIdx.x % NSL;
  const int b = row / hq, h = row % hq;
  const int G = hq / hkv;
  const int unit = b * hkv + h / G, hi = h % G;
  const int lane = threadIdx.x;
  const size_t stride = (size_t)G * (D + kPartialHead);
  const float *base = ws + ((size_t)unit * nsplit * G + hi) * (D + kPartialHead);

  float m = -INFINITY, l = 0.0f;
  float o[kSlice];
#pragma unroll
  for (int c = 0; c < kSlice; ++c) o[c] = 0.0f;
  for (int s = lane; s < nsplit; s += kCombineLanes) {
    const float *p = base + s * stride;
    const float ms = p[0], ls = p[1];
    float4 v[kSlice / 4];
#pragma unroll
    for (int c = 0; c < kSlice / 4; ++c)
      v[c] = *reinterpret_cast<const float4 *>(p + kPartialHead + kSlice * sl + 4 * c);
    if (ls > 0.0f) {
      const float mn = fmaxf(m, ms);
      const float fa = exp2f(m - mn), fb = exp2f(ms - mn);
      l = l * fa + ls * fb;
#pragma unroll
      for (int c = 0; c < kSlice / 4; ++c) {
        o[4 * c + 0] = o[4 * c + 0] * fa + v[c].x * fb;
        o[4 * c + 1] = o[4 * c + 1] * fa + v[c].y * fb;
        o[4 * c + 2] = o[4 * c + 2] * fa + v[c].z * fb;
        o[4 * c + 3] = o[4 * c + 3] * fa + v[c].w * fb;
      }
      m = mn;
    }
  }
  float M = m;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  const float f = l > 0.0f ? exp2f(m - M) : 0.0f;
  float L = l * f;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off, 64);
#pragma unroll
  for (int c = 0; c < kSlice; ++c) part[lane][c] = o[c] * f;
  __syncthreads();
  if (lane < kSlice) {
    float acc = 0.0f;
#pragma unroll 8
    for (int s = 0; s < kCombineLanes; ++s) acc += part[s][lane];
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    out[(size_t)row * D + kSlice * sl + lane] = acc * inv;
  }
}

}  // namespace

hipError_t launch_combine(const float *ws, int batch, int hq, int hkv, int d, int nsplit,
                          float *out, hipStream_t s) {
  const dim3 grid((unsigned)(batch * hq * (d / kSlice)));
  if (d == 64)
    hipLaunchKernelGGL(combine_kernel<64>, grid, dim3(kCombineLanes), 0, s, ws, hq, hkv, nsplit, out);
  else
    hipLaunchKernelGGL(combine_kernel<128>, grid, dim3(kCombineLanes), 0, s, ws, hq, hkv, nsplit, out);
  return hipGetLastError();
}

}  // namespace dqk
