// Online-max combine of split partials (shared by the 2-bit and the bf16 decode).
//
// A decode split leaves, per query head, the running max m (log2 units), the sum
// l of 2^(z - m) and the unnormalized output o.  The combine forms
// M = max m_i, L = sum l_i 2^(m_i - M), out = sum o_i 2^(m_i - M) / L; splits
// with l = 0 (past the sequence end) drop out, and an empty sequence gives 0.
#include "dqk_internal.h"

namespace dqk {
namespace {

// One workgroup per (batch row, query head); the splits are read in parallel
// (lanes over splits for the max and the sum, then lanes over (4-channel slice,
// split subset) with float4 loads for the output).
constexpr int kCombineThreads = 256;

template <int D>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const float *__restrict__ ws,
                                                                  int hq, int hkv, int nsplit,
                                                                  float *__restrict__ out) {
  constexpr int C4 = D / 4;                   // float4 slices of the output row
  constexpr int SG = kCombineThreads / C4;    // split subsets
  __shared__ float red[kCombineThreads / 64];
  __shared__ float4 part[SG][C4];
  const int row = blockIdx.x;
  const int b = row / hq, h = row % hq;
  const int G = hq / hkv;
  const int unit = b * hkv + h / G, hi = h % G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float *base = ws + ((size_t)unit * nsplit * G + hi) * (D + kPartialHead);
  const size_t stride = (size_t)G * (D + kPartialHead);

  float mx = -INFINITY;
  for (int s = tid; s < nsplit; s += kCombineThreads) {
    const float l = base[s * stride + 1];
    const float m = base[s * stride];
    if (l > 0.0f) mx = fmaxf(mx, m);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int w = 1; w < kCombineThreads / 64; ++w) M = fmaxf(M, red[w]);
  __syncthreads();

  float den = 0.0f;
  for (int s = tid; s < nsplit; s += kCombineThreads) {
    const float l = base[s * stride + 1];
    const float m = base[s * stride];
    if (l > 0.0f) den = fmaf(l, exp2f(m - M), den);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) den += __shfl_xor(den, o, 64);
  if (lane == 0) red[wave] = den;

  const int c4 = tid % C4, sg = tid / C4;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll 4
  for (int s = sg; s < nsplit; s += SG) {
    const float *p = base + s * stride;
    const float l = p[1];
    const float f = l > 0.0f ? exp2f(p[0] - M) : 0.0f;
    const float4 o = *reinterpret_cast<const float4 *>(p + kPartialHead + 4 * c4);
    acc.x = fmaf(o.x, f, acc.x);
    acc.y = fmaf(o.y, f, acc.y);
    acc.z = fmaf(o.z, f, acc.z);
    acc.w = fmaf(o.w, f, acc.w);
  }
  part[sg][c4] = acc;
  __syncthreads();
  float dsum = 0.0f;
#pragma unroll
  for (int w = 0; w < kCombineThreads / 64; ++w) dsum += red[w];
  if (tid < C4) {
    float4 t = part[0][tid];
#pragma unroll
    for (int g = 1; g < SG; ++g) {
      t.x += part[g][tid].x;
      t.y += part[g][tid].y;
      t.z += part[g][tid].z;
      t.w += part[g][tid].w;
    }
    const float inv = dsum > 0.0f ? 1.0f / dsum : 0.0f;
    float4 r = make_float4(t.x * inv, t.y * inv, t.z * inv, t.w * inv);
    *reinterpret_cast<float4 *>(out + (size_t)row * D + 4 * tid) = r;
  }
}

}  // namespace

hipError_t launch_combine(const float *ws, int batch, int hq, int hkv, int d, int nsplit,
                          float *out, hipStream_t s) {
  const dim3 grid((unsigned)(batch * hq));
  if (d == 64)
    hipLaunchKernelGGL(combine_kernel<64>, grid, dim3(kCombineThreads), 0, s, ws, hq, hkv, nsplit, out);
  else
    hipLaunchKernelGGL(combine_kernel<128>, grid, dim3(kCombineThreads), 0, s, ws, hq, hkv, nsplit, out);
  return hipGetLastError();
}

}  // namespace dqk
