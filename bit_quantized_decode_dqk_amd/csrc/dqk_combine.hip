// Online-max combine of split partials (shared by the 2-bit and the bf16 decode).
//
// A decode split leaves, per query head, the running max m (log2 units), the sum
// l of 2^(z - m) and the unnormalized output o.  The combine forms
// M = max m_i, L = sum l_i 2^(m_i - M), out = sum o_i 2^(m_i - M) / L; splits
// with l = 0 (past the sequence end) drop out, and an empty sequence gives 0.
#include "dqk_internal.h"

namespace dqk {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// One workgroup per (batch row, query head, 32-channel slice).  Thread (k, c)
// takes float4 column c of the slice and the splits k, k + 32, ... with its own
// running maximum; a batch of kBatch splits per thread is one round trip (all
// of its loads are issued before any is used, and a split past the end reads
// zeros from the range-checked buffer resource, l = 0).  The 32 split classes
// are then merged by the same rule: four per thread of the first wavefront
// through LDS, the remaining eight with cross-lane shuffles.
constexpr int kSlice = 32;                       // channels per workgroup
constexpr int kCols = kSlice / 4;                // float4 columns
constexpr int kThreadsC = 256;
constexpr int kClasses = kThreadsC / kCols;      // 32 split classes
constexpr int kBatch = 4;
constexpr int kRsrcWord3C = 0x00020000;          // raw buffer, 32-bit elements, range-checked

struct State {
  float m, l;
  f32x4 o;
};

// (m, l, o) of two disjoint sets of splits -> their union (m = -inf: empty).
__device__ __forceinline__ State join(State a, State b) {
  const float M = fmaxf(a.m, b.m);
  if (M == -INFINITY) return a;
  const float fa = exp2f(a.m - M), fb = exp2f(b.m - M);   // 0 for an empty side
  return State{M, a.l * fa + b.l * fb, a.o * fa + b.o * fb};
}

__device__ __forceinline__ State shfl_state(State s, int off) {
  State r;
  r.m = __shfl_xor(s.m, off, 64);
  r.l = __shfl_xor(s.l, off, 64);
  r.o.x = __shfl_xor(s.o.x, off, 64);
  r.o.y = __shfl_xor(s.o.y, off, 64);
  r.o.z = __shfl_xor(s.o.z, off, 64);
  r.o.w = __shfl_xor(s.o.w, off, 64);
  return r;
}

template <int D>
__global__ __launch_bounds__(kThreadsC) void combine_kernel(const float *__restrict__ ws, int hq,
                                                            int hkv, int nsplit,
                                                            float *__restrict__ out) {
  constexpr int NSL = D / kSlice;
  constexpr int PH = D + kPartialHead;   // floats per (split, head)
  __shared__ State part[kThreadsC];
  const int row = blockIdx.x / NSL, sl = blockIdx.x % NSL;
  const int b = row / hq, h = row % hq;
  const int G = hq / hkv;
  const int unit = b * hkv + h / G, hi = h % G;
  const int tid = threadIdx.x, c = tid % kCols, k = tid / kCols;
  const float *base = ws + ((size_t)unit * nsplit * G + hi) * PH;
  const int span = ((nsplit - 1) * G + 1) * PH;   // floats from base to the last split's end
  const auto r = __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, span * (int)sizeof(float),
                                                   kRsrcWord3C);
  const uint32_t stride = (uint32_t)G * PH * 4u;   // bytes between splits
  const uint32_t col = (uint32_t)(kPartialHead + kSlice * sl + 4 * c) * 4u;

  State st{-INFINITY, 0.0f, {0.0f, 0.0f, 0.0f, 0.0f}};
  for (int s0 = k; s0 < nsplit; s0 += kClasses * kBatch) {
    f32x2 ml[kBatch];
    f32x4 o[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const uint32_t at = (uint32_t)(s0 + kClasses * j) * stride;
      ml[j] = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(r, at, 0, 0));
      o[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, at + col, 0, 0));
    }
    float bm = st.m;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) bm = ml[j].y > 0.0f ? fmaxf(bm, ml[j].x) : bm;
    const float f = st.m == -INFINITY ? 0.0f : exp2f(st.m - bm);   // l and o are 0 while m is -inf
    st.l *= f;
    st.o *= f;
    st.m = bm;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const float w = ml[j].y > 0.0f ? exp2f(ml[j].x - bm) : 0.0f;   // a partial's o is finite
      st.l = fmaf(w, ml[j].y, st.l);
      st.o += w * o[j];
    }
  }
  part[tid] = st;
  __syncthreads();
  if (tid >= 64) return;
  // thread (k < 8, c) of the first wavefront joins classes k, k + 8, k + 16, k + 24
#pragma unroll
  for (int q = 1; q < kClasses / 8; ++q) st = join(st, part[tid + 64 * q]);
  // lanes k * 8 + c: join over k with shuffles across lane bits 3-5
#pragma unroll
  for (int off = 8; off < 64; off <<= 1) st = join(st, shfl_state(st, off));
  if (k == 0) {
    const float inv = st.l > 0.0f ? 1.0f / st.l : 0.0f;
    *reinterpret_cast<f32x4 *>(out + (size_t)row * D + kSlice * sl + 4 * c) = st.o * inv;
  }
}

}  // namespace

hipError_t launch_combine(const float *ws, int batch, int hq, int hkv, int d, int nsplit,
                          float *out, hipStream_t s) {
  const dim3 grid((unsigned)(batch * hq * (d / kSlice)));
  if (d == 64)
    hipLaunchKernelGGL(combine_kernel<64>, grid, dim3(kThreadsC), 0, s, ws, hq, hkv, nsplit, out);
  else
    hipLaunchKernelGGL(combine_kernel<128>, grid, dim3(kThreadsC), 0, s, ws, hq, hkv, nsplit, out);
  return hipGetLastError();
}

}  // namespace dqk
