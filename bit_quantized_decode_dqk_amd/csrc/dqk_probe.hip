// Streaming-read probe: reads a buffer once with 16-byte loads and folds it into
// a small sink, to measure the HBM read rate a plain kernel reaches on this chip
// (the practical ceiling the decode's byte rate is read against).  Not part of the
// decode method.
#include "dqk_internal.h"

namespace dqk {
namespace {

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

constexpr int kThreadsR = 256;

// Thread i of the grid reads elements i, i + S, i + 2S, ... (S = grid threads),
// U per iteration (U loads in flight), XOR-folds them, and each wavefront
// leaves the XOR of its lanes in sink[workgroup * 4 + wave]: the XOR of the
// sink's first 4 * gridDim words is the XOR of every 32-bit word of the buffer.
template <int kUnrollR>
__global__ __launch_bounds__(kThreadsR) void stream_read_kernel(const u32x4v *__restrict__ p,
                                                                size_t n, uint32_t *__restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kThreadsR;
  size_t i = (size_t)blockIdx.x * kThreadsR + threadIdx.x;
  u32x4v acc = {0u, 0u, 0u, 0u};
  for (; i + (kUnrollR - 1) * stride < n; i += kUnrollR * stride) {
    u32x4v x[kUnrollR];
#pragma unroll
    for (int u = 0; u < kUnrollR; ++u) x[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnrollR; ++u) acc ^= x[u];
  }
  for (; i < n; i += stride) acc ^= p[i];
  uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v ^= (uint32_t)__shfl_xor((int)v, off, 64);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kThreadsR / 64) + threadIdx.x / 64] = v;
}

}  // namespace

hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, int workgroups,
                              int loads_in_flight, hipStream_t s) {
  const dim3 grid((unsigned)workgroups), block(kThreadsR);
  const u32x4v *p = static_cast<const u32x4v *>(buf);
  const size_t n = bytes / 16;
  switch (loads_in_flight) {
    case 1: hipLaunchKernelGGL(stream_read_kernel<1>, grid, block, 0, s, p, n, sink); break;
    case 2: hipLaunchKernelGGL(stream_read_kernel<2>, grid, block, 0, s, p, n, sink); break;
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, grid, block, 0, s, p, n, sink); break;
    case 8: hipLaunchKernelGGL(stream_read_kernel<8>, grid, block, 0, s, p, n, sink); break;
    case 16: hipLaunchKernelGGL(stream_read_kernel<16>, grid, block, 0, s, p, n, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dqk
