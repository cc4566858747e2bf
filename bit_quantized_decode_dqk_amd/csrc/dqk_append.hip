// Append step kernel (the workgroup body, with the length commit, is in
// dqk_append_body.h) and the fp16 conversion hook.  Built with -ffp-contract=off.
#include "dqk_append_body.h"

namespace dqk {
namespace {

using appb::kThreads;

template <int D, bool BF16, bool BULK>
__global__ __launch_bounds__(kThreads) void append_kernel(dqk_cache c, const void *k_new,
                                                          const void *v_new,
                                                          const float *__restrict__ bmat,
                                                          const int32_t *__restrict__ n_new,
                                                          int max_new, int blocks_per_unit) {
  appb::append_block<D, BF16, BULK>(blockIdx.x, c, k_new, v_new, bmat, n_new, max_new, blocks_per_unit);
}

template <int D, bool BF16>
void launch_append_d(const dqk_cache &c, const void *k_new, const void *v_new, const float *bmat,
                     const int32_t *n_new, int max_new, int per_unit, dim3 grid, hipStream_t s) {
  // more new tokens than a workgroup has token slots per channel, and B 16-byte
  // aligned: the bulk form
  if (max_new > kThreads / D && (reinterpret_cast<uintptr_t>(bmat) & 15u) == 0)
    hipLaunchKernelGGL((append_kernel<D, BF16, true>), grid, dim3(kThreads), 0, s, c, k_new, v_new, bmat,
                       n_new, max_new, per_unit);
  else
    hipLaunchKernelGGL((append_kernel<D, BF16, false>), grid, dim3(kThreads), 0, s, c, k_new, v_new, bmat,
                       n_new, max_new, per_unit);
}

__global__ void f16_convert_kernel(const float *x, uint16_t *out, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = f16_bits(x[i]);
}

}  // namespace

hipError_t launch_append(const dqk_cache &c, const void *k_new, const void *v_new, bool bf16,
                         const float *bmat, const int32_t *n_new, int max_new, hipStream_t s) {
  const int units = c.batch * c.num_kv_heads;
  const int per_unit = (max_new + kGroup - 1) / kGroup + 1;  // a range can straddle one more group
  const dim3 grid((unsigned)(units * per_unit));
  if (c.head_dim == 64) {
    if (bf16) launch_append_d<64, true>(c, k_new, v_new, bmat, n_new, max_new, per_unit, grid, s);
    else launch_append_d<64, false>(c, k_new, v_new, bmat, n_new, max_new, per_unit, grid, s);
  } else {
    if (bf16) launch_append_d<128, true>(c, k_new, v_new, bmat, n_new, max_new, per_unit, grid, s);
    else launch_append_d<128, false>(c, k_new, v_new, bmat, n_new, max_new, per_unit, grid, s);
  }
  return hipGetLastError();
}

hipError_t launch_f16_convert(const float *x, uint16_t *out, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(f16_convert_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, out, n);
  return hipGetLastError();
}

}  // namespace dqk
