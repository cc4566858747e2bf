// Query transform and per-head channel selection (the workgroup body is in
// dqk_select_body.h).  Built with -ffp-contract=off.
#include "dqk_select_body.h"

namespace dqk {
namespace {

template <int D, int G, bool BF16>
__global__ __launch_bounds__(selb::kThreads) void select_kernel(const void *q,
                                                                const float *__restrict__ amat,
                                                                int hq, int hkv, int keep,
                                                                float *q_prime, int32_t *sel_idx) {
  selb::select_block<D, G, BF16>(blockIdx.x, q, amat, hq, hkv, keep, q_prime, sel_idx);
}

template <int D, int G, bool BF16>
__global__ __launch_bounds__(selb::kThreads) void select_shared_kernel(
    const void *q, const float *__restrict__ amat, int hq, int hkv, int keep, float *q_prime,
    int32_t *sel_idx) {
  selb::select_shared_block<D, G, BF16>(blockIdx.x, q, amat, hq, hkv, keep, q_prime, sel_idx);
}

template <int D, int G>
void launch_shared_g(const void *q, bool bf16, const float *amat, int batch, int hq, int hkv,
                     int keep, float *q_prime, int32_t *sel_idx, hipStream_t s) {
  const dim3 grid((unsigned)(batch * hkv));
  if (bf16)
    hipLaunchKernelGGL((select_shared_kernel<D, G, true>), grid, dim3(selb::kThreads), 0, s, q, amat, hq, hkv, keep, q_prime, sel_idx);
  else
    hipLaunchKernelGGL((select_shared_kernel<D, G, false>), grid, dim3(selb::kThreads), 0, s, q, amat, hq, hkv, keep, q_prime, sel_idx);
}

template <int D>
hipError_t launch_shared_d(const void *q, bool bf16, const float *amat, int batch, int hq, int hkv,
                           int keep, float *q_prime, int32_t *sel_idx, hipStream_t s) {
  switch (hq / hkv) {
    case 1: launch_shared_g<D, 1>(q, bf16, amat, batch, hq, hkv, keep, q_prime, sel_idx, s); break;
    case 2: launch_shared_g<D, 2>(q, bf16, amat, batch, hq, hkv, keep, q_prime, sel_idx, s); break;
    case 4: launch_shared_g<D, 4>(q, bf16, amat, batch, hq, hkv, keep, q_prime, sel_idx, s); break;
    case 8: launch_shared_g<D, 8>(q, bf16, amat, batch, hq, hkv, keep, q_prime, sel_idx, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, int G>
void launch_g(const void *q, bool bf16, const float *amat, int batch, int hq, int hkv, int keep,
              float *q_prime, int32_t *sel_idx, hipStream_t s) {
  const dim3 grid((unsigned)(batch * hkv * selb::blocks_per_unit<D, G>()));
  if (bf16)
    hipLaunchKernelGGL((select_kernel<D, G, true>), grid, dim3(selb::kThreads), 0, s, q, amat, hq, hkv, keep, q_prime, sel_idx);
  else
    hipLaunchKernelGGL((select_kernel<D, G, false>), grid, dim3(selb::kThreads), 0, s, q, amat, hq, hkv, keep, q_prime, sel_idx);
}

template <int D>
hipError_t launch_d(const void *q, bool bf16, const float *amat, int batch, int hq, int hkv,
                    int keep, float *q_prime, int32_t *sel_idx, hipStream_t s) {
  switch (hq / hkv) {
    case 1: launch_g<D, 1>(q, bf16, amat, batch, hq, hkv, keep, q_prime, sel_idx, s); break;
    case 2: launch_g<D, 2>(q, bf16, amat, batch, hq, hkv, keep, q_prime, sel_idx, s); break;
    case 4: launch_g<D, 4>(q, bf16, amat, batch, hq, hkv, keep, q_prime, sel_idx, s); break;
    case 8: launch_g<D, 8>(q, bf16, amat, batch, hq, hkv, keep, q_prime, sel_idx, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select_shared(const void *q, bool bf16, const float *amat, int batch, int hq,
                                int hkv, int d, int keep, float *q_prime, int32_t *sel_idx,
                                hipStream_t s) {
  if (d == 64) return launch_shared_d<64>(q, bf16, amat, batch, hq, hkv, keep, q_prime, sel_idx, s);
  return launch_shared_d<128>(q, bf16, amat, batch, hq, hkv, keep, q_prime, sel_idx, s);
}

hipError_t launch_select(const void *q, bool bf16, const float *amat, int batch, int hq, int hkv,
                         int d, int keep, float *q_prime, int32_t *sel_idx, hipStream_t s) {
  if (d == 64) return launch_d<64>(q, bf16, amat, batch, hq, hkv, keep, q_prime, sel_idx, s);
  return launch_d<128>(q, bf16, amat, batch, hq, hkv, keep, q_prime, sel_idx, s);
}

}  // namespace dqk
