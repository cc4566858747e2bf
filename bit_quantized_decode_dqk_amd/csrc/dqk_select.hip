// Query transform and per-head channel selection.
//
// Dual-QK (arXiv abstract; tech.dede.sh summary, "Paired transforms instead of
// shared rotation"): the query transform q' = q A concentrates query energy so
// that dynamic channel pruning keeps few channels; "Results at 128K context"
// evaluates it at 40% query-channel sparsity.  Here each query head keeps
// channel 0 (the protected channel) and the keep-1 other channels of largest
// |q'|, equal magnitudes going to the lower index; the kept set is written in
// ascending order.
//
// One workgroup per (batch row, query head), one wavefront-pair of 128 lanes:
// lane j forms q'_j as an fp32 FMA chain over input channels in ascending order
// (bit-reproducible), then ranks |q'_j| against the other channels -- an exact
// top-k by counting -- and a ballot prefix gives each kept channel its slot.
// Built with -ffp-contract=off.
#include "dqk_internal.h"

namespace dqk {
namespace {

constexpr int kThreads = 128;

template <int D>
__global__ __launch_bounds__(kThreads) void select_kernel(const void *q, int bf16,
                                                          const float *__restrict__ amat, int hq,
                                                          int hkv, int keep, float *q_prime,
                                                          int32_t *sel_idx) {
  __shared__ float qs[D];
  __shared__ float mag[D];
  __shared__ int kept[D];
  const int row = blockIdx.x;  // b * hq + h
  const int h = row % hq;
  const int g = h / (hq / hkv);
  const int j = threadIdx.x;
  if (j < D)
    qs[j] = bf16 ? bf16_value(static_cast<const uint16_t *>(q)[(size_t)row * D + j])
                 : static_cast<const float *>(q)[(size_t)row * D + j];
  __syncthreads();
  if (j < D) {
    const float *acol = amat + (size_t)g * D * D + j;
    float acc = 0.0f;
    for (int i = 0; i < D; ++i) acc = __builtin_fmaf(qs[i], acol[(size_t)i * D], acc);
    q_prime[(size_t)row * D + j] = acc;
    mag[j] = fabsf(acc);
  }
  __syncthreads();
  if (j < D) {
    int k = 1;  // channel 0 is always kept
    if (j > 0) {
      const float mj = mag[j];
      int rank = 0;
      for (int c = 1; c < D; ++c) rank += (mag[c] > mj) || (mag[c] == mj && c < j);
      k = rank < keep - 1;
    }
    kept[j] = k;
  }
  __syncthreads();
  if (j < D && kept[j]) {
    int pos = 0;
    for (int c = 0; c < j; ++c) pos += kept[c];
    if (pos < keep) sel_idx[(size_t)row * keep + pos] = j;
  }
}

}  // namespace

hipError_t launch_select(const void *q, bool bf16, const float *amat, int batch, int hq, int hkv,
                         int d, int keep, float *q_prime, int32_t *sel_idx, hipStream_t s) {
  const dim3 grid((unsigned)(batch * hq));
  if (d == 64)
    hipLaunchKernelGGL(select_kernel<64>, grid, dim3(kThreads), 0, s, q, (int)bf16, amat, hq, hkv,
                       keep, q_prime, sel_idx);
  else
    hipLaunchKernelGGL(select_kernel<128>, grid, dim3(kThreads), 0, s, q, (int)bf16, amat, hq,
                       hkv, keep, q_prime, sel_idx);
  return hipGetLastError();
}

}  // namespace dqk
