// The two independent parts of a decode step in one launch: the new token's
// append and the query's channel selection (Dual-QK: tech.dede.sh summary,
// "Paired transforms instead of shared rotation" -- keys and queries go through
// their own transforms; arXiv abstract -- INT2 cache, dynamic channel pruning).
// The selection workgroups (one per query head; they take longer) come first
// in the grid, the append workgroups after them; each runs the same body as in
// its own kernel (the append workgroups commit the lengths).  Built with
// -ffp-contract=off.
#include "dqk_append_body.h"
#include "dqk_select_body.h"

namespace dqk {
namespace {

static_assert(appb::kThreads == selb::kThreads, "one block size for both bodies");

template <int D, int G, bool BF16>
__global__ __launch_bounds__(appb::kThreads) void append_select_kernel(
    dqk_cache c, const void *k_new, const void *v_new, const float *__restrict__ bmat,
    const int32_t *__restrict__ n_new, int max_new, int blocks_per_unit, const void *q,
    const float *__restrict__ amat, int hq, int keep, float *q_prime, int32_t *sel_idx) {
  const int sel_blocks = c.batch * c.num_kv_heads * selb::blocks_per_unit<D, G>();
  if ((int)blockIdx.x < sel_blocks)   // workgroup-uniform
    selb::select_block<D, G, BF16>(blockIdx.x, q, amat, hq, c.num_kv_heads, keep, q_prime, sel_idx);
  else
    appb::append_block<D, BF16>(blockIdx.x - sel_blocks, c, k_new, v_new, bmat, n_new, max_new,
                                blocks_per_unit);
}

template <int D, int G>
void launch_g(const dqk_cache &c, const void *k_new, const void *v_new, bool bf16,
              const float *bmat, const int32_t *n_new, int max_new, const void *q,
              const float *amat, int hq, int keep, float *q_prime, int32_t *sel_idx,
              hipStream_t s) {
  const int units = c.batch * c.num_kv_heads;
  const int per_unit = (max_new + kGroup - 1) / kGroup + 1;  // as in the append launch
  const dim3 grid((unsigned)(units * selb::blocks_per_unit<D, G>() + units * per_unit)),
      block(appb::kThreads);
  if (bf16)
    hipLaunchKernelGGL((append_select_kernel<D, G, true>), grid, block, 0, s, c, k_new, v_new, bmat,
                       n_new, max_new, per_unit, q, amat, hq, keep, q_prime, sel_idx);
  else
    hipLaunchKernelGGL((append_select_kernel<D, G, false>), grid, block, 0, s, c, k_new, v_new, bmat,
                       n_new, max_new, per_unit, q, amat, hq, keep, q_prime, sel_idx);
}

template <int D>
hipError_t launch_d(const dqk_cache &c, const void *k_new, const void *v_new, bool bf16,
                    const float *bmat, const int32_t *n_new, int max_new, const void *q,
                    const float *amat, int hq, int keep, float *q_prime, int32_t *sel_idx,
                    hipStream_t s) {
  switch (hq / c.num_kv_heads) {
    case 1: launch_g<D, 1>(c, k_new, v_new, bf16, bmat, n_new, max_new, q, amat, hq, keep, q_prime, sel_idx, s); break;
    case 2: launch_g<D, 2>(c, k_new, v_new, bf16, bmat, n_new, max_new, q, amat, hq, keep, q_prime, sel_idx, s); break;
    case 4: launch_g<D, 4>(c, k_new, v_new, bf16, bmat, n_new, max_new, q, amat, hq, keep, q_prime, sel_idx, s); break;
    case 8: launch_g<D, 8>(c, k_new, v_new, bf16, bmat, n_new, max_new, q, amat, hq, keep, q_prime, sel_idx, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append_select(const dqk_cache &c, const void *k_new, const void *v_new,
                                bool bf16, const float *bmat, const int32_t *n_new, int max_new,
                                const void *q, const float *amat, int hq, int keep,
                                float *q_prime, int32_t *sel_idx, hipStream_t s) {
  const hipError_t e =
      c.head_dim == 64
          ? launch_d<64>(c, k_new, v_new, bf16, bmat, n_new, max_new, q, amat, hq, keep, q_prime, sel_idx, s)
          : launch_d<128>(c, k_new, v_new, bf16, bmat, n_new, max_new, q, amat, hq, keep, q_prime, sel_idx, s);
  return e;
}

}  // namespace dqk
