// Dense dequantized view of the stored cache (for checking; not on the decode
// path).  Key channel 0 is the protected fp16 value; other key channels are
// s*(2u-3) inside complete 32-token groups and the exact tail after them; value
// channels are s*(2u-3) with the per-token 32-channel scale.  Positions at or
// past the row's length are zero.
#include "dqk_internal.h"

namespace dqk {
namespace {

template <int D>
__global__ __launch_bounds__(256) void dequant_kernel(dqk_cache c, float *k_out, float *v_out) {
  constexpr int TPB = 256 / D;  // tokens per workgroup
  const int unit = blockIdx.y;
  const int t = blockIdx.x * TPB + threadIdx.x / D;
  const int ch = threadIdx.x % D;
  if (t >= c.capacity) return;
  const int b = unit / c.num_kv_heads;
  const int len = max(0, min(c.lengths[b], c.capacity));
  const size_t o = ((size_t)unit * c.capacity + t) * D + ch;
  if (t >= len) {
    k_out[o] = 0.0f;
    v_out[o] = 0.0f;
    return;
  }
  float k;
  if (ch == 0) {
    k = f16_value(c.k_ch0[(size_t)unit * c.capacity + t]);
  } else if (t < (len / kGroup) * kGroup) {
    const size_t row = (size_t)unit * D + ch;
    const uint32_t u = (c.k_codes[row * (c.capacity / 4) + (t >> 2)] >> (2 * (t & 3))) & 3u;
    k = f16_value(c.k_scales[row * (c.capacity / kGroup) + (t >> 5)]) * level_of(u);
  } else {
    k = c.k_tail[((size_t)unit * kGroup + (t & 31)) * D + ch];
  }
  const uint32_t w = c.v_codes[((size_t)unit * (c.capacity / 16) + (t >> 4)) * D + ch];
  const float s = f16_value(c.v_scales[((size_t)unit * c.capacity + t) * (D / kGroup) + ch / kGroup]);
  k_out[o] = k;
  v_out[o] = s * level_of((w >> (2 * (t & 15))) & 3u);
}

}  // namespace

hipError_t launch_dequant(const dqk_cache &c, float *k_out, float *v_out, hipStream_t s) {
  const int units = c.batch * c.num_kv_heads;
  if (c.head_dim == 64) {
    const dim3 grid((unsigned)((c.capacity + 3) / 4), (unsigned)units);
    hipLaunchKernelGGL(dequant_kernel<64>, grid, dim3(256), 0, s, c, k_out, v_out);
  } else {
    const dim3 grid((unsigned)((c.capacity + 1) / 2), (unsigned)units);
    hipLaunchKernelGGL(dequant_kernel<128>, grid, dim3(256), 0, s, c, k_out, v_out);
  }
  return hipGetLastError();
}

}  // namespace dqk
