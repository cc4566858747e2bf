// Growing a cache: the planes of one cache copied into a cache of larger
// capacity (same batch, KV heads and head dimension), so that a sequence can
// outgrow the capacity it was created with (tech.dede.sh summary, "Why the
// cache becomes a bottleneck": the cache grows with every generated token).
// Every plane is laid out per (batch row, KV head) unit with the capacity as a
// row length or a unit stride, and nothing stored depends on the capacity, so
// growing is a re-strided copy: each unit's rows of the source land at the
// start of the destination's longer rows.  The destination's positions past the
// source capacity keep what they held (zeros for a fresh cache).
#include "dqk_internal.h"

namespace dqk {
namespace {

// One copy job: `rows` rows of `row_elems` elements of `esz` bytes (16, 4 or 2),
// row r from src + r*src_stride to dst + r*dst_stride (strides in elements).
struct CopyJob {
  const void *src;
  void *dst;
  long long rows, row_elems, src_stride, dst_stride;
  int esz;
};
constexpr int kMaxJobs = 7;
struct CopyJobs {
  CopyJob j[kMaxJobs];
  int n;
};

template <typename T>
__device__ __forceinline__ void copy_rows(const CopyJob &J, long long start, long long step) {
  const T *s = static_cast<const T *>(J.src);
  T *d = static_cast<T *>(J.dst);
  const long long total = J.rows * J.row_elems;
  for (long long e = start; e < total; e += step) {
    const long long r = e / J.row_elems, k = e - r * J.row_elems;
    d[r * J.dst_stride + k] = s[r * J.src_stride + k];
  }
}

// blockIdx.y is the job; the workgroups along x stride through its elements.
__global__ __launch_bounds__(256) void grow_kernel(CopyJobs jobs) {
  const CopyJob &J = jobs.j[blockIdx.y];
  const long long start = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long step = (long long)gridDim.x * blockDim.x;
  if (J.esz == 16) copy_rows<uint4>(J, start, step);
  else if (J.esz == 4) copy_rows<uint32_t>(J, start, step);
  else copy_rows<uint16_t>(J, start, step);
}

// Largest element size (16, 4 or 2 bytes) that divides the row bytes, both row
// strides and both base addresses.
int elem_size(const void *s, const void *d, long long row_bytes, long long ss, long long ds) {
  for (int e : {16, 4}) {
    if (row_bytes % e == 0 && ss % e == 0 && ds % e == 0 &&
        reinterpret_cast<uintptr_t>(s) % e == 0 && reinterpret_cast<uintptr_t>(d) % e == 0)
      return e;
  }
  return 2;
}

void add_job(CopyJobs &jobs, const void *s, void *d, long long rows, long long row_bytes,
             long long src_stride_bytes, long long dst_stride_bytes) {
  const int e = elem_size(s, d, row_bytes, src_stride_bytes, dst_stride_bytes);
  jobs.j[jobs.n++] = CopyJob{s, d, rows, row_bytes / e, src_stride_bytes / e, dst_stride_bytes / e, e};
}

}  // namespace

hipError_t launch_cache_grow(const dqk_cache &src, const dqk_cache &dst, hipStream_t s) {
  const long long units = (long long)src.batch * src.num_kv_heads, D = src.head_dim;
  const long long cs = src.capacity, cd = dst.capacity;
  CopyJobs jobs{};
  // k_codes [unit][D][cap/4] bytes, k_scales [unit][D][cap/32] fp16: rows of one channel
  add_job(jobs, src.k_codes, dst.k_codes, units * D, cs / 4, cs / 4, cd / 4);
  add_job(jobs, src.k_scales, dst.k_scales, units * D, 2 * (cs / kGroup), 2 * (cs / kGroup), 2 * (cd / kGroup));
  // k_ch0 [unit][cap] fp16, v_codes [unit][cap/16][D] u32, v_scales [unit][cap][D/32] fp16:
  // one row per unit
  add_job(jobs, src.k_ch0, dst.k_ch0, units, 2 * cs, 2 * cs, 2 * cd);
  add_job(jobs, src.v_codes, dst.v_codes, units, 4 * (cs / 16) * D, 4 * (cs / 16) * D, 4 * (cd / 16) * D);
  add_job(jobs, src.v_scales, dst.v_scales, units, 2 * cs * (D / kGroup), 2 * cs * (D / kGroup), 2 * cd * (D / kGroup));
  // k_tail [unit][32][D] f32 and lengths [2][batch] i32: the same size in both
  add_job(jobs, src.k_tail, dst.k_tail, 1, units * kGroup * D * 4, 0, 0);
  add_job(jobs, src.lengths, dst.lengths, 1, 8LL * src.batch, 0, 0);
  const dim3 grid(1024, (unsigned)jobs.n);
  hipLaunchKernelGGL(grow_kernel, grid, dim3(256), 0, s, jobs);
  return hipGetLastError();
}

}  // namespace dqk
