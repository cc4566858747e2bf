// Host side of the C ABI: validation of everything the host can see, workspace
// sizing, and dispatch to the kernels.  Nothing here allocates, synchronizes or
// keeps state; an invalid call returns before any HIP call is made, so every
// error path can be exercised on a machine without a GPU.
#include <math.h>
#include <stdint.h>

#include "dqk_host.h"

namespace {

using dqk::kDefaultSplit;
using dqk::kGroup;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_dim(int d) { return d == 64 || d == 128; }

bool supported_group(int hq, int hkv) {
  if (hkv <= 0 || hq <= 0 || hq % hkv != 0) return false;
  const int g = hq / hkv;
  return g == 1 || g == 2 || g == 4 || g == 8;
}

// Shape and pointers of a cache; returns DQK_OK or the first problem found.
dqk_status check_cache(const dqk_cache *c) {
  if (!c) return DQK_ERR_INVALID;
  if (c->batch <= 0 || c->num_kv_heads <= 0 || c->capacity <= 0) return DQK_ERR_INVALID;
  if (c->capacity % kGroup != 0) return DQK_ERR_INVALID;
  if (!supported_dim(c->head_dim)) return DQK_ERR_UNSUPPORTED;
  const void *planes[] = {c->k_codes, c->k_scales, c->k_ch0, c->k_tail,
                          c->v_codes, c->v_scales, c->lengths};
  for (const void *p : planes)
    if (!p || !aligned16(p)) return DQK_ERR_INVALID;
  // element counts must stay addressable by 32-bit grid arithmetic per unit
  if ((int64_t)c->batch * c->num_kv_heads > (1 << 24)) return DQK_ERR_INVALID;
  return DQK_OK;
}

dqk_status from_hip(hipError_t e) { return e == hipSuccess ? DQK_OK : DQK_ERR_HIP; }

int pick_split(int split) { return split == 0 ? kDefaultSplit : split; }

bool valid_split(int split) { return split == 0 || (split >= kGroup && split % kGroup == 0); }

size_t ws_bytes_for(int batch, int hkv, int hq, int d, int tokens, int split) {
  const int nsplit = dqk::num_splits(tokens, split);
  return (size_t)batch * hkv * nsplit * (size_t)(hq / hkv) * dqk::partial_floats(d) * sizeof(float);
}

// Split of the 2-bit decode: the caller's, else the library's default (*even:
// the splits take equal shares of each row's current blocks).
int decode_split(const dqk_cache *c, int hq, int split, bool *even = nullptr) {
  if (even) *even = false;
  if (split != 0) return split;
  const int units = c->batch * c->num_kv_heads;
  if (hq % (4 * c->num_kv_heads) != 0) return dqk::default_decode_split(c->capacity, units);
  const dqk::DecodeSplit d =
      hq == 8 * c->num_kv_heads && c->capacity % 64 == 0
          ? dqk::matrix_decode_split8(c->capacity, units)
          : dqk::matrix_decode_split(c->capacity, units);
  if (even) *even = d.even;
  return d.split;
}

}  // namespace

extern "C" {

const char *dqk_status_str(dqk_status s) {
  switch (s) {
    case DQK_OK: return "ok";
    case DQK_ERR_INVALID: return "invalid argument";
    case DQK_ERR_UNSUPPORTED: return "unsupported shape";
    case DQK_ERR_WORKSPACE: return "workspace missing or too small";
    case DQK_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

dqk_status dqk_keep_count(int32_t head_dim, int32_t sparsity_pct, int32_t *out_keep) {
  if (!out_keep || head_dim < 1 || sparsity_pct < 0 || sparsity_pct > 100) return DQK_ERR_INVALID;
  *out_keep = (int32_t)(((int64_t)head_dim * (100 - sparsity_pct) + 50) / 100);
  return DQK_OK;
}

dqk_status dqk_cache_plane_bytes(int32_t batch, int32_t hkv, int32_t d, int32_t cap,
                                 size_t *out) {
  if (!out || batch <= 0 || hkv <= 0 || cap <= 0 || cap % kGroup != 0) return DQK_ERR_INVALID;
  if (!supported_dim(d)) return DQK_ERR_UNSUPPORTED;
  const size_t u = (size_t)batch * hkv;
  out[0] = u * d * (cap / 4);                   // k_codes
  out[1] = u * d * (cap / kGroup) * 2;          // k_scales
  out[2] = u * cap * 2;                         // k_ch0
  out[3] = u * kGroup * d * 4;                  // k_tail
  out[4] = u * (cap / 16) * d * 4;              // v_codes
  out[5] = u * cap * (d / kGroup) * 2;          // v_scales
  out[6] = (size_t)batch * 8;                   // lengths, then the append's arrival counters
  return DQK_OK;
}

dqk_status dqk_transform_quantize_append(const dqk_cache *cache, const void *k_new,
                                         const void *v_new, dqk_dtype dtype, const float *bmat,
                                         const int32_t *n_new, int32_t max_new,
                                         dqk_stream_t stream) {
  dqk_status st = check_cache(cache);
  if (st != DQK_OK) return st;
  if (dtype != DQK_F32 && dtype != DQK_BF16) return DQK_ERR_INVALID;
  if (!k_new || !v_new || !bmat || !n_new || max_new < 0) return DQK_ERR_INVALID;
  if (max_new == 0) return DQK_OK;
  if ((int64_t)max_new > cache->capacity) return DQK_ERR_INVALID;
  return from_hip(dqk::launch_append(*cache, k_new, v_new, dtype == DQK_BF16, bmat, n_new, max_new,
                                     reinterpret_cast<hipStream_t>(stream)));
}

dqk_status dqk_select_channels(const void *q, dqk_dtype dtype, const float *amat, int32_t batch,
                               int32_t hq, int32_t hkv, int32_t d, int32_t keep, float *q_prime,
                               int32_t *sel_idx, dqk_stream_t stream) {
  if (!q || !amat || !q_prime || !sel_idx) return DQK_ERR_INVALID;
  if (dtype != DQK_F32 && dtype != DQK_BF16) return DQK_ERR_INVALID;
  if (batch <= 0 || hq <= 0 || hkv <= 0 || hq % hkv != 0) return DQK_ERR_INVALID;
  if (!supported_dim(d) || !supported_group(hq, hkv)) return DQK_ERR_UNSUPPORTED;
  if (keep < 1 || keep > d) return DQK_ERR_INVALID;
  if ((int64_t)batch * hq > (1 << 30)) return DQK_ERR_INVALID;
  return from_hip(dqk::launch_select(q, dtype == DQK_BF16, amat, batch, hq, hkv, d, keep, q_prime,
                                     sel_idx, reinterpret_cast<hipStream_t>(stream)));
}

dqk_status dqk_append_select(const dqk_cache *cache, const void *k_new, const void *v_new,
                             const float *bmat, const int32_t *n_new, int32_t max_new,
                             const void *q, const float *amat, int32_t hq, int32_t keep,
                             dqk_dtype dtype, float *q_prime, int32_t *sel_idx,
                             dqk_stream_t stream) {
  dqk_status st = check_cache(cache);
  if (st != DQK_OK) return st;
  if (dtype != DQK_F32 && dtype != DQK_BF16) return DQK_ERR_INVALID;
  if (!k_new || !v_new || !bmat || !n_new || max_new < 0) return DQK_ERR_INVALID;
  if ((int64_t)max_new > cache->capacity) return DQK_ERR_INVALID;
  if (!q || !amat || !q_prime || !sel_idx) return DQK_ERR_INVALID;
  const int hkv = cache->num_kv_heads;
  if (hq <= 0 || hq % hkv != 0) return DQK_ERR_INVALID;
  if (!supported_group(hq, hkv)) return DQK_ERR_UNSUPPORTED;
  if (keep < 1 || keep > cache->head_dim) return DQK_ERR_INVALID;
  if ((int64_t)cache->batch * hq > (1 << 30)) return DQK_ERR_INVALID;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (max_new == 0)
    return from_hip(dqk::launch_select(q, dtype == DQK_BF16, amat, cache->batch, hq, hkv,
                                       cache->head_dim, keep, q_prime, sel_idx, s));
  return from_hip(dqk::launch_append_select(*cache, k_new, v_new, dtype == DQK_BF16, bmat, n_new,
                                            max_new, q, amat, hq, keep, q_prime, sel_idx, s));
}

dqk_status dqk_decode_workspace_bytes(const dqk_cache *cache, int32_t hq, int32_t split,
                                      size_t *out) {
  if (!out) return DQK_ERR_INVALID;
  dqk_status st = check_cache(cache);
  if (st != DQK_OK) return st;
  if (!supported_group(hq, cache->num_kv_heads)) return DQK_ERR_UNSUPPORTED;
  if (!valid_split(split)) return DQK_ERR_INVALID;
  *out = ws_bytes_for(cache->batch, cache->num_kv_heads, hq, cache->head_dim, cache->capacity,
                      decode_split(cache, hq, split));
  return DQK_OK;
}

}  // extern "C"

namespace {

// Validation and launch shared by the decode entry points (per-head or
// group-shared kept sets; the caller's workspace, or with use_scratch the
// library's device scratch, which then bounds the partials' size).
dqk_status decode_call(const dqk_cache *cache, const float *q_prime, const int32_t *sel_idx,
                       bool shared, int32_t hq, int32_t keep, float sm_scale, int32_t split,
                       float *out, void *workspace, size_t ws_bytes, dqk_stream_t stream,
                       bool use_scratch = false) {
  dqk_status st = check_cache(cache);
  if (st != DQK_OK) return st;
  if (!q_prime || !sel_idx || !out) return DQK_ERR_INVALID;
  if (!supported_group(hq, cache->num_kv_heads)) {
    if (hq <= 0 || hq % cache->num_kv_heads != 0) return DQK_ERR_INVALID;
    return DQK_ERR_UNSUPPORTED;
  }
  if (keep < 1 || keep > cache->head_dim) return DQK_ERR_INVALID;
  if (!isfinite(sm_scale)) return DQK_ERR_INVALID;
  if (!valid_split(split)) return DQK_ERR_INVALID;
  bool even = false;
  const int sp = decode_split(cache, hq, split, &even);
  const size_t need = ws_bytes_for(cache->batch, cache->num_kv_heads, hq, cache->head_dim,
                                   cache->capacity, sp);
  if (use_scratch) {
    if (need > dqk::kScratchBytes) return DQK_ERR_WORKSPACE;
    float *scratch = nullptr;
    if (dqk::decode_scratch(&scratch) != hipSuccess) return DQK_ERR_HIP;
    workspace = scratch;
  } else if (!workspace || ws_bytes < need || !aligned16(workspace)) {
    return DQK_ERR_WORKSPACE;
  }
  return from_hip(dqk::launch_decode(*cache, q_prime, sel_idx, shared, hq, keep, sm_scale, sp,
                                     even, out, static_cast<float *>(workspace),
                                     reinterpret_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

dqk_status dqk_decode_attention(const dqk_cache *cache, const float *q_prime,
                                const int32_t *sel_idx, int32_t hq, int32_t keep, float sm_scale,
                                int32_t split, float *out, void *workspace, size_t ws_bytes,
                                dqk_stream_t stream) {
  return decode_call(cache, q_prime, sel_idx, false, hq, keep, sm_scale, split, out, workspace,
                     ws_bytes, stream);
}

dqk_status dqk_decode_attention_noalloc(const dqk_cache *cache, const float *q_prime,
                                        const int32_t *sel_idx, int32_t hq, int32_t keep,
                                        float sm_scale, int32_t split, float *out,
                                        dqk_stream_t stream) {
  return decode_call(cache, q_prime, sel_idx, false, hq, keep, sm_scale, split, out, nullptr, 0,
                     stream, true);
}

dqk_status dqk_select_channels_shared(const void *q, dqk_dtype dtype, const float *amat,
                                      int32_t batch, int32_t hq, int32_t hkv, int32_t d,
                                      int32_t keep, float *q_prime, int32_t *sel_idx,
                                      dqk_stream_t stream) {
  if (!q || !amat || !q_prime || !sel_idx) return DQK_ERR_INVALID;
  if (dtype != DQK_F32 && dtype != DQK_BF16) return DQK_ERR_INVALID;
  if (batch <= 0 || hq <= 0 || hkv <= 0 || hq % hkv != 0) return DQK_ERR_INVALID;
  if (!supported_dim(d) || !supported_group(hq, hkv)) return DQK_ERR_UNSUPPORTED;
  if (keep < 1 || keep > d) return DQK_ERR_INVALID;
  if ((int64_t)batch * hq > (1 << 30)) return DQK_ERR_INVALID;
  return from_hip(dqk::launch_select_shared(q, dtype == DQK_BF16, amat, batch, hq, hkv, d, keep,
                                            q_prime, sel_idx,
                                            reinterpret_cast<hipStream_t>(stream)));
}

dqk_status dqk_decode_attention_shared(const dqk_cache *cache, const float *q_prime,
                                       const int32_t *sel_idx, int32_t hq, int32_t keep,
                                       float sm_scale, int32_t split, float *out,
                                       void *workspace, size_t ws_bytes, dqk_stream_t stream) {
  return decode_call(cache, q_prime, sel_idx, true, hq, keep, sm_scale, split, out, workspace,
                     ws_bytes, stream);
}

dqk_status dqk_cache_grow(const dqk_cache *src, const dqk_cache *dst, dqk_stream_t stream) {
  dqk_status st = check_cache(src);
  if (st != DQK_OK) return st;
  st = check_cache(dst);
  if (st != DQK_OK) return st;
  if (src->batch != dst->batch || src->num_kv_heads != dst->num_kv_heads ||
      src->head_dim != dst->head_dim || dst->capacity < src->capacity)
    return DQK_ERR_INVALID;
  // the two caches' planes must not overlap
  const size_t units = (size_t)src->batch * src->num_kv_heads, d = (size_t)src->head_dim;
  auto apart = [](const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x + na <= y || y + nb <= x;
  };
  const size_t cs = (size_t)src->capacity, cd = (size_t)dst->capacity;
  const void *sp[] = {src->k_codes, src->k_scales, src->k_ch0, src->k_tail, src->v_codes,
                      src->v_scales, src->lengths};
  const void *dp[] = {dst->k_codes, dst->k_scales, dst->k_ch0, dst->k_tail, dst->v_codes,
                      dst->v_scales, dst->lengths};
  const size_t sn[] = {units * d * (cs / 4), units * d * (cs / 32) * 2, units * cs * 2,
                       units * 32 * d * 4, units * (cs / 16) * d * 4, units * cs * (d / 32) * 2,
                       (size_t)src->batch * 8};
  const size_t dn[] = {units * d * (cd / 4), units * d * (cd / 32) * 2, units * cd * 2,
                       units * 32 * d * 4, units * (cd / 16) * d * 4, units * cd * (d / 32) * 2,
                       (size_t)dst->batch * 8};
  for (int i = 0; i < 7; ++i)
    for (int j = 0; j < 7; ++j)
      if (!apart(sp[i], sn[i], dp[j], dn[j])) return DQK_ERR_INVALID;
  return from_hip(dqk::launch_cache_grow(*src, *dst, reinterpret_cast<hipStream_t>(stream)));
}

dqk_status dqk_dequant_reference(const dqk_cache *cache, float *k_out, float *v_out,
                                 dqk_stream_t stream) {
  dqk_status st = check_cache(cache);
  if (st != DQK_OK) return st;
  if (!k_out || !v_out) return DQK_ERR_INVALID;
  return from_hip(dqk::launch_dequant(*cache, k_out, v_out, reinterpret_cast<hipStream_t>(stream)));
}

dqk_status dqk_bf16_decode_workspace_bytes(int32_t batch, int32_t hq, int32_t hkv, int32_t d,
                                           int32_t ld_t, int32_t split, size_t *out) {
  if (!out || batch <= 0 || ld_t <= 0) return DQK_ERR_INVALID;
  if (!supported_dim(d)) return DQK_ERR_UNSUPPORTED;
  if (!supported_group(hq, hkv)) return DQK_ERR_UNSUPPORTED;
  if (!valid_split(split)) return DQK_ERR_INVALID;
  *out = ws_bytes_for(batch, hkv, hq, d, ld_t, pick_split(split));
  return DQK_OK;
}

dqk_status dqk_bf16_decode_attention(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                     const int32_t *lengths, int32_t batch, int32_t hq,
                                     int32_t hkv, int32_t d, int32_t ld_t, float sm_scale,
                                     int32_t split, float *out, void *workspace, size_t ws_bytes,
                                     dqk_stream_t stream) {
  if (!q || !k || !v || !lengths || !out) return DQK_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return DQK_ERR_INVALID;
  if (batch <= 0 || ld_t <= 0 || hq <= 0 || hkv <= 0 || hq % hkv != 0) return DQK_ERR_INVALID;
  if (!supported_dim(d) || !supported_group(hq, hkv)) return DQK_ERR_UNSUPPORTED;
  if (!isfinite(sm_scale) || !valid_split(split)) return DQK_ERR_INVALID;
  const size_t need = ws_bytes_for(batch, hkv, hq, d, ld_t, pick_split(split));
  if (!workspace || ws_bytes < need || !aligned16(workspace)) return DQK_ERR_WORKSPACE;
  return from_hip(dqk::launch_bf16_decode(q, k, v, lengths, batch, hq, hkv, d, ld_t, sm_scale,
                                          pick_split(split), out, static_cast<float *>(workspace),
                                          reinterpret_cast<hipStream_t>(stream)));
}

dqk_status dqk_debug_f16_from_f32(const float *x, uint16_t *out, size_t n, dqk_stream_t stream) {
  if ((!x || !out) && n > 0) return DQK_ERR_INVALID;
  return from_hip(dqk::launch_f16_convert(x, out, n, reinterpret_cast<hipStream_t>(stream)));
}

dqk_status dqk_stream_read(const void *buf, size_t bytes, uint32_t *sink, dqk_stream_t stream) {
  if (!sink || !aligned16(sink) || bytes % 16 != 0) return DQK_ERR_INVALID;
  if (bytes > 0 && (!buf || !aligned16(buf))) return DQK_ERR_INVALID;
  return from_hip(dqk::launch_stream_read(buf, bytes, sink, dqk::kStreamReadSinkWords / 4, 4,
                                          reinterpret_cast<hipStream_t>(stream)));
}

dqk_status dqk_stream_read_config(const void *buf, size_t bytes, uint32_t *sink,
                                  int32_t workgroups, int32_t loads_in_flight,
                                  dqk_stream_t stream) {
  if (!sink || !aligned16(sink) || bytes % 16 != 0) return DQK_ERR_INVALID;
  if (bytes > 0 && (!buf || !aligned16(buf))) return DQK_ERR_INVALID;
  if (workgroups < 1 || workgroups > dqk::kStreamReadSinkWords / 4) return DQK_ERR_INVALID;
  if (loads_in_flight != 1 && loads_in_flight != 2 && loads_in_flight != 4 &&
      loads_in_flight != 8 && loads_in_flight != 16)
    return DQK_ERR_INVALID;
  return from_hip(dqk::launch_stream_read(buf, bytes, sink, workgroups, loads_in_flight,
                                          reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
