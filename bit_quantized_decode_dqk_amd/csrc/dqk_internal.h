// Internal declarations shared by the HIP sources of libdqk (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dqk.h"

namespace dqk {

constexpr int kGroup = 32;          // tokens (keys) or channels (values) per scale
constexpr int kDefaultSplit = 1024; // bf16 decode split length when the caller passes 0

// Default 2-bit decode split: the capacity spread over about two resident
// workgroups per compute unit on 256 compute units, rounded down to 256-token
// steps (at least 256).  Rounding down keeps every full split inside the first
// wave of workgroups; the short last split of each sequence is launched last.
// Groups of four query heads share the sequence by length (each workgroup takes
// an equal share of the current tokens): the default only fixes the number of
// splits, about two workgroups per compute unit, with at least 256 tokens of
// capacity per split.  `workgroups` is the number of workgroups per split index
// (units times the four-head slices of a group).
inline int balanced_decode_split(int capacity, int workgroups) {
  int nsplit = 512 / workgroups;
  if (nsplit < 1) nsplit = 1;
  const int most = (capacity + 255) / 256;
  if (nsplit > most) nsplit = most;
  const int split = (capacity + nsplit - 1) / nsplit;
  return (split + 31) / 32 * 32;
}

// Default split of the matrix-core decode.  When the capacity alone gives more
// than kFixedSplitBlocks blocks of 256 tokens per resident workgroup slot (512),
// fixed splits of that many whole blocks (two chunks of the kernel: ten blocks,
// then ten and an extra one): work items then outnumber the slots several times
// and the dispatcher evens out rows of different lengths.  Otherwise the balanced
// split count above, each split taking an equal share of its row's current blocks
// (even = true).
constexpr int kFixedSplitBlocks = 21;
struct DecodeSplit {
  int split;
  bool even;
};
inline DecodeSplit matrix_decode_split(int capacity, int workgroups) {
  const long long blocks = (long long)workgroups * ((capacity + 255) / 256);
  if (blocks > (long long)kFixedSplitBlocks * 512) return {kFixedSplitBlocks * 256, false};
  return {balanced_decode_split(capacity, workgroups), true};
}

inline int default_decode_split(int capacity, int units) {
  const long long slots = 2 * 256LL;
  const long long per = ((long long)capacity * units) / slots;
  const int s = (int)(per / 256 * 256);
  return s < 256 ? 256 : s;
}

// fp32 -> binary16 bits: round to nearest even (the hardware conversion), with
// subnormals, and finite values past the largest binary16 clamped to +-65504.
__device__ __forceinline__ uint16_t f16_bits(float x) {
  x = fminf(fmaxf(x, -65504.0f), 65504.0f);
  _Float16 h = (_Float16)x;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_value(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

__device__ __forceinline__ float bf16_value(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// Code u of a 2-bit group with scale s stands for s*(2u-3).
__device__ __forceinline__ float level_of(uint32_t u) { return (float)(int)(2u * u) - 3.0f; }

// 2-bit code of x for the grid s*{-3,-1,1,3}: thresholds -2s, 0, 2s, ties upward.
__device__ __forceinline__ uint32_t code_of(float x, float two_s) {
  return (uint32_t)(x >= -two_s) + (uint32_t)(x >= 0.0f) + (uint32_t)(x >= two_s);
}

struct Shape {
  int batch, hkv, d, cap;
};

// Element offsets of the planes for one unit (batch row b, KV head g).
__host__ __device__ __forceinline__ size_t unit_index(const dqk_cache &c, int b, int g) {
  return (size_t)b * c.num_kv_heads + g;
}

// Compute units of the current device (cached per device; 0 if the query fails).
int compute_units();

// Launchers (return the launch error, if any).
hipError_t launch_append(const dqk_cache &c, const void *k_new, const void *v_new, bool bf16,
                         const float *bmat, const int32_t *n_new, int max_new, hipStream_t s);
hipError_t launch_select(const void *q, bool bf16, const float *amat, int batch, int hq, int hkv,
                         int d, int keep, float *q_prime, int32_t *sel_idx, hipStream_t s);
// the append and the selection of one step in one launch;
// q, k_new and v_new share one dtype, the selection's batch and KV heads are the cache's
hipError_t launch_append_select(const dqk_cache &c, const void *k_new, const void *v_new,
                                bool bf16, const float *bmat, const int32_t *n_new, int max_new,
                                const void *q, const float *amat, int hq, int keep,
                                float *q_prime, int32_t *sel_idx, hipStream_t s);
// even: the split length is the library's choice (each split then takes an equal
// share of its row's current blocks), not the caller's
hipError_t launch_decode(const dqk_cache &c, const float *q_prime, const int32_t *sel_idx, int hq,
                         int keep, float sm_scale, int split, bool even, float *out, float *ws,
                         hipStream_t s);
// the matrix-core decode: groups of a multiple of four query heads, capacity a multiple of 64
bool decode4_supported(const dqk_cache &c, int hq);
hipError_t launch_decode4(const dqk_cache &c, const float *q_prime, const int32_t *sel_idx, int hq,
                          int keep, float scale2, int split, bool even, float *ws, hipStream_t s);
hipError_t launch_dequant(const dqk_cache &c, float *k_out, float *v_out, hipStream_t s);
hipError_t launch_bf16_decode(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const int32_t *lengths, int batch, int hq, int hkv, int d, int ld_t,
                              float sm_scale, int split, float *out, float *ws, hipStream_t s);
hipError_t launch_combine(const float *ws, int batch, int hq, int hkv, int d, int nsplit,
                          float *out, hipStream_t s);
hipError_t launch_f16_convert(const float *x, uint16_t *out, size_t n, hipStream_t s);
constexpr int kStreamReadSinkWords = DQK_STREAM_READ_SINK_WORDS;   // 2048 workgroups x 4 wavefronts
hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t s);

// Workspace: per work item (unit, split) and query head of its group:
// m, l, two pad floats (keeps o 16-byte aligned), o[d].
constexpr int kPartialHead = 4;
inline size_t partial_floats(int d) { return (size_t)d + kPartialHead; }
inline int num_splits(int cap_tokens, int split) { return (cap_tokens + split - 1) / split; }

}  // namespace dqk
