// Host-side internal declarations of libdqk (not installed): constants, split
// rules, the workspace layout and the kernel launchers.  Needs only the HIP
// runtime API, so the host layer also builds with a plain C++ compiler (the
// sanitizer test of the host layer does that).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/dqk.h"

namespace dqk {

constexpr int kGroup = 32;          // tokens (keys) or channels (values) per scale
constexpr int kDefaultSplit = 2048; // bf16 decode split length when the caller passes 0

// Default 2-bit decode split: the capacity spread over about two resident
// workgroups per compute unit on 256 compute units, rounded down to 256-token
// steps (at least 256).  Rounding down keeps every full split inside the first
// wave of workgroups; the short last split of each sequence is launched last.
// Groups of four query heads share the sequence by length (each workgroup takes
// an equal share of the current tokens): the default only fixes the number of
// splits, about two workgroups per compute unit, with at least 256 tokens of
// capacity per split.  `workgroups` is the number of workgroups per split index:
// the units (batch rows times KV heads), one workgroup each.
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

// Default split of the eight-head matrix-core decode (one workgroup per work
// item, blocks of 128 tokens, the same chunks of ten blocks): the rule above in
// its blocks -- fixed splits of kFixedSplitBlocks8 whole blocks when the capacity
// alone gives more than that many per resident workgroup slot, else the balanced
// split count with equal (or uneven, two workgroups per compute unit) shares.
constexpr int kFixedSplitBlocks8 = 31;
inline DecodeSplit matrix_decode_split8(int capacity, int units) {
  const long long blocks = (long long)units * ((capacity + 127) / 128);
  if (blocks > (long long)kFixedSplitBlocks8 * 512) return {kFixedSplitBlocks8 * 128, false};
  return {balanced_decode_split(capacity, units), true};
}

// Blocks of 256 tokens per chunk of the matrix-core decode: a chunk's logits
// stay in registers; a share of kDecodeChunkBlocks + 1 blocks still runs as one
// chunk, so n blocks take max(1, (n - 2) / kDecodeChunkBlocks + 1) chunks.
constexpr int kDecodeChunkBlocks = 10;

// Uneven shares of a row's nblk blocks over nsplit splits in the matrix-core
// decode when two workgroups share each compute unit: fs first-slot splits
// (dispatched first on their unit), the rest second-slot.  The first workgroup
// on a unit issues ahead of the second (older wavefronts win the issue
// arbitration) and would finish well before it, so the second-slot splits take
// 7/8 of the average share, rounded down, all the same, and the first-slot
// splits share the rest.  No split may need a chunk more than an even share:
// with shares of one chunk the first-slot splits take at most a chunk's blocks
// each, with longer shares at most a chunk's blocks per chunk of the even
// share; the second-slot share is raised until the rest fits, and where it
// would then exceed the even share the row is shared evenly (second = -1).
// The last split takes one block less (cut = 1) when it also works out the
// exact logits of an unfinished last key group.  Shares apply from 4 to 50
// blocks per split on average.  The arithmetic is 32-bit: the library uses the
// rule only with nsplit at most twice the compute units (below 4096) and fs at
// least (nsplit - 1) / 2, so that every product stays below 2^32.  (constexpr:
// the same function runs in the kernel and in the host-side checks.)
struct SplitShares {
  int second;        // blocks of each second-slot split (-1: share evenly)
  int first_total;   // blocks of the fs first-slot splits together
};
constexpr SplitShares uneven_shares(int nblk, int nsplit, int fs, int cut) {
  const int ss = nsplit - fs;
  if (fs <= 0 || ss <= 0 || nblk < 4 * nsplit || nblk > 50 * nsplit) return {-1, 0};
  const int e = (nblk + nsplit - 1) / nsplit;                        // the even share
  const bool one = nblk <= kDecodeChunkBlocks * fs + 8 * ss;         // shares of one chunk
  const int cap1 = one ? kDecodeChunkBlocks : kDecodeChunkBlocks * ((e - 2) / kDecodeChunkBlocks + 1);
  const uint32_t wt = 9u * (uint32_t)fs + 7u * (uint32_t)ss;
  const int w = (int)((7u * (uint32_t)nblk) / wt);
  const int fit = (nblk + cut - cap1 * fs + ss - 1) / ss;
  const int a2 = w > fit ? w : fit;
  if (!one && a2 > e) return {-1, 0};
  return {a2, nblk - a2 * ss + cut};
}

// Blocks [lo, hi) of split s under uneven shares: the first-slot splits share
// their total evenly, the second-slot splits follow with sh.second blocks each
// and the last one ends the row.
struct BlockRange {
  int lo, hi;
};
constexpr BlockRange uneven_split_range(SplitShares sh, int s, int fs, int nsplit, int nblk) {
  if (s < fs)
    return {(int)(((uint32_t)sh.first_total * (uint32_t)s) / (uint32_t)fs),
            (int)(((uint32_t)sh.first_total * (uint32_t)(s + 1)) / (uint32_t)fs)};
  const int lo = sh.first_total + sh.second * (s - fs);
  return {lo, s == nsplit - 1 ? nblk : lo + sh.second};
}

// Default split of the general decode: about two workgroups per CU, splits of 256
// tokens or more.  (One split of a 1024-token row, which needs no combine launch,
// measured slower in a replayed step: 18.6 against 12.9 us for select + decode.)
inline int default_decode_split(int capacity, int units) {
  const long long slots = 2 * 256LL;
  const long long per = ((long long)capacity * units) / slots;
  const int s = (int)(per / 256 * 256);
  return s < 256 ? 256 : s;
}

struct Shape {
  int batch, hkv, d, cap;
};

// Compute units of the current device (cached per device; 0 if the query fails).
int compute_units();

// Launchers (return the launch error, if any).
hipError_t launch_append(const dqk_cache &c, const void *k_new, const void *v_new, bool bf16,
                         const float *bmat, const int32_t *n_new, int max_new, hipStream_t s);
hipError_t launch_select(const void *q, bool bf16, const float *amat, int batch, int hq, int hkv,
                         int d, int keep, float *q_prime, int32_t *sel_idx, hipStream_t s);
// one kept set per (batch row, KV head), scored over the group's heads; sel_idx [batch][hkv][keep]
hipError_t launch_select_shared(const void *q, bool bf16, const float *amat, int batch, int hq,
                                int hkv, int d, int keep, float *q_prime, int32_t *sel_idx,
                                hipStream_t s);
// the append and the selection of one step in one launch;
// q, k_new and v_new share one dtype, the selection's batch and KV heads are the cache's
hipError_t launch_append_select(const dqk_cache &c, const void *k_new, const void *v_new,
                                bool bf16, const float *bmat, const int32_t *n_new, int max_new,
                                const void *q, const float *amat, int hq, int keep,
                                float *q_prime, int32_t *sel_idx, hipStream_t s);
// even: the split length is the library's choice (each split then takes an equal
// share of its row's current blocks), not the caller's; shared: sel_idx holds one
// kept set per (batch row, KV head) [batch][hkv][keep] instead of one per query head
hipError_t launch_decode(const dqk_cache &c, const float *q_prime, const int32_t *sel_idx,
                         bool shared, int hq, int keep, float sm_scale, int split, bool even,
                         float *out, float *ws, hipStream_t s);
// the matrix-core decodes: groups of four (hq == 4 hkv) or eight (hq == 8 hkv) query
// heads, per-head or group-shared kept sets, capacity a multiple of 64; partials to
// ws, or (out != nullptr, one split per row) the normalized output to out
bool decode4_supported(const dqk_cache &c, int hq);
hipError_t launch_decode4(const dqk_cache &c, const float *q_prime, const int32_t *sel_idx,
                          bool shared, int hq, int keep, float scale2, int split, bool even,
                          float *ws, float *out, hipStream_t s);
bool decode8_supported(const dqk_cache &c, int hq);
hipError_t launch_decode8(const dqk_cache &c, const float *q_prime, const int32_t *sel_idx, bool shared,
                          int hq, int keep, float scale2, int split, bool even, float *ws, float *out,
                          hipStream_t s);
hipError_t launch_dequant(const dqk_cache &c, float *k_out, float *v_out, hipStream_t s);
// every plane of src re-strided into dst (same batch, KV heads, head_dim; larger capacity)
hipError_t launch_cache_grow(const dqk_cache &src, const dqk_cache &dst, hipStream_t s);
hipError_t launch_bf16_decode(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const int32_t *lengths, int batch, int hq, int hkv, int d, int ld_t,
                              float sm_scale, int split, float *out, float *ws, hipStream_t s);
hipError_t launch_combine(const float *ws, int batch, int hq, int hkv, int d, int nsplit,
                          float *out, hipStream_t s);
hipError_t launch_f16_convert(const float *x, uint16_t *out, size_t n, hipStream_t s);
constexpr int kStreamReadSinkWords = DQK_STREAM_READ_SINK_WORDS;   // 2048 workgroups x 4 wavefronts
// workgroups of 256 threads (1 .. kStreamReadSinkWords / 4), loads_in_flight in {1, 2, 4, 8, 16}
hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, int workgroups,
                              int loads_in_flight, hipStream_t s);

// Device scratch of the decode entry point that allocates nothing: the split
// partials of one call, at most kScratchBytes (one file-scope device array per
// GPU).  decode_scratch gives the array's device address on the current device
// (looked up on the first call per device and kept).
constexpr size_t kScratchBytes = (size_t)16 << 20;
hipError_t decode_scratch(float **ptr);

// Workspace: per work item (unit, split) and query head of its group:
// m, l, two pad floats (keeps o 16-byte aligned), o[d].
constexpr int kPartialHead = 4;
inline size_t partial_floats(int d) { return (size_t)d + kPartialHead; }
inline int num_splits(int cap_tokens, int split) { return (cap_tokens + split - 1) / split; }

}  // namespace dqk
