/*
 * dqk.h -- C ABI of the MI355X (gfx950) library for the Dual-QK decode step:
 * single-token attention over a 2-bit KV cache whose keys and queries pass
 * through paired transforms, reading only the key channels each query keeps.
 *
 * Source of the method: "Dual-QK: Sharp Queries and Flat Keys for Prunable
 * 2-bit KV Caches" (arXiv abstract) and the tech.dede.sh summary of it, sections
 * "Why the cache becomes a bottleneck", "Paired transforms instead of shared
 * rotation", "Results at 128K context" and "Throughput on SGLang".  The pages
 * fix the ingredients (paired non-orthogonal transforms, INT2 storage, channel-0
 * protection, query-channel pruning at a given sparsity); the concrete formats
 * and rules below are this library's definitions of them.
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless marked "host".  The caller owns all
 *    memory; the library allocates nothing and keeps no pointer after
 *    returning.  Its only process state is a per-device cache of the compute
 *    unit count (queried once per device on first use by the decode, never
 *    freed; it changes no result, only how a row's blocks are shared out over
 *    the splits) and, for dqk_decode_attention_noalloc only, that call's
 *    per-device scratch array and its looked-up address (below).  Calls are
 *    thread-safe, except that noalloc calls overlapping on one GPU race.
 *  - Work is enqueued on `stream` (0 = the null stream); no call synchronizes.
 *  - Every argument the host can see is validated before anything is launched:
 *    an invalid call returns an error status and launches nothing.  A launch
 *    failure returns DQK_ERR_HIP.  Conditions only the device can see (the
 *    contents of lengths/n_new/sel_idx, non-finite data) are preconditions; the
 *    kernels clamp counts and indices so they never write out of bounds.
 *
 * Cache layout, version 2 (per batch row b and KV head g, "unit" = b*hkv + g):
 *   k_codes  u8   [batch][hkv][d][cap/4]   key channel c, token t: byte t>>2 of the
 *                                          channel's row, bits 2(t&3) (channel-major,
 *                                          so a dropped channel is never read)
 *   k_scales f16  [batch][hkv][d][cap/32]  scale of (channel c, tokens 32j..32j+31)
 *   k_ch0    f16  [batch][hkv][cap]        key channel 0 of every token (protected)
 *   k_tail   f32  [batch][hkv][32][d]      exact transformed keys of the unfinished
 *                                          32-token group; row r valid for r < len%32
 *   v_codes  u32  [batch][hkv][cap/16][d]  value token t, channel c: 32-bit word
 *                                          (t>>4)*d + c, bits 2(t&15)
 *   v_scales f16  [batch][hkv][cap][d/32]  scale of (token t, channels 32j..32j+31)
 *   lengths  i32  [2][batch]               tokens stored per row, then one
 *                                          arrival counter per row that the append
 *                                          uses to commit the lengths (zero before
 *                                          and after every append)
 * A 2-bit code u with scale s stands for s*(2u-3).  Rows of channel 0 in
 * k_codes/k_scales exist but are never written or read.  All planes must be
 * zero-filled before the first append (the counters must start at zero; the
 * other planes then have byte-reproducible contents).
 */
#ifndef DQK_H
#define DQK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *dqk_stream_t; /* the same type as hipStream_t */

typedef enum {
    DQK_OK = 0,
    DQK_ERR_INVALID = -1,     /* bad pointer, size, shape or count */
    DQK_ERR_UNSUPPORTED = -2, /* valid in general, not built here (e.g. head_dim) */
    DQK_ERR_WORKSPACE = -3,   /* workspace missing or too small */
    DQK_ERR_HIP = -4          /* a HIP runtime call or launch failed */
} dqk_status;

typedef enum { DQK_F32 = 0, DQK_BF16 = 1 } dqk_dtype;

typedef struct {
    int32_t batch, num_kv_heads, head_dim, capacity; /* head_dim in {64, 128}; capacity % 32 == 0 */
    uint8_t *k_codes;
    uint16_t *k_scales;
    uint16_t *k_ch0;
    float *k_tail;
    uint32_t *v_codes;
    uint16_t *v_scales;
    int32_t *lengths;
} dqk_cache;

/* Human-readable name of a status (static string). */
const char *dqk_status_str(dqk_status s);

/* Host query, no device work: channels kept per query head at a query-channel
 * sparsity of sparsity_pct percent (tech.dede.sh summary, "Results at 128K
 * context": 40% query-channel sparsity).  *out_keep = floor((head_dim *
 * (100 - sparsity_pct) + 50) / 100), i.e. head_dim * (1 - s) rounded half up,
 * in integers; channel 0 counts toward it.  77 / 51 / 128 at head_dim 128 for
 * 40 / 60 / 0 %.  A result of 0 (sparsity 100) is not a valid keep for the
 * selection calls.  Errors: DQK_ERR_INVALID for a null out_keep, head_dim < 1
 * or sparsity_pct outside [0, 100]. */
dqk_status dqk_keep_count(int32_t head_dim, int32_t sparsity_pct, int32_t *out_keep);

/* Host query, no device work: byte sizes of the planes k_codes, k_scales, k_ch0,
 * k_tail, v_codes, v_scales, lengths for the given shape (out_bytes: host [7]). */
dqk_status dqk_cache_plane_bytes(int32_t batch, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t capacity, size_t *out_bytes);

/* Append step: each generated token's key and value join the cache for all later
 * decode steps (tech.dede.sh summary, "Why the cache becomes a bottleneck"); the
 * key goes through the key transform ("Paired transforms instead of shared
 * rotation"), keys and values are stored in 2 bits ("Throughput on SGLang"), and
 * channel 0 is protected (arXiv abstract).
 * For each batch row b, n = min(n_new[b], max_new, capacity - lengths[b]) tokens
 * k_new[b][g][i][:], v_new[b][g][i][:] (i < n) are stored at positions
 * lengths[b]..lengths[b]+n-1 of every KV head g, then lengths[b] += n:
 *   k' = k B_g, one fp32 fused-multiply-add chain per output channel over input
 *   channels in ascending order; k'_0 -> fp16 (round to nearest even, saturating
 *   at +-65504); k' -> k_tail row p%32; when position p closes its 32-token group,
 *   channels 1..d-1 of the group are quantized per channel; each value row is
 *   quantized in groups of 32 channels.  Quantizer: s = fp16(max|x|/3),
 *   u = [x >= -2s] + [x >= 0] + [x >= 2s].
 * k_new, v_new: [batch][hkv][max_new][head_dim] of `dtype`; bmat: [hkv][d][d] fp32
 * row-major; n_new: [batch] i32.  One kernel: the last of a row's workgroups to
 * finish writes the row's new length. */
dqk_status dqk_transform_quantize_append(const dqk_cache *cache, const void *k_new,
                                         const void *v_new, dqk_dtype dtype,
                                         const float *bmat, const int32_t *n_new,
                                         int32_t max_new, dqk_stream_t stream);

/* Query transform and channel selection: the query transform concentrates query
 * energy in few channels so that the rest can be dropped per query (tech.dede.sh
 * summary, "Paired transforms instead of shared rotation"; arXiv abstract,
 * dynamic channel pruning at a query-channel sparsity).  For each (b, query head h), with KV head g = h / (hq/hkv):
 * q' = q A_g (same FMA chain as above), written to q_prime; sel_idx receives, in
 * ascending order, channel 0 plus the keep-1 channels c >= 1 of largest |q'_c|,
 * equal magnitudes going to the lower index.
 * q: [batch][hq][d] of `dtype`; amat: [hkv][d][d] fp32; q_prime: [batch][hq][d]
 * fp32; sel_idx: [batch][hq][keep] i32; 1 <= keep <= d; hq/hkv in {1, 2, 4, 8}. */
dqk_status dqk_select_channels(const void *q, dqk_dtype dtype, const float *amat,
                               int32_t batch, int32_t hq, int32_t hkv, int32_t head_dim,
                               int32_t keep, float *q_prime, int32_t *sel_idx,
                               dqk_stream_t stream);

/* The append and the channel selection of one decode step in one launch: the
 * new token's keys and values and its query are all inputs of the step, and the
 * two parts share no data (tech.dede.sh summary, "Paired transforms instead of
 * shared rotation": keys and queries each pass through their own transform).
 * Same arguments, results and errors as dqk_transform_quantize_append followed
 * by dqk_select_channels, except: q, k_new and v_new share `dtype`; the
 * selection's batch and KV-head count are the cache's; hq / num_kv_heads in
 * {1, 2, 4, 8}.  One kernel.  With max_new == 0 only the selection runs. */
dqk_status dqk_append_select(const dqk_cache *cache, const void *k_new, const void *v_new,
                             const float *bmat, const int32_t *n_new, int32_t max_new,
                             const void *q, const float *amat, int32_t hq, int32_t keep,
                             dqk_dtype dtype, float *q_prime, int32_t *sel_idx,
                             dqk_stream_t stream);

/* Host query: workspace bytes dqk_decode_attention needs for this cache shape,
 * hq query heads and split length (split_tokens = 0: the library's choice). */
dqk_status dqk_decode_workspace_bytes(const dqk_cache *cache, int32_t hq,
                                      int32_t split_tokens, size_t *out_bytes);

/* Decode attention over the stored cache: the key channels a head does not keep
 * are never read from HBM; values are never pruned.  For each (b, h) with T = lengths[b]:
 *   z_t = sm_scale * sum_{c in sel_idx[b][h]} q'_c k~_{t,c}
 *   out[b][h] = sum_t softmax(z)_t v~_t        (T = 0 gives zeros)
 * where k~ is channel 0's fp16 value, the 2-bit value of complete groups, or the
 * exact tail.  Only the kept key channels' codes and scales are read from HBM.
 * The work is split along the sequence and the partial results are reduced with
 * an online-max combine.  split_tokens (a positive multiple of 32, or 0 for the
 * library's choice) fixes the number of splits, ceil(capacity / split_tokens).
 * For groups of 4 or 8 query heads per KV head and a capacity that is a multiple of
 * 64, the products run on the matrix cores with fp32 accumulation; there a multiple
 * of the kernel's block (256 tokens for groups of 4, 128 for groups of 8) gives each
 * split exactly its split_tokens tokens of every row, and other values share each
 * row's current blocks out over the splits.  Otherwise
 * split s covers tokens [s split_tokens, (s + 1) split_tokens).  The result does not
 * depend on the split beyond fp32 rounding.  With a single split (split_tokens >=
 * capacity) the decode writes out itself and the workspace is not touched.
 * q_prime: [batch][hq][d] fp32; sel_idx: [batch][hq][keep] as produced by
 * dqk_select_channels; out: [batch][hq][d] fp32; workspace: device scratch of at
 * least dqk_decode_workspace_bytes (contents need no initialization). */
dqk_status dqk_decode_attention(const dqk_cache *cache, const float *q_prime,
                                const int32_t *sel_idx, int32_t hq, int32_t keep,
                                float sm_scale, int32_t split_tokens, float *out,
                                void *workspace, size_t workspace_bytes,
                                dqk_stream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): dqk_decode_attention
 * without a workspace argument.  Same arguments, kernels, splits, results and
 * errors, except that the split partials go to the library's own device
 * scratch: one file-scope array of DQK_DECODE_SCRATCH_BYTES per GPU, held from
 * the library's load until the process ends.  Its device address is looked up
 * once per device, on the first call with that device current.  The call
 * allocates nothing (no hipMalloc or hipFree, no allocating library routine).
 * Errors: DQK_ERR_WORKSPACE when the partials this shape and split need
 * (dqk_decode_workspace_bytes) exceed DQK_DECODE_SCRATCH_BYTES; DQK_ERR_HIP if
 * the scratch address cannot be looked up.  Every call on one GPU uses that
 * GPU's one array: calls that overlap on a GPU (on different streams or host
 * threads) race and must be ordered by the caller.  The array keeps the last
 * call's contents; no call needs it cleared. */
#define DQK_DECODE_SCRATCH_BYTES ((size_t)16 << 20)
dqk_status dqk_decode_attention_noalloc(const dqk_cache *cache, const float *q_prime,
                                        const int32_t *sel_idx, int32_t hq, int32_t keep,
                                        float sm_scale, int32_t split_tokens, float *out,
                                        dqk_stream_t stream);

/* Group-shared channel selection: one kept set for all query heads of a KV head,
 * so that under grouped-query attention the channels dropped are dropped for the
 * whole group and leave the key reads (tech.dede.sh summary, "Throughput on
 * SGLang": pruning removes key channels from the cache reads; the pages state
 * the selection per query, and this group rule is the library's reading of it
 * for grouped heads).  q' is written exactly as by dqk_select_channels.  For each
 * (b, KV head g): score_c = |q'_{h0,c}| + |q'_{h0+1,c}| + ... over the group's
 * query heads h0 = g*(hq/hkv).. in ascending order, added in fp32 from +0;
 * sel_idx[b][g] receives, ascending, channel 0 plus the keep-1 channels c >= 1 of
 * largest score, equal scores going to the lower index.
 * q: [batch][hq][d] of `dtype`; amat: [hkv][d][d] fp32; q_prime: [batch][hq][d]
 * fp32; sel_idx: [batch][hkv][keep] i32; 1 <= keep <= d; hq/hkv in {1, 2, 4, 8}.
 * Errors as dqk_select_channels. */
dqk_status dqk_select_channels_shared(const void *q, dqk_dtype dtype, const float *amat,
                                      int32_t batch, int32_t hq, int32_t hkv, int32_t head_dim,
                                      int32_t keep, float *q_prime, int32_t *sel_idx,
                                      dqk_stream_t stream);

/* Decode attention with group-shared kept sets: exactly dqk_decode_attention with
 * every query head h of KV head g using the set sel_idx[b][g] (as produced by
 * dqk_select_channels_shared, [batch][hkv][keep]).  The key channels outside the
 * set are not read for the group.  Same workspace (dqk_decode_workspace_bytes),
 * splits, results and errors. */
dqk_status dqk_decode_attention_shared(const dqk_cache *cache, const float *q_prime,
                                       const int32_t *sel_idx, int32_t hq, int32_t keep,
                                       float sm_scale, int32_t split_tokens, float *out,
                                       void *workspace, size_t workspace_bytes,
                                       dqk_stream_t stream);

/* Growing a cache: the cache grows with every generated token (tech.dede.sh
 * summary, "Why the cache becomes a bottleneck"), and a sequence that outgrows
 * the capacity its cache was created with moves to a larger one.  Copies every
 * plane of src into dst, which has the same batch, num_kv_heads and head_dim and
 * capacity >= src's: each unit's rows of src go to the start of dst's rows, and
 * the lengths plane (lengths and arrival counters) is copied whole.  Nothing
 * stored depends on the capacity, so when dst's planes were zero-filled the
 * result is byte for byte the cache that the same appends would have built at
 * dst's capacity; later appends and decodes on dst continue as on src.  dst's
 * positions past src's capacity keep their contents.  Must not run concurrently
 * with an append to src.  Errors: DQK_ERR_INVALID for an invalid cache, shapes
 * that differ, a smaller dst capacity, or planes of src and dst that overlap. */
dqk_status dqk_cache_grow(const dqk_cache *src, const dqk_cache *dst, dqk_stream_t stream);

/* Dense dequantized cache for checking and inspection: k_out, v_out
 * [batch][hkv][capacity][d] fp32 hold k~ and v~ as defined above for t < len and
 * zero past it.  Not on the decode path. */
dqk_status dqk_dequant_reference(const dqk_cache *cache, float *k_out, float *v_out,
                                 dqk_stream_t stream);

/* Unpruned BF16 decode, the comparison the pages measure against ("relative to
 * unpruned BF16"): out[b][h] = softmax(sm_scale * q K^T) V over raw bf16 keys and
 * values, no transforms, no quantization, fp32 accumulation.
 * q: [batch][hq][d] bf16; k, v: [batch][hkv][ld_t][d] bf16 (token-major);
 * lengths: [batch] i32 (<= ld_t); out: [batch][hq][d] fp32; workspace as for
 * dqk_decode_attention, sized by dqk_bf16_decode_workspace_bytes.  q, k and v
 * must be 16-byte aligned (DQK_ERR_INVALID otherwise).  The logits are fp32 sums
 * of the exact bf16 products; with the same inputs the result does not depend
 * on the split beyond fp32 rounding. */
dqk_status dqk_bf16_decode_workspace_bytes(int32_t batch, int32_t hq, int32_t hkv,
                                           int32_t head_dim, int32_t ld_t,
                                           int32_t split_tokens, size_t *out_bytes);
dqk_status dqk_bf16_decode_attention(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                     const int32_t *lengths, int32_t batch, int32_t hq,
                                     int32_t hkv, int32_t head_dim, int32_t ld_t,
                                     float sm_scale, int32_t split_tokens, float *out,
                                     void *workspace, size_t workspace_bytes,
                                     dqk_stream_t stream);

/* Diagnostic: the device's fp32 -> fp16 conversion used for every stored scale
 * and channel-0 key (round to nearest even, subnormals kept, saturating at
 * +-65504), element-wise over n values.  x: [n] fp32, out: [n] u16. */
dqk_status dqk_debug_f16_from_f32(const float *x, uint16_t *out, size_t n,
                                  dqk_stream_t stream);

/* Measurement aid, not part of the method: reads `bytes` of device memory at buf
 * once with 16-byte loads (a plain streaming kernel, 2048 workgroups of 256
 * threads) and leaves in sink a fold of what it read: the XOR of the
 * DQK_STREAM_READ_SINK_WORDS sink words equals the XOR of every 32-bit word of
 * the buffer.  Its run time over a buffer far larger than the 256 MB Infinity
 * Cache gives the read rate a plain kernel reaches, against which the decode's
 * byte rate is read.  buf: 16-byte aligned, bytes a multiple of 16 (0 is a valid
 * no-op read that still writes zeros); sink: device u32 [DQK_STREAM_READ_SINK_WORDS],
 * every word overwritten.  Errors: DQK_ERR_INVALID for null or misaligned
 * pointers or sizes. */
#define DQK_STREAM_READ_SINK_WORDS 8192
dqk_status dqk_stream_read(const void *buf, size_t bytes, uint32_t *sink, dqk_stream_t stream);

/* The same probe with its launch shape as arguments, for a sweep of the read
 * rate: `workgroups` workgroups of 256 threads (1 .. DQK_STREAM_READ_SINK_WORDS/4;
 * dqk_stream_read uses the maximum) and loads_in_flight 16-byte loads per thread
 * and iteration (1, 2, 4, 8 or 16; dqk_stream_read uses 4).  The XOR of the first
 * 4 * workgroups sink words equals the XOR of the buffer's 32-bit words; the other
 * sink words are not written.  Errors: DQK_ERR_INVALID as dqk_stream_read, or for
 * a launch shape outside these ranges. */
dqk_status dqk_stream_read_config(const void *buf, size_t bytes, uint32_t *sink,
                                  int32_t workgroups, int32_t loads_in_flight,
                                  dqk_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif
