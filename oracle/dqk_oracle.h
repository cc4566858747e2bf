/*
 * dqk_oracle.h -- plain CPU reference for the Dual-QK decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  This library exists to check the GPU library: only
 * the tests, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header, table or helper with the GPU library.
 *
 * What it computes (Dual-QK, "Sharp Queries and Flat Keys for Prunable 2-bit KV
 * Caches"; arXiv abstract, and the tech.dede.sh summary sections "Paired
 * transforms instead of shared rotation", "Results at 128K context" and
 * "Throughput on SGLang"):
 *   - paired transforms q' = q A, k' = k B (row vectors, A B^T = I, so that
 *     q'.k' = q.k, the invariance the abstract requires of any transform pair);
 *   - keys and values stored as 2-bit codes with an fp16 scale per group of 32;
 *     key channel 0 kept in fp16 ("channel-0 protection");
 *   - per query head, keep channel 0 plus the top-(keep-1) other channels by
 *     |q'| ("dynamic channel pruning" at a given query-channel sparsity);
 *   - attention over the stored cache using only the kept key channels.
 * The pages give no formulas for the quantizer, the bit layout, the selection
 * rule or the arithmetic; the readings used here are listed next to each
 * function.  Attention sums run in fp64.
 *
 * Cache layout (one definition, restated independently by the GPU library):
 *   k_codes  u8   [batch][hkv][d][cap/4]     key channel c, token t: byte t>>2, bits 2(t&3)
 *   k_scales f16  [batch][hkv][d][cap/32]    one scale per (channel, 32-token group)
 *   k_ch0    f16  [batch][hkv][cap]          channel 0 of every token
 *   k_tail   f32  [batch][hkv][32][d]        exact k' of the unfinished group
 *                                            (row r defined for r < len mod 32)
 *   v_codes  u32  [batch][hkv][cap/16][d]    value token t, channel c:
 *                                            word (t>>4)*d + c, bits 2(t&15)
 *   v_scales f16  [batch][hkv][cap][d/32]    one scale per (token, 32-channel group)
 *   lengths  i32  [batch]
 * Key channel 0 has rows in k_codes/k_scales that are never written or read.
 */
#ifndef DQK_ORACLE_H
#define DQK_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int32_t batch, hkv, d, cap;
    uint8_t *k_codes;
    uint16_t *k_scales;
    uint16_t *k_ch0;
    float *k_tail;
    uint32_t *v_codes;
    uint16_t *v_scales;
    int32_t *lengths;
} dqko_cache;

/* IEEE binary16 from fp32: round to nearest even, subnormals kept, finite
 * values that would round to infinity saturate to +-65504. */
uint16_t dqko_f16_from_f32(float x);
float dqko_f32_from_f16(uint16_t h);
/* Element-wise over arrays of n values (for exhaustive checks). */
void dqko_f16_from_f32_n(const float *x, size_t n, uint16_t *out);
void dqko_f32_from_f16_n(const uint16_t *h, size_t n, float *out);

/* y = x M for a row vector x[d] and row-major M[d][d]; each y_j is one fp32
 * fused-multiply-add chain over i = 0..d-1 in ascending order from +0. */
void dqko_transform(const float *x, const float *m, int d, float *y);

/* 2-bit quantizer for 32 values x[i*stride]: sigma = f16(max|x| / 3),
 * codes u = [x >= -2s] + [x >= 0] + [x >= 2s] with s = float(sigma);
 * the value of code u is s*(2u-3). */
void dqko_quantize32(const float *x, ptrdiff_t stride, uint16_t *sigma, uint8_t *codes);

/* keep = floor((d*(100-sparsity_pct) + 50) / 100): channels kept per query. */
int dqko_keep_count(int d, int sparsity_pct);

/* Channel selection for one query head: channel 0, then the keep-1 channels
 * c >= 1 with the largest |q'_c| (equal magnitudes: lower index first), written
 * in ascending order to idx[keep]. */
void dqko_select(const float *qp, int d, int keep, int32_t *idx);

/* q' and the selection for a batch of queries: q[batch][hq][d], A[hkv][d][d];
 * query head h uses KV head h / (hq/hkv). */
void dqko_queries(const float *q, const float *a, int batch, int hq, int hkv, int d,
                  int keep, float *qp, int32_t *idx);

/* Group-shared selection for the grp query heads of one KV head, qp[grp][d]:
 * score_c = |q'_{0,c}| + |q'_{1,c}| + ... in fp32 from +0 in ascending head
 * order; channel 0 plus the keep-1 channels c >= 1 of largest score (equal
 * scores: lower index first), ascending, to idx[keep]. */
void dqko_select_shared(const float *qp, int grp, int d, int keep, int32_t *idx);

/* q' [batch][hq][d] as dqko_queries, and one group-shared kept set per (batch
 * row, KV head): idx [batch][hkv][keep]. */
void dqko_queries_shared(const float *q, const float *a, int batch, int hq, int hkv, int d,
                         int keep, float *qp, int32_t *idx);

/* Append n_new[b] tokens per batch row (clamped to max_new and to the free
 * capacity).  k_new, v_new: [batch][hkv][max_new][d] fp32; bm: [hkv][d][d].
 * Writes the new tokens at positions lengths[b].., then lengths[b] += n. */
void dqko_append(const dqko_cache *c, const float *k_new, const float *v_new,
                 const float *bm, const int32_t *n_new, int32_t max_new);

/* Copy every stored element of src to the same (unit, channel, token) place of
 * dst, whose batch, hkv and d are src's and whose cap is at least src's. */
void dqko_cache_grow(const dqko_cache *src, const dqko_cache *dst);

/* Dense dequantized cache: k_out, v_out [batch][hkv][cap][d]; zero past lengths. */
void dqko_dequant(const dqko_cache *c, float *k_out, float *v_out);

/* Attention of one query head over dense keys/values [t_len][d] (row stride
 * ld), using only channels idx[0..keep-1] of q' and the keys:
 * z_t = sm * sum_c q'_c k_tc (fp64), o = softmax(z) V (fp64), rounded to fp32. */
void dqko_attend_dense(const float *qp, const int32_t *idx, int keep, const float *k,
                       const float *v, int t_len, int d, ptrdiff_t ld, double sm,
                       float *out);

/* Decode attention over the stored cache for all (batch, query head).
 * qp [batch][hq][d], idx [batch][hq][keep], out [batch][hq][d].
 * heads_mask: NULL for all heads, else [batch*hq] flags (nonzero = compute;
 * skipped heads are left untouched).  nthreads: OpenMP threads (0 = default). */
void dqko_decode(const dqko_cache *c, const float *qp, const int32_t *idx, int hq, int keep,
                 double sm, float *out, const uint8_t *heads_mask, int nthreads);

/* Plain attention on raw inputs, fp64: q [batch][hq][d], k/v [batch][hkv][ld_t][d]. */
void dqko_plain_attention(const float *q, const float *k, const float *v,
                          const int32_t *lengths, int batch, int hq, int hkv, int d,
                          int ld_t, double sm, float *out);

/* Bytes of the stored cache and of the per-query inputs/outputs that a decode
 * must touch, found by marking every byte the decode above reads or writes.
 * out[0..6] = k_codes, k_scales, k_ch0, k_tail, v_codes, v_scales,
 * per-query (q' of kept channels, idx, out). */
void dqko_decode_bytes(const dqko_cache *c, const int32_t *idx, int hq, int keep,
                       uint64_t out[7]);

#ifdef __cplusplus
}
#endif
#endif
