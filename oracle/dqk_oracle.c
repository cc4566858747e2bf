/*
 * dqk_oracle.c -- plain, slow CPU reference for the Dual-QK decode path.
 *
 * TEST INFRASTRUCTURE ONLY (see dqk_oracle.h).  Written for reading, not speed:
 * scalar loops, one query head at a time, fp64 attention sums.  Built with
 * -ffp-contract=off so that every fused multiply-add below is an explicit fmaf.
 *
 * Sources: Dual-QK arXiv abstract; tech.dede.sh summary of Dual-QK, sections
 * "Why the cache becomes a bottleneck", "Paired transforms instead of shared
 * rotation", "Results at 128K context", "Throughput on SGLang".  Where the pages
 * leave a step open, the reading taken is stated at the function.
 */
#include "dqk_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ fp16 */

/* binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits.  Reading: round to
 * nearest even, keep subnormals, saturate at the largest finite value (the pages
 * only say "fp16 scale"). */
uint16_t dqko_f16_from_f32(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return (uint16_t)(sign | 0x7e00u);      /* NaN */
    if (a >= 0x477ff000u) return (uint16_t)(sign | 0x7bffu);     /* >= 65520: saturate */
    uint32_t e32 = a >> 23;
    uint32_t m = a & 0x7fffffu;
    if (e32 >= 113) {                 /* >= 2^-14: a normal binary16 */
        uint32_t h = ((e32 - 112) << 10) | (m >> 13);
        uint32_t rest = m & 0x1fffu;
        if (rest > 0x1000u || (rest == 0x1000u && (h & 1u))) h += 1; /* may carry into exponent */
        return (uint16_t)(sign | h);
    }
    if (e32 == 0) return sign;        /* fp32 zero or subnormal: far below 2^-25 */
    /* Subnormal binary16: value = q * 2^-24.  x = (2^23 + m) * 2^(e32-150),
     * so q = (2^23 + m) / 2^(126 - e32), rounded to nearest even. */
    uint32_t full = m | 0x800000u;
    uint32_t shift = 126 - e32;       /* >= 14 */
    if (shift > 25) return sign;      /* below half of 2^-24 */
    uint32_t q = full >> shift;
    uint32_t rem = full & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u))) q += 1;          /* may reach 0x400 */
    return (uint16_t)(sign | q);
}

float dqko_f32_from_f16(uint16_t h)
{
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    float v;
    if (e == 0) v = ldexpf((float)f, -24);
    else if (e == 31) v = f ? NAN : INFINITY;
    else v = ldexpf((float)(1024 + f), e - 25);
    return (h & 0x8000) ? -v : v;
}

void dqko_f16_from_f32_n(const float *x, size_t n, uint16_t *out)
{
    for (size_t i = 0; i < n; ++i) out[i] = dqko_f16_from_f32(x[i]);
}

void dqko_f32_from_f16_n(const uint16_t *h, size_t n, float *out)
{
    for (size_t i = 0; i < n; ++i) out[i] = dqko_f32_from_f16(h[i]);
}

/* ------------------------------------------------------------- transform */

/* Paired transforms act on row vectors: q' = q A, k' = k B with A B^T = I
 * (arXiv abstract: a query transform and a key transform that are not
 * orthogonal and come as a pair, so that query-key dot products survive).  Reading: fp32, one fused multiply-add chain per
 * output over the input index in ascending order, starting from +0. */
void dqko_transform(const float *x, const float *m, int d, float *y)
{
    for (int j = 0; j < d; ++j) {
        float acc = 0.0f;
        for (int i = 0; i < d; ++i) acc = fmaf(x[i], m[(size_t)i * d + j], acc);
        y[j] = acc;
    }
}

/* ------------------------------------------------------------- quantizer */

/* INT2 with an fp16 scale per group of 32 (tech.dede.sh summary, "Throughput on
 * SGLang": two bits per stored value).  Reading: symmetric four-level grid s*{-3,-1,1,3}, s = fp16 of
 * max|x|/3 (one correctly rounded fp32 division), no zero point; a value goes
 * to the level whose decision interval holds it, thresholds -2s, 0, 2s, a value
 * on a threshold going up. */
void dqko_quantize32(const float *x, ptrdiff_t stride, uint16_t *sigma, uint8_t *codes)
{
    float mx = 0.0f;
    for (int i = 0; i < 32; ++i) {
        float a = fabsf(x[i * stride]);
        if (a > mx) mx = a;
    }
    uint16_t s = dqko_f16_from_f32(mx / 3.0f);
    float sf = dqko_f32_from_f16(s);
    float t = 2.0f * sf;
    for (int i = 0; i < 32; ++i) {
        float v = x[i * stride];
        codes[i] = (uint8_t)((v >= -t) + (v >= 0.0f) + (v >= t));
    }
    *sigma = s;
}

static float level(uint16_t sigma, unsigned u)
{
    return dqko_f32_from_f16(sigma) * (float)(2 * (int)u - 3);
}

/* ------------------------------------------------------------- selection */

/* Keep count for a sparsity in percent, rounded half up in integers. */
int dqko_keep_count(int d, int sparsity_pct)
{
    return (d * (100 - sparsity_pct) + 50) / 100;
}

typedef struct {
    float mag;
    int32_t c;
} ranked;

static int by_magnitude_then_index(const void *pa, const void *pb)
{
    const ranked *a = (const ranked *)pa, *b = (const ranked *)pb;
    if (a->mag > b->mag) return -1;
    if (a->mag < b->mag) return 1;
    return (a->c < b->c) ? -1 : (a->c > b->c);
}

static int ascending_i32(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

/* Channel 0 plus the keep-1 channels c >= 1 of largest score, equal scores by
 * lower index, emitted in ascending order. */
static void keep_top_scores(const float *score, int d, int keep, int32_t *idx)
{
    ranked *r = (ranked *)malloc(sizeof(ranked) * (size_t)(d > 1 ? d - 1 : 1));
    for (int c = 1; c < d; ++c) {
        r[c - 1].mag = score[c];
        r[c - 1].c = c;
    }
    qsort(r, (size_t)(d - 1), sizeof(ranked), by_magnitude_then_index);
    idx[0] = 0;
    for (int i = 1; i < keep; ++i) idx[i] = r[i - 1].c;
    qsort(idx, (size_t)keep, sizeof(int32_t), ascending_i32);
    free(r);
}

/* "Dynamic channel pruning" at a given query-channel sparsity: each query keeps
 * its largest-|q'| channels.  Reading: channel 0 (the protected channel) is
 * always kept and counts toward keep; the rest are ordered by |q'| descending,
 * equal magnitudes by lower index; the kept set is emitted in ascending order. */
void dqko_select(const float *qp, int d, int keep, int32_t *idx)
{
    float *score = (float *)malloc(sizeof(float) * (size_t)d);
    for (int c = 0; c < d; ++c) score[c] = fabsf(qp[c]);
    keep_top_scores(score, d, keep, idx);
    free(score);
}

/* Group-shared selection: one kept set for all query heads of a KV head, so that
 * under grouped-query attention the dropped key channels are dropped for the
 * whole group and really leave the reads (tech.dede.sh summary, "Throughput on
 * SGLang": pruning removes key channels from the cache reads).  The pages state
 * the per-query rule only; the group's rule here is this build's reading: the
 * score of channel c is sum over the group's heads h (ascending) of |q'_{h,c}|,
 * added in fp32 from +0, then the same channel-0 and tie rules. */
void dqko_select_shared(const float *qp, int grp, int d, int keep, int32_t *idx)
{
    float *score = (float *)malloc(sizeof(float) * (size_t)d);
    for (int c = 0; c < d; ++c) {
        float s = 0.0f;
        for (int h = 0; h < grp; ++h) s = s + fabsf(qp[(size_t)h * d + c]);
        score[c] = s;
    }
    keep_top_scores(score, d, keep, idx);
    free(score);
}

void dqko_queries(const float *q, const float *a, int batch, int hq, int hkv, int d,
                  int keep, float *qp, int32_t *idx)
{
    int grp = hq / hkv;
    for (int b = 0; b < batch; ++b)
        for (int h = 0; h < hq; ++h) {
            size_t row = (size_t)b * hq + h;
            dqko_transform(q + row * d, a + (size_t)(h / grp) * d * d, d, qp + row * d);
            dqko_select(qp + row * d, d, keep, idx + row * keep);
        }
}

void dqko_queries_shared(const float *q, const float *a, int batch, int hq, int hkv, int d,
                         int keep, float *qp, int32_t *idx)
{
    int grp = hq / hkv;
    for (int b = 0; b < batch; ++b) {
        for (int h = 0; h < hq; ++h) {
            size_t row = (size_t)b * hq + h;
            dqko_transform(q + row * d, a + (size_t)(h / grp) * d * d, d, qp + row * d);
        }
        for (int g = 0; g < hkv; ++g)
            dqko_select_shared(qp + ((size_t)b * hq + (size_t)g * grp) * d, grp, d, keep,
                               idx + ((size_t)b * hkv + g) * keep);
    }
}

/* ------------------------------------------------------------- layout */

static size_t unit_of(const dqko_cache *c, int b, int g) { return (size_t)b * c->hkv + g; }

static uint8_t *kc_row(const dqko_cache *c, int b, int g, int ch)
{
    return c->k_codes + (unit_of(c, b, g) * c->d + ch) * (size_t)(c->cap / 4);
}
static uint16_t *ks_row(const dqko_cache *c, int b, int g, int ch)
{
    return c->k_scales + (unit_of(c, b, g) * c->d + ch) * (size_t)(c->cap / 32);
}
static uint16_t *ch0_row(const dqko_cache *c, int b, int g)
{
    return c->k_ch0 + unit_of(c, b, g) * (size_t)c->cap;
}
static float *tail_of(const dqko_cache *c, int b, int g)
{
    return c->k_tail + unit_of(c, b, g) * (size_t)32 * c->d;
}
static uint32_t *vword(const dqko_cache *c, int b, int g, int t, int ch)
{
    return c->v_codes + unit_of(c, b, g) * (size_t)(c->cap / 16) * c->d +
           (size_t)(t >> 4) * c->d + ch;
}
static uint16_t *vs_row(const dqko_cache *c, int b, int g, int t)
{
    return c->v_scales + (unit_of(c, b, g) * (size_t)c->cap + t) * (size_t)(c->d / 32);
}

static unsigned key_code(const dqko_cache *c, int b, int g, int t, int ch)
{
    return (kc_row(c, b, g, ch)[t >> 2] >> (2 * (t & 3))) & 3u;
}
static unsigned value_code(const dqko_cache *c, int b, int g, int t, int ch)
{
    return (*vword(c, b, g, t, ch) >> (2 * (t & 15))) & 3u;
}

/* Stored key value at (token t, channel ch) for a sequence of length len:
 * channel 0 from its fp16 row; other channels from their 2-bit group while
 * the 32-token group is complete, else the exact fp32 tail. */
static float key_value(const dqko_cache *c, int b, int g, int len, int t, int ch)
{
    if (ch == 0) return dqko_f32_from_f16(ch0_row(c, b, g)[t]);
    if (t < (len / 32) * 32) return level(ks_row(c, b, g, ch)[t >> 5], key_code(c, b, g, t, ch));
    return tail_of(c, b, g)[(size_t)(t & 31) * c->d + ch];
}

static float value_value(const dqko_cache *c, int b, int g, int t, int ch)
{
    return level(vs_row(c, b, g, t)[ch >> 5], value_code(c, b, g, t, ch));
}

/* ------------------------------------------------------------- append */

/* Each generated token's key and value stay in the cache for every later step
 * (tech.dede.sh summary, "Why the cache becomes a bottleneck").  Per new token at position p: k' = k B; channel 0 of k' to fp16;
 * k' into tail row p mod 32; when p closes a 32-token group, channels 1..d-1 of
 * the 32 tail rows are quantized per channel.  Values are quantized per token in
 * groups of 32 channels at once. */
void dqko_append(const dqko_cache *c, const float *k_new, const float *v_new,
                 const float *bm, const int32_t *n_new, int32_t max_new)
{
    const int d = c->d;
    float *kp = (float *)malloc(sizeof(float) * (size_t)d);
    uint8_t codes[32];
    for (int b = 0; b < c->batch; ++b) {
        int len = c->lengths[b];
        int n = n_new[b];
        if (n > max_new) n = max_new;
        if (n > c->cap - len) n = c->cap - len;
        if (n < 0) n = 0;
        for (int g = 0; g < c->hkv; ++g) {
            const float *bmat = bm + (size_t)g * d * d;
            float *tail = tail_of(c, b, g);
            for (int i = 0; i < n; ++i) {
                int p = len + i;
                const float *kr = k_new + ((unit_of(c, b, g) * (size_t)max_new) + i) * d;
                const float *vr = v_new + ((unit_of(c, b, g) * (size_t)max_new) + i) * d;
                dqko_transform(kr, bmat, d, kp);
                ch0_row(c, b, g)[p] = dqko_f16_from_f32(kp[0]);
                memcpy(tail + (size_t)(p & 31) * d, kp, sizeof(float) * (size_t)d);
                if ((p & 31) == 31) {
                    int t0 = p - 31;
                    for (int ch = 1; ch < d; ++ch) {
                        uint16_t s;
                        dqko_quantize32(tail + ch, d, &s, codes);
                        ks_row(c, b, g, ch)[t0 >> 5] = s;
                        uint8_t *row = kc_row(c, b, g, ch);
                        for (int j = 0; j < 32; ++j) {
                            int t = t0 + j;
                            row[t >> 2] = (uint8_t)((row[t >> 2] & ~(3u << (2 * (t & 3)))) |
                                                    ((unsigned)codes[j] << (2 * (t & 3))));
                        }
                    }
                }
                for (int grp = 0; grp < d / 32; ++grp) {
                    uint16_t s;
                    dqko_quantize32(vr + 32 * grp, 1, &s, codes);
                    vs_row(c, b, g, p)[grp] = s;
                    for (int j = 0; j < 32; ++j) {
                        uint32_t *w = vword(c, b, g, p, 32 * grp + j);
                        int sh = 2 * (p & 15);
                        *w = (*w & ~(3u << sh)) | ((uint32_t)codes[j] << sh);
                    }
                }
            }
        }
        c->lengths[b] = len + n;
    }
    free(kp);
}

/* The cache grows with every generated token (tech.dede.sh summary, "Why the
 * cache becomes a bottleneck"); a sequence that outgrows its capacity moves to a
 * larger cache.  Every stored element keeps its (unit, channel, token) place:
 * element by element, each plane of src is copied to the same indices of dst. */
void dqko_cache_grow(const dqko_cache *src, const dqko_cache *dst)
{
    const int d = src->d;
    for (int b = 0; b < src->batch; ++b) {
        for (int g = 0; g < src->hkv; ++g) {
            for (int ch = 0; ch < d; ++ch) {
                for (int i = 0; i < src->cap / 4; ++i) kc_row(dst, b, g, ch)[i] = kc_row(src, b, g, ch)[i];
                for (int i = 0; i < src->cap / 32; ++i) ks_row(dst, b, g, ch)[i] = ks_row(src, b, g, ch)[i];
            }
            for (int t = 0; t < src->cap; ++t) {
                ch0_row(dst, b, g)[t] = ch0_row(src, b, g)[t];
                for (int j = 0; j < d / 32; ++j) vs_row(dst, b, g, t)[j] = vs_row(src, b, g, t)[j];
            }
            for (int t = 0; t < src->cap; t += 16)
                for (int ch = 0; ch < d; ++ch) *vword(dst, b, g, t, ch) = *vword(src, b, g, t, ch);
            for (int i = 0; i < 32 * d; ++i) tail_of(dst, b, g)[i] = tail_of(src, b, g)[i];
        }
        dst->lengths[b] = src->lengths[b];
    }
}

/* ------------------------------------------------------------- dequant */

void dqko_dequant(const dqko_cache *c, float *k_out, float *v_out)
{
    const int d = c->d;
    for (int b = 0; b < c->batch; ++b)
        for (int g = 0; g < c->hkv; ++g) {
            int len = c->lengths[b];
            float *ko = k_out + unit_of(c, b, g) * (size_t)c->cap * d;
            float *vo = v_out + unit_of(c, b, g) * (size_t)c->cap * d;
            for (int t = 0; t < c->cap; ++t)
                for (int ch = 0; ch < d; ++ch) {
                    ko[(size_t)t * d + ch] = t < len ? key_value(c, b, g, len, t, ch) : 0.0f;
                    vo[(size_t)t * d + ch] = t < len ? value_value(c, b, g, t, ch) : 0.0f;
                }
        }
}

/* ------------------------------------------------------------- attention */

/* Softmax attention with max subtraction, all sums in fp64. */
static void softmax_weighted_sum(const double *z, int t_len, int d,
                                 float (*val)(const void *, int, int), const void *ctx,
                                 float *out)
{
    if (t_len <= 0) {
        for (int ch = 0; ch < d; ++ch) out[ch] = 0.0f;
        return;
    }
    double mx = z[0];
    for (int t = 1; t < t_len; ++t)
        if (z[t] > mx) mx = z[t];
    double den = 0.0;
    double *acc = (double *)calloc((size_t)d, sizeof(double));
    for (int t = 0; t < t_len; ++t) {
        double w = exp(z[t] - mx);
        den += w;
        for (int ch = 0; ch < d; ++ch) acc[ch] += w * (double)val(ctx, t, ch);
    }
    for (int ch = 0; ch < d; ++ch) out[ch] = (float)(acc[ch] / den);
    free(acc);
}

typedef struct {
    const float *v;
    ptrdiff_t ld;
} dense_ctx;

static float dense_value(const void *p, int t, int ch)
{
    const dense_ctx *c = (const dense_ctx *)p;
    return c->v[(size_t)t * c->ld + ch];
}

void dqko_attend_dense(const float *qp, const int32_t *idx, int keep, const float *k,
                       const float *v, int t_len, int d, ptrdiff_t ld, double sm, float *out)
{
    double *z = (double *)malloc(sizeof(double) * (size_t)(t_len > 0 ? t_len : 1));
    for (int t = 0; t < t_len; ++t) {
        double s = 0.0;
        for (int i = 0; i < keep; ++i) s += (double)qp[idx[i]] * (double)k[(size_t)t * ld + idx[i]];
        z[t] = sm * s;
    }
    dense_ctx ctx = {v, ld};
    softmax_weighted_sum(z, t_len, d, dense_value, &ctx, out);
    free(z);
}

typedef struct {
    const dqko_cache *c;
    int b, g;
} cache_ctx;

static float cached_value(const void *p, int t, int ch)
{
    const cache_ctx *x = (const cache_ctx *)p;
    return value_value(x->c, x->b, x->g, t, ch);
}

/* One query head over the stored cache: the logit reads only the kept key
 * channels ("pruning removes ... key channels from reads"); values are never
 * pruned.  Reading: no rescaling for the dropped channels; sm is the caller's
 * softmax scale. */
static void decode_head(const dqko_cache *c, int b, int g, const float *qp, const int32_t *idx,
                        int keep, double sm, float *out)
{
    int len = c->lengths[b];
    double *z = (double *)malloc(sizeof(double) * (size_t)(len > 0 ? len : 1));
    for (int t = 0; t < len; ++t) {
        double s = 0.0;
        for (int i = 0; i < keep; ++i)
            s += (double)qp[idx[i]] * (double)key_value(c, b, g, len, t, idx[i]);
        z[t] = sm * s;
    }
    cache_ctx ctx = {c, b, g};
    softmax_weighted_sum(z, len, c->d, cached_value, &ctx, out);
    free(z);
}

void dqko_decode(const dqko_cache *c, const float *qp, const int32_t *idx, int hq, int keep,
                 double sm, float *out, const uint8_t *heads_mask, int nthreads)
{
    int grp = hq / c->hkv;
    int total = c->batch * hq;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int r = 0; r < total; ++r) {
        if (heads_mask && !heads_mask[r]) continue;
        int b = r / hq, h = r % hq;
        decode_head(c, b, h / grp, qp + (size_t)r * c->d, idx + (size_t)r * keep, keep, sm,
                    out + (size_t)r * c->d);
    }
    (void)nthreads;
}

void dqko_plain_attention(const float *q, const float *k, const float *v,
                          const int32_t *lengths, int batch, int hq, int hkv, int d,
                          int ld_t, double sm, float *out)
{
    int grp = hq / hkv;
    int32_t *all = (int32_t *)malloc(sizeof(int32_t) * (size_t)d);
    for (int ch = 0; ch < d; ++ch) all[ch] = ch;
    for (int b = 0; b < batch; ++b)
        for (int h = 0; h < hq; ++h) {
            size_t unit = (size_t)b * hkv + h / grp;
            const float *kb = k + unit * (size_t)ld_t * d;
            const float *vb = v + unit * (size_t)ld_t * d;
            dqko_attend_dense(q + ((size_t)b * hq + h) * d, all, d, kb, vb, lengths[b], d, d, sm,
                              out + ((size_t)b * hq + h) * d);
        }
    free(all);
}

/* ------------------------------------------------------------- read accounting */

static void mark(uint8_t *touched, size_t off, size_t n)
{
    memset(touched + off, 1, n);
}

static uint64_t count_marked(const uint8_t *touched, size_t n)
{
    uint64_t s = 0;
    for (size_t i = 0; i < n; ++i) s += touched[i];
    return s;
}

/* Walks exactly the element reads of decode_head/key_value/value_value for every
 * head and marks the bytes each one touches, unit by unit. */
void dqko_decode_bytes(const dqko_cache *c, const int32_t *idx, int hq, int keep,
                       uint64_t out[7])
{
    const int d = c->d, cap = c->cap, grp = hq / c->hkv;
    size_t n_kc = (size_t)d * (cap / 4), n_ks = (size_t)d * (cap / 32) * 2, n_c0 = (size_t)cap * 2;
    size_t n_tl = (size_t)32 * d * 4, n_vc = (size_t)(cap / 16) * d * 4, n_vs = (size_t)cap * (d / 32) * 2;
    uint8_t *kc = (uint8_t *)malloc(n_kc), *ks = (uint8_t *)malloc(n_ks), *c0 = (uint8_t *)malloc(n_c0);
    uint8_t *tl = (uint8_t *)malloc(n_tl), *vc = (uint8_t *)malloc(n_vc), *vs = (uint8_t *)malloc(n_vs);
    for (int i = 0; i < 7; ++i) out[i] = 0;
    for (int b = 0; b < c->batch; ++b)
        for (int g = 0; g < c->hkv; ++g) {
            memset(kc, 0, n_kc); memset(ks, 0, n_ks); memset(c0, 0, n_c0);
            memset(tl, 0, n_tl); memset(vc, 0, n_vc); memset(vs, 0, n_vs);
            int len = c->lengths[b];
            for (int h = g * grp; h < (g + 1) * grp; ++h) {
                const int32_t *sel = idx + ((size_t)b * hq + h) * keep;
                for (int t = 0; t < len; ++t) {
                    for (int i = 0; i < keep; ++i) {
                        int ch = sel[i];
                        if (ch == 0) mark(c0, (size_t)t * 2, 2);
                        else if (t < (len / 32) * 32) {
                            mark(kc, (size_t)ch * (cap / 4) + (t >> 2), 1);
                            mark(ks, ((size_t)ch * (cap / 32) + (t >> 5)) * 2, 2);
                        } else mark(tl, ((size_t)(t & 31) * d + ch) * 4, 4);
                    }
                    for (int ch = 0; ch < d; ++ch) {
                        mark(vc, ((size_t)(t >> 4) * d + ch) * 4 + ((t & 15) >> 2), 1);
                        mark(vs, ((size_t)t * (d / 32) + (ch >> 5)) * 2, 2);
                    }
                }
                if (len > 0) out[6] += (uint64_t)keep * 4 /* q' */ + (uint64_t)keep * 4 /* idx */ +
                                       (uint64_t)d * 4 /* out */;
                else out[6] += (uint64_t)d * 4;
            }
            out[0] += count_marked(kc, n_kc);
            out[1] += count_marked(ks, n_ks);
            out[2] += count_marked(c0, n_c0);
            out[3] += count_marked(tl, n_tl);
            out[4] += count_marked(vc, n_vc);
            out[5] += count_marked(vs, n_vs);
        }
    free(kc); free(ks); free(c0); free(tl); free(vc); free(vs);
}
