/* The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer: every
 * entry point runs on small seeded inputs (ragged rows, an empty row, unfinished
 * and closed key groups, every selection size), and a few properties the oracle
 * must have are checked on the way: one bulk append equals token-by-token
 * appends byte for byte, a grown cache decodes like the original, and outputs
 * are finite.  Exit status 0 means every check passed. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/dqk_oracle.h"

static unsigned long long rng_state = 88172645463325252ull;
static float uniform(void) {   /* xorshift64, in [-1, 1) */
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (float)((double)(rng_state >> 11) / 4503599627370496.0 - 1.0);
}

typedef struct {
    dqko_cache c;
    void *mem[7];
} owned;

static owned make(int batch, int hkv, int d, int cap) {
    owned o;
    size_t u = (size_t)batch * hkv;
    o.c.batch = batch; o.c.hkv = hkv; o.c.d = d; o.c.cap = cap;
    o.mem[0] = o.c.k_codes = calloc(u * d * (cap / 4), 1);
    o.mem[1] = o.c.k_scales = calloc(u * d * (cap / 32), 2);
    o.mem[2] = o.c.k_ch0 = calloc(u * cap, 2);
    o.mem[3] = o.c.k_tail = calloc(u * 32 * d, 4);
    o.mem[4] = o.c.v_codes = calloc(u * (cap / 16) * d, 4);
    o.mem[5] = o.c.v_scales = calloc(u * cap * (d / 32), 2);
    o.mem[6] = o.c.lengths = calloc((size_t)batch, 4);
    return o;
}

static void release(owned *o) {
    for (int i = 0; i < 7; ++i) free(o->mem[i]);
}

static int same_planes(const dqko_cache *a, const dqko_cache *b) {
    size_t u = (size_t)a->batch * a->hkv;
    int d = a->d, cap = a->cap;
    return !memcmp(a->k_codes, b->k_codes, u * d * (cap / 4)) &&
           !memcmp(a->k_scales, b->k_scales, u * d * (cap / 32) * 2) &&
           !memcmp(a->k_ch0, b->k_ch0, u * cap * 2) &&
           !memcmp(a->v_codes, b->v_codes, u * (cap / 16) * d * 4) &&
           !memcmp(a->v_scales, b->v_scales, u * cap * (d / 32) * 2) &&
           !memcmp(a->lengths, b->lengths, (size_t)a->batch * 4);
}

int main(void) {
    int fails = 0;
    const int batch = 3, hq = 8, hkv = 2, d = 64, cap = 160, maxn = 150;
    const int n_new[3] = {150, 0, 33};
    float x[32];
    uint16_t sig;
    uint8_t codes[32];
    for (int i = 0; i < 32; ++i) x[i] = uniform() * 10.0f;
    dqko_quantize32(x, 1, &sig, codes);
    for (float v = -70000.0f; v < 70000.0f; v += 977.25f)
        if (isnan(dqko_f32_from_f16(dqko_f16_from_f32(v)))) ++fails;

    size_t nk = (size_t)batch * hkv * maxn * d;
    float *k = malloc(nk * 4), *v = malloc(nk * 4), *bm = malloc((size_t)hkv * d * d * 4);
    float *am = malloc((size_t)hkv * d * d * 4), *q = malloc((size_t)batch * hq * d * 4);
    for (size_t i = 0; i < nk; ++i) { k[i] = uniform() * 4.0f; v[i] = uniform(); }
    for (int g = 0; g < hkv; ++g)
        for (int i = 0; i < d; ++i)
            for (int j = 0; j < d; ++j) {
                float e = (i == j) ? 1.0f : 0.0f;
                am[((size_t)g * d + i) * d + j] = e + 0.1f * uniform();
                bm[((size_t)g * d + i) * d + j] = e + 0.1f * uniform();
            }
    for (int i = 0; i < batch * hq * d; ++i) q[i] = uniform() * 3.0f;

    owned bulk = make(batch, hkv, d, cap), one = make(batch, hkv, d, cap);
    dqko_append(&bulk.c, k, v, bm, n_new, maxn);
    /* token by token: slice i of each row as a one-token append */
    float *k1 = malloc((size_t)batch * hkv * d * 4), *v1 = malloc((size_t)batch * hkv * d * 4);
    for (int i = 0; i < maxn; ++i) {
        int cnt[3];
        for (int b = 0; b < batch; ++b) {
            cnt[b] = i < n_new[b] ? 1 : 0;
            for (int g = 0; g < hkv; ++g)
                for (int c = 0; c < d; ++c) {
                    size_t src = ((((size_t)b * hkv + g) * maxn) + i) * d + c;
                    k1[((size_t)b * hkv + g) * d + c] = k[src];
                    v1[((size_t)b * hkv + g) * d + c] = v[src];
                }
        }
        dqko_append(&one.c, k1, v1, bm, cnt, 1);
    }
    if (!same_planes(&bulk.c, &one.c)) { fprintf(stderr, "bulk != token by token\n"); ++fails; }

    float *kd = malloc((size_t)batch * hkv * cap * d * 4), *vd = malloc((size_t)batch * hkv * cap * d * 4);
    dqko_dequant(&bulk.c, kd, vd);
    float *qp = malloc((size_t)batch * hq * d * 4), *out = malloc((size_t)batch * hq * d * 4);
    float *out2 = malloc((size_t)batch * hq * d * 4);
    int32_t *idx = malloc((size_t)batch * hq * d * 4), *idxs = malloc((size_t)batch * hkv * d * 4);
    uint64_t nbytes[7];
    for (int keep = 1; keep <= d; keep += 21) {
        dqko_queries(q, am, batch, hq, hkv, d, keep, qp, idx);
        dqko_queries_shared(q, am, batch, hq, hkv, d, keep, qp, idxs);
        dqko_decode(&bulk.c, qp, idx, hq, keep, 0.125, out, NULL, 2);
        dqko_decode_bytes(&bulk.c, idx, hq, keep, nbytes);
        for (int i = 0; i < batch * hq * d; ++i)
            if (!isfinite(out[i])) { ++fails; break; }
    }
    dqko_attend_dense(qp, idx, 1, kd, vd, 150, d, d, 0.125, out2);
    dqko_plain_attention(q, kd, vd, bulk.c.lengths, batch, hq, hkv, d, cap, 0.125, out2);

    owned grown = make(batch, hkv, d, cap + 96);
    dqko_cache_grow(&bulk.c, &grown.c);
    dqko_queries(q, am, batch, hq, hkv, d, 38, qp, idx);
    dqko_decode(&bulk.c, qp, idx, hq, 38, 0.125, out, NULL, 1);
    dqko_decode(&grown.c, qp, idx, hq, 38, 0.125, out2, NULL, 1);
    if (memcmp(out, out2, (size_t)batch * hq * d * 4)) { fprintf(stderr, "grown decode differs\n"); ++fails; }

    release(&bulk); release(&one); release(&grown);
    free(k); free(v); free(bm); free(am); free(q); free(k1); free(v1); free(kd); free(vd);
    free(qp); free(out); free(out2); free(idx); free(idxs);
    printf("oracle driver: %d failures\n", fails);
    return fails == 0 ? 0 : 1;
}
