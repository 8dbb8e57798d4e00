/*
 * Drives every function of the CPU oracle (oracle/fa_oracle.c) over small
 * inputs, valid and invalid, so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer sees every code path: pooling, the router, the
 * block plan, the token predicate, prefill (fp32 and bf16, all rows and a row
 * list, one and several threads) and decode (all heads and a head list).  It
 * also checks one closed form (V = 1 gives O = 1) so that a silently skipped
 * path shows.  Exit status 0 means every call behaved.  Test infrastructure.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_pool(const void *x, int dtype, const int32_t *cu_seqlens, int batch, int hidden,
             int pool_tokens, float *p32, double *p64);
int orc_router(const void *x, int dtype, const int32_t *cu_seqlens, int batch, int hidden,
               int pool_tokens, const float *w1, const float *b1, int router_hidden,
               const float *w2, const float *b2, int n_layers, uint8_t *route, float *logits32,
               double *logits64);
int orc_block_plan(const int32_t *seqlens, int batch, int max_qblocks, const uint8_t *route,
                   int n_layers, int layer, int sink, int window, int block, int32_t *plan);
int orc_visible_predicate(int t, int s, int is_fa, int sink, int window, int block);
int64_t orc_visible_pairs(int T, int is_fa, int sink, int window, int block);
int orc_attn_prefill(const void *q, const void *k, const void *v, int dtype,
                     const int32_t *cu_seqlens, int batch, int hq, int hkv, int d,
                     const uint8_t *route, int n_layers, int layer, int sink, int window,
                     int block, double sm_scale, const int32_t *rows, int n_rows, double *o,
                     double *lse, int n_threads);
int orc_attn_decode(const void *q, const void *k_cache, const void *v_cache, int max_cache,
                    const int32_t *cache_len, int dtype, int batch, int hq, int hkv, int d,
                    const uint8_t *route, int n_layers, int layer, int sink, int window,
                    int block, double sm_scale, const int32_t *heads, int n_heads, double *o,
                    double *lse, int n_threads);

static int failures = 0;
#define CHECK(cond)                                                        \
    do {                                                                   \
        if (!(cond)) {                                                     \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            failures++;                                                    \
        }                                                                  \
    } while (0)

static uint32_t rng_state = 12345u;
static float frand(void)
{
    rng_state = rng_state * 1664525u + 1013904223u;
    return (float)((rng_state >> 8) & 0xffff) / 32768.0f - 1.0f;
}

static uint16_t to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

int main(void)
{
    /* two sequences of 70 and 33 tokens */
    const int32_t cu[3] = {0, 70, 103};
    const int total = 103, B = 2, hq = 4, hkv = 2, d = 16, hidden = 24, rh = 8, L = 3;
    const int sink = 16, window = 32, block = 16;

    float *x = malloc(sizeof(float) * total * hidden);
    for (int i = 0; i < total * hidden; ++i) x[i] = frand();
    float p32[2 * 24];
    double p64[2 * 24];
    CHECK(orc_pool(x, 0, cu, B, hidden, 64, p32, p64) == 0);
    CHECK(orc_pool(NULL, 0, cu, B, hidden, 64, p32, p64) != 0);

    float w1[8 * 24], b1[8], w2[3 * 8], b2[3];
    for (int i = 0; i < rh * hidden; ++i) w1[i] = frand();
    for (int i = 0; i < rh; ++i) b1[i] = 0.1f * frand();
    for (int i = 0; i < L * rh; ++i) w2[i] = frand();
    for (int i = 0; i < L; ++i) b2[i] = 0.1f * frand();
    uint8_t route[2 * 3];
    float l32[6];
    double l64[6];
    CHECK(orc_router(x, 0, cu, B, hidden, 64, w1, b1, rh, w2, b2, L, route, l32, l64) == 0);
    CHECK(orc_router(x, 0, cu, B, hidden, 64, w1, b1, 0, w2, b2, L, route, l32, l64) != 0);
    route[0] = 1; route[1] = 0; route[2] = 1;  /* fixed mask for the attention calls */
    route[3] = 0; route[4] = 1; route[5] = 1;

    int32_t seqlens[2] = {70, 33};
    int32_t plan[2 * 6 * 4];
    CHECK(orc_block_plan(seqlens, B, 6, route, L, 1, sink, window, block, plan) == 0);
    CHECK(orc_block_plan(seqlens, B, 6, route, L, 3, sink, window, block, plan) != 0);
    CHECK(orc_visible_predicate(5, 3, 0, sink, window, block) == 1);
    CHECK(orc_visible_pairs(70, 1, sink, window, block) == 70 * 71 / 2);

    float *q = malloc(sizeof(float) * total * hq * d);
    float *k = malloc(sizeof(float) * total * hkv * d);
    float *v = malloc(sizeof(float) * total * hkv * d);
    uint16_t *qb = malloc(2 * total * hq * d), *kb = malloc(2 * total * hkv * d),
             *vb = malloc(2 * total * hkv * d);
    for (int i = 0; i < total * hq * d; ++i) { q[i] = frand(); qb[i] = to_bf16(q[i]); }
    for (int i = 0; i < total * hkv * d; ++i) {
        k[i] = frand();
        v[i] = 1.0f;
        kb[i] = to_bf16(k[i]);
        vb[i] = to_bf16(v[i]);
    }
    double *o = malloc(sizeof(double) * total * hq * d), *lse = malloc(sizeof(double) * total * hq);
    for (int layer = 0; layer < L; ++layer)
        for (int nt = 1; nt <= 4; nt += 3) {
            CHECK(orc_attn_prefill(q, k, v, 0, cu, B, hq, hkv, d, route, L, layer, sink, window,
                                   block, 0.25, NULL, 0, o, lse, nt) == 0);
            for (int i = 0; i < total * hq * d; ++i) CHECK(fabs(o[i] - 1.0) < 1e-12);
            CHECK(orc_attn_prefill(qb, kb, vb, 1, cu, B, hq, hkv, d, route, L, layer, sink,
                                   window, block, 0.25, NULL, 0, o, NULL, nt) == 0);
        }
    const int32_t rows[4] = {0, 69, 70, 102};
    CHECK(orc_attn_prefill(q, k, v, 0, cu, B, hq, hkv, d, route, L, 1, sink, window, block, 0.25,
                           rows, 4, o, lse, 2) == 0);
    const int32_t bad_rows[1] = {103};
    CHECK(orc_attn_prefill(q, k, v, 0, cu, B, hq, hkv, d, route, L, 1, sink, window, block, 0.25,
                           bad_rows, 1, o, lse, 2) != 0);
    CHECK(orc_attn_prefill(q, k, v, 0, cu, B, 3, hkv, d, route, L, 1, sink, window, block, 0.25,
                           NULL, 0, o, lse, 1) != 0);

    /* decode over [B][hkv][max_cache][d] caches */
    const int max_cache = 80;
    float *kc = malloc(sizeof(float) * B * hkv * max_cache * d);
    float *vc = malloc(sizeof(float) * B * hkv * max_cache * d);
    for (int i = 0; i < B * hkv * max_cache * d; ++i) { kc[i] = frand(); vc[i] = 1.0f; }
    const int32_t cl[2] = {80, 17};
    double od[2 * 4 * 16], ld[2 * 4];
    for (int layer = 0; layer < L; ++layer) {
        CHECK(orc_attn_decode(q, kc, vc, max_cache, cl, 0, B, hq, hkv, d, route, L, layer, sink,
                              window, block, 0.25, NULL, 0, od, ld, 3) == 0);
        for (int i = 0; i < B * hq * d; ++i) CHECK(fabs(od[i] - 1.0) < 1e-12);
    }
    const int32_t heads[2] = {0, 3};
    CHECK(orc_attn_decode(q, kc, vc, max_cache, cl, 0, B, hq, hkv, d, route, L, 0, sink, window,
                          block, 0.25, heads, 2, od, ld, 2) == 0);
    const int32_t bad_cl[2] = {81, 1};
    CHECK(orc_attn_decode(q, kc, vc, max_cache, bad_cl, 0, B, hq, hkv, d, route, L, 0, sink,
                          window, block, 0.25, NULL, 0, od, ld, 1) != 0);

    free(x); free(q); free(k); free(v); free(qb); free(kb); free(vb); free(o); free(lse);
    free(kc); free(vc);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle driver ok\n");
    return 0;
}
