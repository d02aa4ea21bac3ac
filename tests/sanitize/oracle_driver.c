/*
 * Runs the CPU oracle (oracle/qsa_oracle.c, linked in) on small inputs under
 * AddressSanitizer and UBSan: compaction, the BF16 and FP8 prefills, the
 * E4M3 decoding of every code and the indexer's scores and selection, with
 * closed-form checks (a single selected slot returns that V row, an empty row
 * returns +0.0, the compaction's counts).  Exit status 0 when every check
 * holds and the sanitizers report nothing.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int qsa_oracle_compact(const int32_t *, int64_t, int64_t, int64_t, int64_t, int32_t *, int64_t *,
                       int64_t *);
int qsa_oracle_prefill(const uint16_t *, int64_t, int64_t, const uint16_t *, int64_t, int64_t,
                       const uint16_t *, int64_t, int64_t, const int32_t *, int64_t, int64_t,
                       int64_t, int32_t, int32_t, int32_t, float, const int64_t *, int64_t, float *,
                       int32_t);
int qsa_oracle_prefill_fp8kv(const uint16_t *, int64_t, int64_t, const uint8_t *, int64_t, int64_t,
                             const uint8_t *, int64_t, int64_t, float, float, const int32_t *,
                             int64_t, int64_t, int64_t, int32_t, int32_t, int32_t, float,
                             const int64_t *, int64_t, float *, int32_t);
float qsa_oracle_e4m3_to_float(uint8_t);
int qsa_oracle_indexer_scores(const uint16_t *, int64_t, int64_t, const uint16_t *, int64_t, int64_t,
                              int64_t, int32_t, int32_t, float *, int32_t);
int qsa_oracle_indexer_select(const float *, int64_t, int64_t, const int32_t *, const int32_t *,
                              int64_t, int32_t, int32_t *);

static int failures = 0;
#define CHECK(c)                                                              \
    do {                                                                      \
        if (!(c)) {                                                           \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
            ++failures;                                                       \
        }                                                                     \
    } while (0)

static uint32_t rng = 12345u;
static uint32_t next(void) { rng = rng * 1664525u + 1013904223u; return rng >> 8; }

/* A BF16 value in (-2, 2): the top half of a float. */
static uint16_t rand_bf16(void) {
    float f = ((float)(next() % 4000) - 2000.0f) / 1000.0f;
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static float bf(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

int main(void) {
    enum { T = 5, S = 9, Hq = 4, Hkv = 2, D = 256, W = 6 };
    uint16_t *q = malloc(sizeof(uint16_t) * T * Hq * D);
    uint16_t *k = malloc(sizeof(uint16_t) * S * Hkv * D);
    uint16_t *v = malloc(sizeof(uint16_t) * S * Hkv * D);
    uint8_t *k8 = malloc(S * Hkv * D), *v8 = malloc(S * Hkv * D);
    for (int i = 0; i < T * Hq * D; ++i) q[i] = rand_bf16();
    for (int i = 0; i < S * Hkv * D; ++i) {
        k[i] = rand_bf16();
        v[i] = rand_bf16();
        k8[i] = (uint8_t)(next() & 0x77);   /* finite E4M3 codes */
        v8[i] = (uint8_t)(next() & 0x77);
    }
    const int32_t sel[T][W] = {{3, -1, -1, -1, -1, -1},   /* one slot */
                               {-1, -1, -1, -1, -1, -1},  /* empty */
                               {0, 8, -1, 4, 2, 2},       /* duplicates, interior -1 */
                               {7, 6, 5, 4, 3, 1},
                               {1, -1, 0, -1, 8, -1}};
    int32_t list[T * W];
    int64_t count[T], n_bad[T];
    CHECK(qsa_oracle_compact(&sel[0][0], W, T, W, S, list, count, n_bad) == 0);
    CHECK(count[0] == 1 && count[1] == 0 && count[2] == 5 && count[3] == 6 && count[4] == 3);
    for (int t = 0; t < T; ++t) CHECK(n_bad[t] == 0);
    const int32_t bad_row[W] = {1, -2, 9, 100, -1, 3};
    CHECK(qsa_oracle_compact(bad_row, W, 1, W, S, list, count, n_bad) == 0 && count[0] == 2 &&
          n_bad[0] == 3);

    float *out = malloc(sizeof(float) * T * Hq * D);
    int64_t rows[T];
    for (int t = 0; t < T; ++t) rows[t] = t;
    CHECK(qsa_oracle_prefill(q, Hq * D, D, k, Hkv * D, D, v, Hkv * D, D, &sel[0][0], W, S, W, Hq,
                             Hkv, D, 0.0625f, rows, T, out, 1) == 0);
    for (int h = 0; h < Hq; ++h)
        for (int d = 0; d < D; ++d) {
            CHECK(out[(0 * Hq + h) * D + d] == bf(v[(3 * Hkv + h / 2) * D + d]));
            CHECK(out[(1 * Hq + h) * D + d] == 0.0f && !signbit(out[(1 * Hq + h) * D + d]));
        }
    for (int i = 0; i < T * Hq * D; ++i) CHECK(isfinite(out[i]));
    /* an entry outside [0, S) is refused */
    int32_t sel_bad[T][W];
    memcpy(sel_bad, sel, sizeof sel);
    sel_bad[3][2] = S;
    CHECK(qsa_oracle_prefill(q, Hq * D, D, k, Hkv * D, D, v, Hkv * D, D, &sel_bad[0][0], W, S, W,
                             Hq, Hkv, D, 0.0625f, rows, T, out, 1) == 1);
    CHECK(qsa_oracle_prefill_fp8kv(q, Hq * D, D, k8, Hkv * D, D, v8, Hkv * D, D, 0.5f, 2.0f,
                                   &sel[0][0], W, S, W, Hq, Hkv, D, 0.0625f, rows, T, out, 1) == 0);
    for (int d = 0; d < D; ++d)
        CHECK(out[d] == qsa_oracle_e4m3_to_float(v8[(3 * Hkv + 0) * D + d]) * 2.0f);
    for (int c = 0; c < 256; ++c) {
        const float f = qsa_oracle_e4m3_to_float((uint8_t)c);
        CHECK(((c & 0x7f) == 0x7f) ? isnan(f) : (isfinite(f) && fabsf(f) <= 448.0f));
    }

    /* indexer: 3 queries, 4 heads, dim 128, 10 keys, positions near the ends */
    enum { TI = 3, HI = 4, DI = 128, C = 10, L = 40, BUDGET = 3 };
    uint16_t *iq = malloc(sizeof(uint16_t) * TI * HI * DI), *ik = malloc(sizeof(uint16_t) * C * DI);
    for (int i = 0; i < TI * HI * DI; ++i) iq[i] = rand_bf16();
    for (int i = 0; i < C * DI; ++i) ik[i] = rand_bf16();
    float scores[TI * C];
    CHECK(qsa_oracle_indexer_scores(iq, HI * DI, DI, ik, DI, TI, C, HI, DI, scores, 1) == 0);
    for (int i = 0; i < TI * C; ++i) CHECK(scores[i] >= 0.0f);
    const int32_t pos[TI] = {2, 17, 39};
    int32_t slot_of_pos[L];
    for (int i = 0; i < L; ++i) slot_of_pos[i] = 1000 + i;
    int32_t picked[TI * (4 * BUDGET + 3)];
    CHECK(qsa_oracle_indexer_select(scores, TI, C, pos, slot_of_pos, L, BUDGET, picked) == 0);
    CHECK(picked[0] == 1000 && picked[1] == 1001 && picked[2] == 1002 && picked[3] == -1);
    CHECK(picked[2 * (4 * BUDGET + 3) + 4 * BUDGET] == -1);   /* p = 39: (p+1) % 4 = 0, no tail */
    free(q); free(k); free(v); free(k8); free(v8); free(out); free(iq); free(ik);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("all oracle checks passed\n");
    return 0;
}
