/*
 * QSA sparse main-attention prefill -- plain FP32 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the slow, obviously correct statement of
 * what the GPU path must compute.  Only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg may load it.  The product library never
 * calls it, and the two share no code, headers, tables or helpers.
 *
 * Source of the definition: the page "Qwen4-Exp QSA comes to Huawei's Ascend:
 * inside SGLang's opt-in CANN prefill PR" (orcarouter.ai blog).
 *
 *  - Section "What the pull request actually adds", layout-embedding
 *    paragraph: main attention is ordinary softmax(scale * Q K^T) V; the
 *    Ascend packing [K,V] / [Q,0] only re-expresses it, so the plain
 *    definition below is the exact target.  The D=256 scale is kept.
 *  - Same section, "Sizing bounds" bullet: -1 marks an unused selection entry
 *    (tail or interior), and a row with nothing selected outputs zero.
 *  - Section "Nine tests that passed, ...": the reference is FP32 on the CPU,
 *    computed from the same BF16 inputs; slots are unordered physical cache
 *    slots; widths include zero.
 *
 * Readings where the page is silent (each is listed in the design notes):
 *  - query head h uses KV head floor(h / G), G = Hq / Hkv (contiguous groups);
 *  - -1 anywhere in a row is "no slot"; any other value outside [0, S) is an
 *    error (the oracle refuses the whole call);
 *  - duplicates are kept: every selection entry is one softmax term;
 *  - scores accumulate in FP32 in d order, exp is libm expf, and the output
 *    stays FP32 (the GPU's BF16 output is compared against it).
 *
 * FP8 KV-cache variant (qsa_oracle_prefill_fp8kv): K and V bytes are FP8
 * E4M3 codes, decoded from the format's definition and multiplied by one
 * scale per tensor; everything after that is the same FP32 computation.
 *
 * Parity pins (tests, not here): FP64 brute-force dense masked attention,
 * torch's scaled_dot_product_attention for full and causal selections, and
 * closed forms (single slot, uniform weights, identical V rows, empty rows).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum {
    ORACLE_OK = 0,
    ORACLE_BAD_SLOT = 1,  /* an entry is neither -1 nor in [0, S) */
    ORACLE_BAD_SHAPE = 2, /* Hq % Hkv != 0, negative sizes, ... */
    ORACLE_NO_MEMORY = 3,
};

/* BF16 is the upper half of an IEEE binary32; widening is exact. */
static float bf16_to_float(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/*
 * FP8 E4M3 ("fn" variant of the OCP 8-bit floating point formats): 1 sign
 * bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 encodes
 * subnormals m/8 * 2^-6; no infinities; exponent 15 with mantissa 7 is NaN.
 * Used for the FP8 KV-cache variant (the page's section "Where this sits in
 * the Qwen4Exp serving build-out" mentions an fp8_e4m3 KV cache).
 */
float qsa_oracle_e4m3_to_float(uint8_t b)
{
    const int sign = b >> 7, e = (b >> 3) & 15, m = b & 7;
    float v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexpf((float)m / 8.0f, -6);
    else
        v = ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return sign ? -v : v;
}

/* One K or V element as a real number: BF16 as is, FP8 decoded and scaled by
 * the tensor's scale (reading: real = decode(byte) * scale, one scale per
 * tensor). */
static float kv_elem(const void *row, int32_t d, int fp8, float kv_scale)
{
    if (fp8)
        return qsa_oracle_e4m3_to_float(((const uint8_t *)row)[d]) * kv_scale;
    return bf16_to_float(((const uint16_t *)row)[d]);
}

/*
 * Selection-list filter (the "-1 padding" rule of the "Sizing bounds" bullet):
 * for each token row t keep, in their original order, the entries that name a
 * slot in [0, S).  list[t*W + i] for i < count[t] receives the kept entries;
 * n_bad[t] counts entries that are neither -1 nor a valid slot.
 */
int qsa_oracle_compact(const int32_t *slot_idx, int64_t stride_t, int64_t T,
                       int64_t W, int64_t S, int32_t *list, int64_t *count,
                       int64_t *n_bad)
{
    if (T < 0 || W < 0 || S < 0)
        return ORACLE_BAD_SHAPE;
    for (int64_t t = 0; t < T; ++t) {
        const int32_t *row = slot_idx + t * stride_t;
        int64_t n = 0, bad = 0;
        for (int64_t j = 0; j < W; ++j) {
            int32_t s = row[j];
            if (s >= 0 && (int64_t)s < S)
                list[t * W + n++] = s;
            else if (s != -1)
                ++bad;
        }
        count[t] = n;
        n_bad[t] = bad;
    }
    return ORACLE_OK;
}

/*
 * One (token, query head) output row, straight from the definition:
 *   z_j = scale * sum_d q[d] k_j[d]          (FP32, d order)
 *   m   = max_j z_j
 *   p_j = expf(z_j - m),  l = sum_j p_j      (j order)
 *   o[d] = (sum_j p_j v_j[d]) / l
 * An empty selection gives +0.0 everywhere.
 */
static int one_row(const uint16_t *q_row, const void *k, int64_t k_ss,
                   const void *v, int64_t v_ss, int fp8, float k_scale,
                   float v_scale, const int32_t *sel, int64_t W, int64_t S,
                   int32_t D, float scale, float *z, int32_t *slots, float *o)
{
    const size_t esz = fp8 ? 1 : 2;   /* bytes per K/V element */
    int64_t n = 0;
    for (int64_t j = 0; j < W; ++j) {
        int32_t s = sel[j];
        if (s == -1)
            continue;
        if (s < 0 || (int64_t)s >= S)
            return ORACLE_BAD_SLOT;
        const char *k_row = (const char *)k + (size_t)((int64_t)s * k_ss) * esz;
        float dot = 0.0f;
        for (int32_t d = 0; d < D; ++d)
            dot += bf16_to_float(q_row[d]) * kv_elem(k_row, d, fp8, k_scale);
        z[n] = scale * dot;
        slots[n] = s;
        ++n;
    }
    for (int32_t d = 0; d < D; ++d)
        o[d] = 0.0f;
    if (n == 0)
        return ORACLE_OK;

    float m = z[0];
    for (int64_t i = 1; i < n; ++i)
        if (z[i] > m)
            m = z[i];
    float l = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        z[i] = expf(z[i] - m);
        l += z[i];
    }
    for (int64_t i = 0; i < n; ++i) {
        const char *v_row = (const char *)v + (size_t)((int64_t)slots[i] * v_ss) * esz;
        for (int32_t d = 0; d < D; ++d)
            o[d] += z[i] * kv_elem(v_row, d, fp8, v_scale);
    }
    for (int32_t d = 0; d < D; ++d)
        o[d] = o[d] / l;
    return ORACLE_OK;
}

/*
 * Sparse prefill for a chosen set of token rows.
 *
 * q        [T, Hq, D]  bf16 bits, element strides (q_st, q_sh, 1)
 * k, v     [S, Hkv, D] bf16 bits, element strides (x_ss, x_sh, 1)
 * slot_idx [T, W]      int32, element strides (s_st, 1)
 * rows     token indices to evaluate (nrows of them); NULL means 0..nrows-1
 * out      [nrows, Hq, D] FP32, contiguous
 * nthreads OpenMP threads (<= 0: the runtime default)
 *
 * Returns ORACLE_OK, or ORACLE_BAD_SLOT if any evaluated row holds an entry
 * outside [0, S) other than -1 (then out is unspecified).
 */
static int prefill_any(const uint16_t *q, int64_t q_st, int64_t q_sh,
                       const void *k, int64_t k_ss, int64_t k_sh,
                       const void *v, int64_t v_ss, int64_t v_sh, int fp8,
                       float k_scale, float v_scale,
                       const int32_t *slot_idx, int64_t s_st, int64_t S,
                       int64_t W, int32_t Hq, int32_t Hkv, int32_t D,
                       float scale, const int64_t *rows, int64_t nrows,
                       float *out, int32_t nthreads)
{
    const size_t esz = fp8 ? 1 : 2;
    if (Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0 || W < 0 || S < 0 ||
        nrows < 0)
        return ORACLE_BAD_SHAPE;
    const int32_t G = Hq / Hkv;
    int status = ORACLE_OK;

#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

#pragma omp parallel
    {
        float *z = (float *)malloc(sizeof(float) * (size_t)(W > 0 ? W : 1));
        int32_t *slots =
            (int32_t *)malloc(sizeof(int32_t) * (size_t)(W > 0 ? W : 1));
        if (!z || !slots) {
#pragma omp atomic write
            status = ORACLE_NO_MEMORY;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t work = 0; work < nrows * (int64_t)Hq; ++work) {
                int64_t r = work / Hq;
                int32_t h = (int32_t)(work % Hq);
                int64_t t = rows ? rows[r] : r;
                int32_t g = h / G;
                int rc = one_row(q + t * q_st + (int64_t)h * q_sh,
                                 (const char *)k + (size_t)((int64_t)g * k_sh) * esz, k_ss,
                                 (const char *)v + (size_t)((int64_t)g * v_sh) * esz, v_ss,
                                 fp8, k_scale, v_scale, slot_idx + t * s_st, W, S, D,
                                 scale, z, slots, out + (r * Hq + h) * (int64_t)D);
                if (rc != ORACLE_OK) {
#pragma omp atomic write
                    status = rc;
                }
            }
        }
        free(z);
        free(slots);
    }
    return status;
}

int qsa_oracle_prefill(const uint16_t *q, int64_t q_st, int64_t q_sh,
                       const uint16_t *k, int64_t k_ss, int64_t k_sh,
                       const uint16_t *v, int64_t v_ss, int64_t v_sh,
                       const int32_t *slot_idx, int64_t s_st, int64_t S,
                       int64_t W, int32_t Hq, int32_t Hkv, int32_t D,
                       float scale, const int64_t *rows, int64_t nrows,
                       float *out, int32_t nthreads)
{
    return prefill_any(q, q_st, q_sh, k, k_ss, k_sh, v, v_ss, v_sh, 0, 1.0f,
                       1.0f, slot_idx, s_st, S, W, Hq, Hkv, D, scale, rows,
                       nrows, out, nthreads);
}

/*
 * The same sparse prefill with an FP8 E4M3 KV cache: k8, v8 hold one byte
 * per element (strides in elements = bytes) and every element means
 * decode(byte) * k_scale (resp. v_scale).
 */
int qsa_oracle_prefill_fp8kv(const uint16_t *q, int64_t q_st, int64_t q_sh,
                             const uint8_t *k8, int64_t k_ss, int64_t k_sh,
                             const uint8_t *v8, int64_t v_ss, int64_t v_sh,
                             float k_scale, float v_scale,
                             const int32_t *slot_idx, int64_t s_st, int64_t S,
                             int64_t W, int32_t Hq, int32_t Hkv, int32_t D,
                             float scale, const int64_t *rows, int64_t nrows,
                             float *out, int32_t nthreads)
{
    return prefill_any(q, q_st, q_sh, k8, k_ss, k_sh, v8, v_ss, v_sh, 1,
                       k_scale, v_scale, slot_idx, s_st, S, W, Hq, Hkv, D,
                       scale, rows, nrows, out, nthreads);
}

/* Threads the oracle will use when nthreads <= 0. */
int qsa_oracle_default_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * QSA indexer and Top-K selection (the step before main attention; page
 * section "Why QSA is the awkward part, in numbers": a multi-query indexer
 * with 4 query heads sharing 1 key head, head dim 128, compression ratio 4,
 * a fixed budget; section "Nine tests that passed, ...": causal tails of 0-3
 * tokens).  Readings (the page gives the structure, not the formulas):
 *  - one index key per compressed block of 4 consecutive positions;
 *  - score(t, c) = sum_h max(0, iq[t,h] . ik[c]), FP32, d order then h order;
 *  - a query at position p ranks the complete blocks before it
 *    (4c + 3 <= p) and keeps the `budget` best, ties to the lower c;
 *  - its selection is the positions of the kept blocks (ascending c, each
 *    block's 4 positions in order) followed by its r = (p+1) % 4 tail
 *    positions p-r+1..p, mapped to physical slots by slot_of_pos, then -1 up
 *    to the row width 4*budget + 3.
 */
int qsa_oracle_indexer_scores(const uint16_t *iq, int64_t q_st, int64_t q_sh,
                              const uint16_t *ik, int64_t k_st, int64_t T,
                              int64_t C, int32_t H, int32_t D, float *scores,
                              int32_t nthreads)
{
    if (T < 0 || C < 0 || H <= 0 || D <= 0)
        return ORACLE_BAD_SHAPE;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t c = 0; c < C; ++c) {
            float total = 0.0f;
            for (int32_t h = 0; h < H; ++h) {
                const uint16_t *qr = iq + t * q_st + (int64_t)h * q_sh;
                const uint16_t *kr = ik + c * k_st;
                float dot = 0.0f;
                for (int32_t d = 0; d < D; ++d)
                    dot += bf16_to_float(qr[d]) * bf16_to_float(kr[d]);
                total += dot > 0.0f ? dot : 0.0f;
            }
            scores[t * C + c] = total;
        }
    }
    return ORACLE_OK;
}

typedef struct {
    float score;
    int32_t block;
} ranked;

/* Better first: higher score, then lower block index. */
static int rank_order(const void *a, const void *b)
{
    const ranked *x = (const ranked *)a, *y = (const ranked *)b;
    if (x->score != y->score)
        return x->score > y->score ? -1 : 1;
    return (x->block > y->block) - (x->block < y->block);
}

static int int_order(const void *a, const void *b)
{
    const int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

int qsa_oracle_indexer_select(const float *scores, int64_t T, int64_t C,
                              const int32_t *positions,
                              const int32_t *slot_of_pos, int64_t L,
                              int32_t budget, int32_t *slot_idx)
{
    if (T < 0 || C < 0 || budget < 0)
        return ORACLE_BAD_SHAPE;
    const int64_t width = 4 * (int64_t)budget + 3;
    ranked *cand = (ranked *)malloc(sizeof(ranked) * (size_t)(C > 0 ? C : 1));
    int32_t *kept = (int32_t *)malloc(sizeof(int32_t) * (size_t)(C > 0 ? C : 1));
    if (!cand || !kept) {
        free(cand);
        free(kept);
        return ORACLE_NO_MEMORY;
    }
    int status = ORACLE_OK;
    for (int64_t t = 0; t < T && status == ORACLE_OK; ++t) {
        const int64_t p = positions[t];
        const int64_t eligible = (p + 1) / 4 < C ? (p + 1) / 4 : C;
        if (p < 0 || p >= L) {
            status = ORACLE_BAD_SHAPE;
            break;
        }
        for (int64_t c = 0; c < eligible; ++c) {
            cand[c].score = scores[t * C + c];
            cand[c].block = (int32_t)c;
        }
        qsort(cand, (size_t)eligible, sizeof(ranked), rank_order);
        const int64_t n = eligible < budget ? eligible : budget;
        for (int64_t i = 0; i < n; ++i)
            kept[i] = cand[i].block;
        qsort(kept, (size_t)n, sizeof(int32_t), int_order);
        int32_t *row = slot_idx + t * width;
        int64_t w = 0;
        for (int64_t i = 0; i < n; ++i)
            for (int j = 0; j < 4; ++j)
                row[w++] = slot_of_pos[4 * (int64_t)kept[i] + j];
        const int64_t r = (p + 1) % 4;
        for (int64_t pos = p - r + 1; pos <= p; ++pos)
            row[w++] = slot_of_pos[pos];
        while (w < width)
            row[w++] = -1;
    }
    free(cand);
    free(kept);
    return status;
}
