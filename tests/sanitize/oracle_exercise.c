/* Host program that runs the CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.
 * Small problems of every shape class (decode, prefill, GQA, bf16, W >= n, k = 0, k > |R_i|,
 * n = 1), row subsets, the restricted and full forms, and argument errors. Exit status 0 when
 * every call returned what it should and the outputs are finite. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t batch, heads, kv_heads, n, nq, d, W, topk;
    int32_t dtype;
    int32_t threads;
} oracle_problem;

int oracle_condensate(const oracle_problem *p, const void *q, const void *k, const void *v,
                      int32_t *out_idx, double *out, double *diag);
int oracle_condensate_rows(const oracle_problem *p, const void *q, const void *k, const void *v,
                           const int64_t *rows, int64_t nrows, int32_t *out_idx, double *out,
                           double *diag);
int oracle_restricted(const oracle_problem *p, const void *q, const void *k, const void *v,
                      const int32_t *idx, int64_t idx_stride, double *out);
int oracle_full(const oracle_problem *p, const void *q, const void *k, const void *v, double *out);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static float urand(void) {
    rng = rng * 6364136223846793005ull + 1442695040888963407ull;
    return (float)((rng >> 40) & 0xFFFFFF) / 16777216.0f * 2.0f - 1.0f;
}

static void *fill(int64_t count, int32_t dtype) {
    if (dtype == 0) {
        float *a = malloc((size_t)count * sizeof(float));
        for (int64_t i = 0; i < count; ++i) a[i] = urand();
        return a;
    }
    uint16_t *a = malloc((size_t)count * sizeof(uint16_t));
    for (int64_t i = 0; i < count; ++i) {
        float f = urand();
        uint32_t u;
        memcpy(&u, &f, 4);
        a[i] = (uint16_t)(u >> 16);
    }
    return a;
}

static int failures = 0;
#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                                   \
        }                                                                 \
    } while (0)

static void run(int64_t B, int64_t Hq, int64_t Hkv, int64_t n, int64_t nq, int64_t d, int64_t W,
                int64_t topk, int32_t dtype) {
    oracle_problem p = {B, Hq, Hkv, n, nq, d, W, topk, dtype, 2};
    void *q = fill(B * Hq * nq * d, dtype), *k = fill(B * Hkv * n * d, dtype), *v = fill(B * Hkv * n * d, dtype);
    const int64_t nv = B * Hq * nq, cap = 1 + W + topk;
    int32_t *idx = malloc((size_t)(nv * cap) * sizeof(int32_t));
    double *out = malloc((size_t)(nv * d) * sizeof(double)), *diag = malloc((size_t)(nv * 8) * sizeof(double));
    double *out2 = malloc((size_t)(nv * d) * sizeof(double));
    CHECK(oracle_condensate(&p, q, k, v, idx, out, diag) == 0);
    for (int64_t e = 0; e < nv * d; ++e) CHECK(isfinite(out[e]));
    for (int64_t r = 0; r < nv; ++r) {
        double s = diag[r * 8 + 2] + diag[r * 8 + 5] + diag[r * 8 + 6] + diag[r * 8 + 7];
        CHECK(fabs(s - 1.0) < 1e-9);
    }
    CHECK(oracle_restricted(&p, q, k, v, idx, cap, out2) == 0);
    for (int64_t e = 0; e < nv * d; ++e) CHECK(out2[e] == out[e]);
    CHECK(oracle_full(&p, q, k, v, out2) == 0);
    /* A subset of rows, last first: the same rows as the whole call. */
    int64_t rows[3] = {nv - 1, 0, nv / 2};
    int32_t *idx3 = malloc((size_t)(3 * cap) * sizeof(int32_t));
    double *out3 = malloc((size_t)(3 * d) * sizeof(double)), *diag3 = malloc(3 * 8 * sizeof(double));
    CHECK(oracle_condensate_rows(&p, q, k, v, rows, 3, idx3, out3, diag3) == 0);
    for (int t = 0; t < 3; ++t)
        for (int64_t c = 0; c < cap; ++c) CHECK(idx3[t * cap + c] == idx[rows[t] * cap + c]);
    /* Argument errors. */
    int64_t bad_rows[1] = {nv};
    CHECK(oracle_condensate_rows(&p, q, k, v, bad_rows, 1, idx3, out3, diag3) != 0);
    oracle_problem bad = p;
    bad.kv_heads = Hq + 1;
    CHECK(oracle_condensate(&bad, q, k, v, idx, out, diag) != 0);
    bad = p;
    bad.nq = n + 1;
    CHECK(oracle_condensate(&bad, q, k, v, idx, out, diag) != 0);
    bad = p;
    bad.W = 0;
    CHECK(oracle_condensate(&bad, q, k, v, idx, out, diag) != 0);
    CHECK(oracle_condensate(&p, NULL, k, v, idx, out, diag) != 0);
    free(q); free(k); free(v); free(idx); free(out); free(diag); free(out2);
    free(idx3); free(out3); free(diag3);
}

int main(void) {
    run(1, 2, 1, 200, 1, 16, 16, 8, 0);      /* decode, GQA 2 */
    run(2, 4, 2, 120, 30, 32, 20, 12, 1);    /* bf16, batch 2, multi-query */
    run(1, 1, 1, 97, 97, 8, 8, 4, 0);        /* full prefill, rows with i < W */
    run(1, 3, 3, 64, 64, 8, 1, 5, 0);        /* W = 1 */
    run(1, 2, 2, 50, 10, 8, 40, 30, 1);      /* k larger than |R_i| */
    run(1, 2, 1, 120, 7, 16, 10, 0, 0);      /* k = 0 */
    run(1, 2, 1, 30, 5, 8, 64, 8, 0);        /* the window covers every position */
    run(1, 1, 1, 1, 1, 8, 4, 4, 1);          /* n = 1 */
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle exercise: all checks passed\n");
    return 0;
}
