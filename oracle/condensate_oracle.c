/*
 * CPU oracle for condensate ("topological") attention.
 *
 * TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the benchmark's CPU-baseline
 * leg are the only code allowed to load this library. The product path (the HIP library
 * and its Python binding) never calls it, and the two share no source, header or helper.
 *
 * Plain float64 C, one query at a time, so that each step can be checked by eye against the
 * pages of "The Condensate Theorem: Transformers Are O(n), Not O(n^2)" (arXiv:2602.06317);
 * the section names below are those of the metaphor-xennon blog page about it, the only
 * page with equations:
 *
 *   step 1  scores       s_j = (q . k_j) / sqrt(d) for j <= i              (sec. 1.1 eq.; sec. 2.1 S = QK^T/sqrt(d_k))
 *   step 2  anchor {0}, window {max(0,i-W+1)..i}, candidates R = {1..i-W}   (sec. 2.1 Definition 1; 2.2.1; 2.2.2)
 *   step 3  top-k: sort R by (score descending, index ascending), keep
 *           the first min(k, |R|); tau = score of the last one kept         (sec. 2.2.3 eq.; 3.2.1 lemma, tau_min)
 *   step 4  C = anchor u window u top-k, ascending, padded with -1          (sec. 2.1 Definition 1; 2.4 Corollary 2)
 *   step 5  softmax restricted to C, times V: m = max_C s, p_j = exp(s_j-m),
 *           o = sum_C p_j v_j / sum_C p_j, summed in ascending j            (sec. 2.3 Theorem 1 Attention_C; 3.2.4 Theorem 4)
 *   full    the same step 5 with C = {0..i}: plain causal attention         (sec. 1.1 eq.)
 *   eps     excluded mass: full-softmax weight of positions outside C       (sec. 3.2.2)
 *   masses  full-softmax weight of the anchor, the window (without 0) and
 *           the top-k positions; with eps they sum to 1                     (sec. 2.2.1-2.2.3, 3.2.2)
 *
 * Readings where the pages are silent or loose (each also listed with the design notes):
 *   - top-k ranks only R, the positions outside the anchor and the window (the section 4.2.1
 *     table counts the three parts as disjoint, 1+64+32 = 97, and Corollary 2 bounds |C_i| by
 *     1+W+k); ranks are over causal positions j <= i only;
 *   - if |R| < k all of R is taken, so |C_i| = min(i+1, 1+W+k);
 *   - equal scores: the smaller position wins;
 *   - queries are the last nq positions: query row r sits at position i = n - nq + r;
 *   - GQA: query head h reads KV head h / (heads / kv_heads).
 *
 * Inputs are read as stored (float32, or bfloat16 widened exactly) and every sum runs in
 * float64 in index order. Parity of this file is pinned by the CPU tests (closed forms,
 * brute force on tiny inputs, library attention with masks, special cases, identities).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int64_t batch, heads, kv_heads, n, nq, d, W, topk;
    int32_t dtype; /* 0 = float32, 1 = bfloat16 */
    int32_t threads; /* OpenMP threads to use; <= 0 means the runtime default */
} oracle_problem;

enum { OR_OK = 0, OR_BAD_ARG = -1, OR_NO_MEM = -2 };

/* One stored element, widened exactly to double. */
static double load_elem(const void *base, int32_t dtype, int64_t idx)
{
    if (dtype == 0)
        return (double)((const float *)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static int check_problem(const oracle_problem *p)
{
    if (!p) return OR_BAD_ARG;
    if (p->batch < 1 || p->heads < 1 || p->kv_heads < 1 || p->heads % p->kv_heads) return OR_BAD_ARG;
    if (p->n < 1 || p->nq < 1 || p->nq > p->n || p->d < 1) return OR_BAD_ARG;
    if (p->W < 1 || p->topk < 0) return OR_BAD_ARG;
    if (p->dtype != 0 && p->dtype != 1) return OR_BAD_ARG;
    return OR_OK;
}

/* Where query (b, h, r) and its keys live. */
typedef struct {
    int64_t i;        /* absolute position of the query */
    int64_t q_off;    /* element offset of the query row */
    int64_t kv_off;   /* element offset of key/value row 0 of its KV head */
} query_loc;

static query_loc locate(const oracle_problem *p, int64_t flat)
{
    int64_t r = flat % p->nq;
    int64_t bh = flat / p->nq;
    int64_t h = bh % p->heads;
    int64_t b = bh / p->heads;
    int64_t kvh = h / (p->heads / p->kv_heads);
    query_loc L;
    L.i = p->n - p->nq + r;
    L.q_off = flat * p->d;
    L.kv_off = (b * p->kv_heads + kvh) * p->n * p->d;
    return L;
}

/* Step 1: s_j = (sum_t q[t] k_j[t]) / sqrt(d), accumulated in t order. */
static double score(const oracle_problem *p, const double *qrow, const void *k, int64_t kv_off, int64_t j)
{
    double acc = 0.0;
    int64_t base = kv_off + j * p->d;
    for (int64_t t = 0; t < p->d; ++t)
        acc += qrow[t] * load_elem(k, p->dtype, base + t);
    return acc * (1.0 / sqrt((double)p->d));
}

/* Step 5: softmax over the listed positions (ascending), times V. */
static void attend(const oracle_problem *p, const int64_t *list, int64_t count, const double *s_of_list,
                   const void *v, int64_t kv_off, double *o)
{
    double m = -INFINITY;
    for (int64_t c = 0; c < count; ++c)
        if (s_of_list[c] > m) m = s_of_list[c];
    double l = 0.0;
    for (int64_t t = 0; t < p->d; ++t) o[t] = 0.0;
    for (int64_t c = 0; c < count; ++c) {
        double w = exp(s_of_list[c] - m);
        l += w;
        int64_t base = kv_off + list[c] * p->d;
        for (int64_t t = 0; t < p->d; ++t)
            o[t] += w * load_elem(v, p->dtype, base + t);
    }
    for (int64_t t = 0; t < p->d; ++t) o[t] /= l;
}

typedef struct { double s; int64_t j; } ranked;

/* Higher score first; equal scores: smaller position first. A total order on distinct j. */
static int rank_order(const void *pa, const void *pb)
{
    const ranked *a = (const ranked *)pa, *b = (const ranked *)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->j < b->j) ? -1 : (a->j > b->j);
}

typedef struct {
    double *qrow, *s, *s_list;
    ranked *cand;
    unsigned char *member;
    int64_t *list;
} scratch_bufs;

static int scratch_alloc(scratch_bufs *w, int64_t n, int64_t d)
{
    w->qrow = (double *)malloc(sizeof(double) * d);
    w->s = (double *)malloc(sizeof(double) * n);
    w->s_list = (double *)malloc(sizeof(double) * n);
    w->cand = (ranked *)malloc(sizeof(ranked) * n);
    w->member = (unsigned char *)malloc(n);
    w->list = (int64_t *)malloc(sizeof(int64_t) * n);
    return (w->qrow && w->s && w->s_list && w->cand && w->member && w->list) ? OR_OK : OR_NO_MEM;
}

static void scratch_free(scratch_bufs *w)
{
    free(w->qrow); free(w->s); free(w->s_list); free(w->cand); free(w->member); free(w->list);
}

static void load_query(const oracle_problem *p, const void *q, const query_loc *L, double *qrow)
{
    for (int64_t t = 0; t < p->d; ++t) qrow[t] = load_elem(q, p->dtype, L->q_off + t);
}

/* Steps 1-6 for one query. diag gets {tau, max_j |s_j|, eps, |C|, k', and the full-softmax
 * mass of position 0, of the window positions other than 0, and of the top-k positions}. */
static void condensate_query(const oracle_problem *p, const void *q, const void *k, const void *v,
                             int64_t flat, scratch_bufs *w, int32_t *idx_row, double *o, double *diag)
{
    const query_loc L = locate(p, flat);
    const int64_t i = L.i;
    load_query(p, q, &L, w->qrow);

    /* Step 1: every causal score. */
    for (int64_t j = 0; j <= i; ++j) w->s[j] = score(p, w->qrow, k, L.kv_off, j);

    /* Step 2: anchor {0}, window {wlo..i}, candidates R = {1..i-W}. */
    const int64_t wlo = (i - p->W + 1 > 0) ? i - p->W + 1 : 0;
    const int64_t r_last = i - p->W; /* R is empty when r_last < 1 */
    const int64_t n_r = r_last >= 1 ? r_last : 0;

    /* Step 3: explicit sort of R by (score desc, index asc); keep the first k'. */
    for (int64_t t = 0; t < n_r; ++t) { w->cand[t].s = w->s[1 + t]; w->cand[t].j = 1 + t; }
    qsort(w->cand, (size_t)n_r, sizeof(ranked), rank_order);
    const int64_t kp = p->topk < n_r ? p->topk : n_r;
    const double tau = kp > 0 ? w->cand[kp - 1].s : NAN;

    /* Step 4: C = {0} u window u top-k', listed in ascending position. */
    memset(w->member, 0, (size_t)(i + 1));
    w->member[0] = 1;
    for (int64_t j = wlo; j <= i; ++j) w->member[j] = 1;
    for (int64_t t = 0; t < kp; ++t) w->member[w->cand[t].j] = 1;
    int64_t count = 0;
    for (int64_t j = 0; j <= i; ++j)
        if (w->member[j]) { w->list[count] = j; w->s_list[count] = w->s[j]; ++count; }
    const int64_t cap = 1 + p->W + p->topk;
    for (int64_t c = 0; c < cap; ++c) idx_row[c] = c < count ? (int32_t)w->list[c] : -1;

    /* Step 5: softmax restricted to C, times V. */
    attend(p, w->list, count, w->s_list, v, L.kv_off, o);

    /* Step 6: diagnostics -- max |s|, and the full-softmax mass outside C. */
    double mabs = 0.0, mall = -INFINITY;
    for (int64_t j = 0; j <= i; ++j) {
        if (fabs(w->s[j]) > mabs) mabs = fabs(w->s[j]);
        if (w->s[j] > mall) mall = w->s[j];
    }
    double z_all = 0.0, z_out = 0.0;
    for (int64_t j = 0; j <= i; ++j) {
        double e = exp(w->s[j] - mall);
        z_all += e;
        if (!w->member[j]) z_out += e;
    }
    /* The parts of C: the anchor (sec. 2.2.1, its share of the mass), the window without
     * position 0 (sec. 2.2.2), and the top-k positions (sec. 2.2.3), which lie in R. */
    const double z_anchor = exp(w->s[0] - mall);
    double z_window = 0.0, z_topk = 0.0;
    for (int64_t j = wlo > 1 ? wlo : 1; j <= i; ++j) z_window += exp(w->s[j] - mall);
    for (int64_t t = 0; t < kp; ++t) z_topk += exp(w->s[w->cand[t].j] - mall);
    if (diag) {
        diag[0] = tau;
        diag[1] = mabs;
        diag[2] = z_out / z_all;
        diag[3] = (double)count;
        diag[4] = (double)kp;
        diag[5] = z_anchor / z_all;
        diag[6] = z_window / z_all;
        diag[7] = z_topk / z_all;
    }
}

static void set_threads(const oracle_problem *p)
{
#ifdef _OPENMP
    if (p->threads > 0) omp_set_num_threads(p->threads);
#else
    (void)p;
#endif
}

#define N_DIAG 8

int oracle_condensate_rows(const oracle_problem *p, const void *q, const void *k, const void *v,
                           const int64_t *rows, int64_t nrows, int32_t *out_idx, double *out,
                           double *diag);
int oracle_restricted_rows(const oracle_problem *p, const void *q, const void *k, const void *v,
                           const int64_t *rows, int64_t nrows, const int32_t *idx,
                           int64_t idx_stride, double *out);
int oracle_full_rows(const oracle_problem *p, const void *q, const void *k, const void *v,
                     const int64_t *rows, int64_t nrows, double *out);

/* The whole method for every query of the problem.
 * out_idx: [batch][heads][nq][1+W+topk] int32; out: [batch][heads][nq][d] float64;
 * diag (may be NULL): [batch][heads][nq][8] float64 = {tau, max|s|, eps, |C|, k', mass of
 * position 0, of the window without 0, of the top-k}. */
int oracle_condensate(const oracle_problem *p, const void *q, const void *k, const void *v,
                      int32_t *out_idx, double *out, double *diag)
{
    return oracle_condensate_rows(p, q, k, v, NULL, 0, out_idx, out, diag);
}

/* Checks a row list (NULL = every query, in flat order) and returns how many rows it names,
 * or -1 if an entry is outside [0, nflat). */
static int64_t row_count(const oracle_problem *p, const int64_t *rows, int64_t nrows)
{
    const int64_t nflat = p->batch * p->heads * p->nq;
    if (!rows) return nflat;
    if (nrows < 0) return -1;
    for (int64_t t = 0; t < nrows; ++t)
        if (rows[t] < 0 || rows[t] >= nflat) return -1;
    return nrows;
}

/* The whole method for the listed queries only: rows[t] is a flat query index
 * b*heads*nq + h*nq + r, and result t goes to out_idx[t][1+W+topk], out[t][d], diag[t][8].
 * rows == NULL means every query in flat order (then nrows is ignored). */
int oracle_condensate_rows(const oracle_problem *p, const void *q, const void *k, const void *v,
                           const int64_t *rows, int64_t nrows, int32_t *out_idx, double *out,
                           double *diag)
{
    int rc = check_problem(p);
    if (rc) return rc;
    if (!q || !k || !v || !out_idx || !out) return OR_BAD_ARG;
    const int64_t count = row_count(p, rows, nrows);
    if (count < 0) return OR_BAD_ARG;
    const int64_t cap = 1 + p->W + p->topk;
    int failed = 0;
    set_threads(p);
#pragma omp parallel reduction(| : failed)
    {
        scratch_bufs w;
        if (scratch_alloc(&w, p->n, p->d) != OR_OK) {
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t t = 0; t < count; ++t) {
                const int64_t f = rows ? rows[t] : t;
                condensate_query(p, q, k, v, f, &w, out_idx + t * cap, out + t * p->d,
                                 diag ? diag + t * N_DIAG : NULL);
            }
        }
        scratch_free(&w);
    }
    return failed ? OR_NO_MEM : OR_OK;
}

/* Step 5 alone on caller-supplied sets. idx: [batch][heads][nq][idx_stride] int32, each row a
 * set of distinct positions in 0..i in any order, padded with -1. out: [..][d] float64.
 * Returns OR_BAD_ARG (and leaves that row's output untouched) if a row is empty, holds an
 * out-of-range position or repeats one. */
int oracle_restricted(const oracle_problem *p, const void *q, const void *k, const void *v,
                      const int32_t *idx, int64_t idx_stride, double *out)
{
    return oracle_restricted_rows(p, q, k, v, NULL, 0, idx, idx_stride, out);
}

/* Step 5 alone for the listed queries (rows as in oracle_condensate_rows): idx[t] is the set
 * of query rows[t], out[t] its result. */
int oracle_restricted_rows(const oracle_problem *p, const void *q, const void *k, const void *v,
                           const int64_t *rows, int64_t nrows, const int32_t *idx,
                           int64_t idx_stride, double *out)
{
    int rc = check_problem(p);
    if (rc) return rc;
    if (!q || !k || !v || !idx || !out || idx_stride < 1) return OR_BAD_ARG;
    const int64_t count = row_count(p, rows, nrows);
    if (count < 0) return OR_BAD_ARG;
    int bad = 0, failed = 0;
    set_threads(p);
#pragma omp parallel reduction(| : bad, failed)
    {
        scratch_bufs w;
        if (scratch_alloc(&w, p->n, p->d) != OR_OK) {
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t t = 0; t < count; ++t) {
                const int64_t f = rows ? rows[t] : t;
                const query_loc L = locate(p, f);
                memset(w.member, 0, (size_t)(L.i + 1));
                int row_bad = 0;
                for (int64_t c = 0; c < idx_stride; ++c) {
                    int32_t j = idx[t * idx_stride + c];
                    if (j < 0) continue;
                    if (j > L.i || w.member[j]) { row_bad = 1; break; }
                    w.member[j] = 1;
                }
                int64_t members = 0;
                if (!row_bad) {
                    load_query(p, q, &L, w.qrow);
                    for (int64_t j = 0; j <= L.i; ++j)
                        if (w.member[j]) {
                            w.list[members] = j;
                            w.s_list[members] = score(p, w.qrow, k, L.kv_off, j);
                            ++members;
                        }
                }
                if (row_bad || members == 0) { bad = 1; continue; }
                attend(p, w.list, members, w.s_list, v, L.kv_off, out + t * p->d);
            }
        }
        scratch_free(&w);
    }
    if (failed) return OR_NO_MEM;
    return bad ? OR_BAD_ARG : OR_OK;
}

/* Plain causal attention (step 5 with C = {0..i}) for every query. out: [..][d] float64. */
int oracle_full(const oracle_problem *p, const void *q, const void *k, const void *v, double *out)
{
    return oracle_full_rows(p, q, k, v, NULL, 0, out);
}

/* Plain causal attention for the listed queries (rows as in oracle_condensate_rows). */
int oracle_full_rows(const oracle_problem *p, const void *q, const void *k, const void *v,
                     const int64_t *rows, int64_t nrows, double *out)
{
    int rc = check_problem(p);
    if (rc) return rc;
    if (!q || !k || !v || !out) return OR_BAD_ARG;
    const int64_t count = row_count(p, rows, nrows);
    if (count < 0) return OR_BAD_ARG;
    int failed = 0;
    set_threads(p);
#pragma omp parallel reduction(| : failed)
    {
        scratch_bufs w;
        if (scratch_alloc(&w, p->n, p->d) != OR_OK) {
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t t = 0; t < count; ++t) {
                const int64_t f = rows ? rows[t] : t;
                const query_loc L = locate(p, f);
                load_query(p, q, &L, w.qrow);
                for (int64_t j = 0; j <= L.i; ++j) {
                    w.list[j] = j;
                    w.s_list[j] = score(p, w.qrow, k, L.kv_off, j);
                }
                attend(p, w.list, L.i + 1, w.s_list, v, L.kv_off, out + t * p->d);
            }
        }
        scratch_free(&w);
    }
    return failed ? OR_NO_MEM : OR_OK;
}

/* Step 1 alone for one query (flat index b*heads*nq + h*nq + r): s[0..i]. */
int oracle_scores(const oracle_problem *p, const void *q, const void *k, int64_t flat, double *s)
{
    int rc = check_problem(p);
    if (rc) return rc;
    if (!q || !k || !s || flat < 0 || flat >= p->batch * p->heads * p->nq) return OR_BAD_ARG;
    const query_loc L = locate(p, flat);
    double *qrow = (double *)malloc(sizeof(double) * p->d);
    if (!qrow) return OR_NO_MEM;
    load_query(p, q, &L, qrow);
    for (int64_t j = 0; j <= L.i; ++j) s[j] = score(p, qrow, k, L.kv_off, j);
    free(qrow);
    return OR_OK;
}

/* Threads an OpenMP region of this library will use for the given request. */
int oracle_threads(int32_t requested)
{
#ifdef _OPENMP
    if (requested > 0) return requested;
    return omp_get_max_threads();
#else
    (void)requested;
    return 1;
#endif
}
