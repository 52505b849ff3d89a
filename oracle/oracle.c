/*
 * oracle.c -- plain, slow, obviously-correct CPU oracle for exact resident top-K.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's cpu_baseline leg may load or call this library.  The product
 * (libresident_topk and its Python binding) never links, imports or calls it,
 * and shares no code, header, table or helper with it.
 *
 * What it computes, and where the definition comes from:
 *
 *  - Order ("better"): a (score, index) pair beats another iff its score is
 *    larger, or the scores compare equal and its index is smaller.  This is the
 *    comparator of "GPU-Resident Top-K for Agentic RAG" (A. Banerjee), section 3,
 *    "Problem B": the same rule is used on host and device so ties resolve
 *    identically.  Float equality is IEEE equality, so -0.0 ties +0.0.
 *    Indices are unique, so on NaN-free inputs this is a strict total order and
 *    sorting by it gives the same result as a stable sort by descending score.
 *
 *  - Retrieval: the score of corpus row i for query q is the inner product
 *    sum_d C[i,d] * q[d] (same article, section 4 "Step 2", dot-product mode).
 *    Every fp32*fp32 product is exact in fp64 (24+24 significand bits <= 53), and
 *    the sum is taken in fp64 in ascending d.  All N rows are scored, the (score,
 *    index) pairs are fully sorted by "better", and the first K are returned
 *    best-first (section 4 "Step 4": results come back best-first; the method is
 *    exact brute force, section 6).
 *
 *  - Cosine mode (same article, section 4 "Step 2", the cosine branch of the
 *    scoring kernel; section 7 on the two metrics): the inner product divided by
 *    the product of the query's and the row's L2 norms, and -inf when that
 *    product is not positive (a zero row or a zero query).  Norms are the square
 *    root of the fp64 sum of squares taken in ascending d.
 *
 *  - Plain top-K over a raw int32 / fp32 array: the K largest values, ties to
 *    the lower index ("CUDA Programming Model Series 9: Efficient TopK, two-stage
 *    reduction kernel design", section 1 and 2.1 state the largest-K task; the tie
 *    rule is the comparator above).  int32 values are widened to int64 before
 *    comparison so no negation or subtraction can overflow; fp32 values are
 *    compared as floats.  Returned values are the input's own bits.
 *
 * Precondition (not checked): inputs are NaN-free.  The comparator is not an
 * order on NaN.
 *
 * Parallelism: only the row-scoring loop is split across OpenMP threads; each
 * row's sum is still a single sequential fp64 loop, so the result does not depend
 * on the thread count.  Sorting uses the C library qsort with a total-order
 * comparator, so its output is unique.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ order */

typedef struct {
    double score;
    int64_t index;
} scored_row;

typedef struct {
    int64_t value;
    int64_t index;
} int_item;

typedef struct {
    float value;
    int64_t index;
} float_item;

/* qsort comparators: negative when a must come first, i.e. when a is better. */
static int better_first_scored(const void *pa, const void *pb) {
    const scored_row *a = (const scored_row *)pa;
    const scored_row *b = (const scored_row *)pb;
    if (a->score != b->score) return (a->score > b->score) ? -1 : 1;
    if (a->index != b->index) return (a->index < b->index) ? -1 : 1;
    return 0;
}

static int better_first_int(const void *pa, const void *pb) {
    const int_item *a = (const int_item *)pa;
    const int_item *b = (const int_item *)pb;
    if (a->value != b->value) return (a->value > b->value) ? -1 : 1;
    if (a->index != b->index) return (a->index < b->index) ? -1 : 1;
    return 0;
}

static int better_first_float(const void *pa, const void *pb) {
    const float_item *a = (const float_item *)pa;
    const float_item *b = (const float_item *)pb;
    if (a->value != b->value) return (a->value > b->value) ? -1 : 1;
    if (a->index != b->index) return (a->index < b->index) ? -1 : 1;
    return 0;
}

/* ------------------------------------------------------------------ API */

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* scores[i] = sum_{d=0}^{D-1} (double)corpus[i*D+d] * (double)query[d], for i < n. */
int oracle_scores(const float *corpus, int64_t n, int64_t d, const float *query, double *scores) {
    if (n < 0 || d < 1 || (n > 0 && (!corpus || !query || !scores))) return 1;
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i) {
        const float *row = corpus + i * d;
        double acc = 0.0;
        for (int64_t c = 0; c < d; ++c) acc += (double)row[c] * (double)query[c];
        scores[i] = acc;
    }
    return 0;
}

/*
 * Cosine scores: scores[i] = <row i, query> / (|query| |row i|), or -inf when
 * |query| |row i| is not positive.  The inner products are oracle_scores'.
 */
int oracle_cosine_scores(const float *corpus, int64_t n, int64_t d, const float *query, double *scores) {
    if (n < 0 || d < 1 || (n > 0 && (!corpus || !query || !scores))) return 1;
    int rc = oracle_scores(corpus, n, d, query, scores);
    if (rc) return rc;
    double q_sq = 0.0;
    for (int64_t c = 0; c < d; ++c) q_sq += (double)query[c] * (double)query[c];
    const double q_norm = sqrt(q_sq);
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i) {
        const float *row = corpus + i * d;
        double r_sq = 0.0;
        for (int64_t c = 0; c < d; ++c) r_sq += (double)row[c] * (double)row[c];
        const double denom = q_norm * sqrt(r_sq);
        scores[i] = (denom > 0.0) ? scores[i] / denom : -INFINITY;
    }
    return 0;
}

/*
 * As oracle_search, with metric 0 = inner product, 1 = cosine.
 */
int oracle_search_metric(const float *corpus, int64_t n, int64_t d, const float *queries, int64_t q,
                         int64_t k, int32_t metric, int32_t *out_idx, double *out_score) {
    if (n < 1 || d < 1 || q < 1 || k < 1 || k > n || metric < 0 || metric > 1) return 1;
    if (!corpus || !queries || !out_idx || !out_score) return 1;
    double *scores = (double *)malloc(sizeof(double) * (size_t)n);
    scored_row *rows = (scored_row *)malloc(sizeof(scored_row) * (size_t)n);
    if (!scores || !rows) {
        free(scores);
        free(rows);
        return 2;
    }
    for (int64_t qi = 0; qi < q; ++qi) {
        if (metric == 1)
            oracle_cosine_scores(corpus, n, d, queries + qi * d, scores);
        else
            oracle_scores(corpus, n, d, queries + qi * d, scores);
        for (int64_t i = 0; i < n; ++i) {
            rows[i].score = scores[i];
            rows[i].index = i;
        }
        qsort(rows, (size_t)n, sizeof(scored_row), better_first_scored);
        for (int64_t r = 0; r < k; ++r) {
            out_idx[qi * k + r] = (int32_t)rows[r].index;
            out_score[qi * k + r] = rows[r].score;
        }
    }
    free(scores);
    free(rows);
    return 0;
}

/*
 * For each of the q queries (row-major q x d), score all n corpus rows by inner
 * product, sort all (score, index) pairs by "better" and write the first k:
 * indices to out_idx[qi*k + r], fp64 scores to out_score[qi*k + r].
 * Returns 0 on success, 1 on bad arguments, 2 if memory runs out.
 */
int oracle_search(const float *corpus, int64_t n, int64_t d, const float *queries, int64_t q,
                  int64_t k, int32_t *out_idx, double *out_score) {
    return oracle_search_metric(corpus, n, d, queries, q, k, 0, out_idx, out_score);
}

/* K largest of an int32 array, ties to the lower index; values widened to int64. */
int oracle_topk_i32(const int32_t *values, int64_t n, int64_t k, int32_t *out_idx, int32_t *out_val) {
    if (n < 1 || k < 1 || k > n || !values || !out_idx || !out_val) return 1;
    int_item *items = (int_item *)malloc(sizeof(int_item) * (size_t)n);
    if (!items) return 2;
    for (int64_t i = 0; i < n; ++i) {
        items[i].value = (int64_t)values[i];
        items[i].index = i;
    }
    qsort(items, (size_t)n, sizeof(int_item), better_first_int);
    for (int64_t r = 0; r < k; ++r) {
        out_idx[r] = (int32_t)items[r].index;
        out_val[r] = values[items[r].index];
    }
    free(items);
    return 0;
}

/* K largest of an fp32 array under float comparison (-0.0 == +0.0), ties to the
 * lower index; the returned values are the input's own bit patterns. */
int oracle_topk_f32(const float *values, int64_t n, int64_t k, int32_t *out_idx, float *out_val) {
    if (n < 1 || k < 1 || k > n || !values || !out_idx || !out_val) return 1;
    float_item *items = (float_item *)malloc(sizeof(float_item) * (size_t)n);
    if (!items) return 2;
    for (int64_t i = 0; i < n; ++i) {
        items[i].value = values[i];
        items[i].index = i;
    }
    qsort(items, (size_t)n, sizeof(float_item), better_first_float);
    for (int64_t r = 0; r < k; ++r) {
        out_idx[r] = (int32_t)items[r].index;
        memcpy(&out_val[r], &values[items[r].index], sizeof(float));
    }
    free(items);
    return 0;
}
