/* Host-sanitizer driver for the CPU oracle (test infrastructure): runs every
 * oracle entry point on small and medium seeded inputs -- edge sizes, k = n,
 * INT32 extremes, +-0, +-inf, denormals, zero rows -- and the argument
 * rejections, checking that each result is sorted by the comparator.  Built
 * with -fsanitize=address,undefined by tests/test_host_sanitizers.py; any
 * sanitizer report aborts the run. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_search_metric(const float *corpus, int64_t n, int64_t d, const float *queries, int64_t q, int64_t k,
                         int32_t metric, int32_t *out_idx, double *out_score);
int oracle_topk_i32(const int32_t *values, int64_t n, int64_t k, int32_t *out_idx, int32_t *out_val);
int oracle_topk_f32(const float *values, int64_t n, int64_t k, int32_t *out_idx, float *out_val);
int oracle_num_threads(void);

static uint64_t state = 0x9e3779b97f4a7c15ull;
static uint64_t next(void) { /* splitmix64 */
    uint64_t z = (state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}
static float unit(void) { return (float)((double)(next() >> 11) / 9007199254740992.0 * 2.0 - 1.0); }

static int fail(const char *what) {
    fprintf(stderr, "FAIL: %s\n", what);
    return 1;
}

static int check_search(int64_t n, int64_t d, int64_t q, int64_t k, int32_t metric, int zero_rows) {
    float *c = malloc(sizeof(float) * (size_t)(n * d));
    float *qs = malloc(sizeof(float) * (size_t)(q * d));
    int32_t *idx = malloc(sizeof(int32_t) * (size_t)(q * k));
    double *sc = malloc(sizeof(double) * (size_t)(q * k));
    for (int64_t i = 0; i < n * d; ++i) c[i] = unit();
    for (int64_t i = 0; i < q * d; ++i) qs[i] = unit();
    if (zero_rows)
        for (int64_t i = 0; i < n; i += 3) memset(c + i * d, 0, sizeof(float) * (size_t)d);
    int rc = oracle_search_metric(c, n, d, qs, q, k, metric, idx, sc);
    int bad = rc != 0;
    for (int64_t qi = 0; qi < q && !bad; ++qi)
        for (int64_t r = 0; r + 1 < k; ++r) {
            const double a = sc[qi * k + r], b = sc[qi * k + r + 1];
            if (!(a > b || (a == b && idx[qi * k + r] < idx[qi * k + r + 1]))) bad = 1;
        }
    free(c);
    free(qs);
    free(idx);
    free(sc);
    return bad;
}

int main(void) {
    int bad = 0;
    if (oracle_num_threads() < 1) bad |= fail("threads");
    /* retrieval: tiny to medium sizes, both metrics, k up to n */
    const int64_t ns[] = {1, 2, 7, 64, 65, 1000, 20000};
    for (size_t a = 0; a < sizeof(ns) / sizeof(ns[0]); ++a)
        for (int64_t d = 1; d <= 9; d += 4)
            for (int32_t metric = 0; metric <= 1; ++metric) {
                const int64_t n = ns[a];
                const int64_t ks[] = {1, n < 5 ? n : 5, n};
                for (int j = 0; j < 3; ++j)
                    if (check_search(n, d, 3, ks[j], metric, metric)) bad |= fail("search");
            }
    /* int32: extremes and k = n */
    {
        const int64_t n = 4096;
        int32_t *v = malloc(sizeof(int32_t) * n), *oi = malloc(sizeof(int32_t) * n), *ov = malloc(sizeof(int32_t) * n);
        for (int64_t i = 0; i < n; ++i) v[i] = (int32_t)(uint32_t)next();
        v[0] = INT32_MIN;
        v[1] = INT32_MAX;
        v[2] = INT32_MIN;
        v[3] = INT32_MAX;
        if (oracle_topk_i32(v, n, n, oi, ov) != 0) bad |= fail("topk_i32");
        for (int64_t r = 0; r + 1 < n; ++r)
            if (!((int64_t)ov[r] > (int64_t)ov[r + 1] || (ov[r] == ov[r + 1] && oi[r] < oi[r + 1])))
                bad |= fail("topk_i32 order");
        if (ov[0] != INT32_MAX || oi[0] != 1 || oi[1] != 3) bad |= fail("topk_i32 extremes");
        if (ov[n - 1] != INT32_MIN || oi[n - 1] != 2) bad |= fail("topk_i32 minimum");
        if (oracle_topk_i32(v, 1, 1, oi, ov) != 0 || oi[0] != 0) bad |= fail("topk_i32 n=1");
        free(v);
        free(oi);
        free(ov);
    }
    /* fp32: +-0, +-inf, denormals, k = n */
    {
        const int64_t n = 2048;
        float *v = malloc(sizeof(float) * n), *ov = malloc(sizeof(float) * n);
        int32_t *oi = malloc(sizeof(int32_t) * n);
        for (int64_t i = 0; i < n; ++i) v[i] = unit();
        v[5] = -0.0f;
        v[6] = 0.0f;
        v[7] = INFINITY;
        v[8] = -INFINITY;
        v[9] = 1e-45f;
        v[10] = -1e-45f;
        if (oracle_topk_f32(v, n, n, oi, ov) != 0) bad |= fail("topk_f32");
        for (int64_t r = 0; r + 1 < n; ++r)
            if (!(ov[r] > ov[r + 1] || (ov[r] == ov[r + 1] && oi[r] < oi[r + 1]))) bad |= fail("topk_f32 order");
        if (oi[0] != 7 || oi[n - 1] != 8) bad |= fail("topk_f32 infinities");
        free(v);
        free(ov);
        free(oi);
    }
    /* argument rejections */
    {
        float f = 0.f;
        int32_t i32 = 0;
        double dd = 0.0;
        if (oracle_search_metric(&f, 1, 1, &f, 1, 2, 0, &i32, &dd) != 1) bad |= fail("k > n");
        if (oracle_search_metric(&f, 1, 1, &f, 1, 1, 2, &i32, &dd) != 1) bad |= fail("metric");
        if (oracle_search_metric(NULL, 1, 1, &f, 1, 1, 0, &i32, &dd) != 1) bad |= fail("null corpus");
        if (oracle_topk_i32(&i32, 0, 1, &i32, &i32) != 1) bad |= fail("n = 0");
        if (oracle_topk_f32(&f, 1, 0, &i32, &f) != 1) bad |= fail("k = 0");
    }
    if (!bad) printf("ok\n");
    return bad;
}
