// Host-sanitizer driver for the C ABI's argument checks and status names
// (validate.cpp), test infrastructure: every documented rule at its
// boundaries, built with -fsanitize=address,undefined by
// tests/test_host_sanitizers.py.
#include <stdint.h>
#include <stdio.h>

#include "../../include/resident_topk.h"

static int bad = 0;
static void expect(rt_status got, rt_status want, const char *what) {
    if (got != want) {
        fprintf(stderr, "FAIL: %s: got %d want %d\n", what, (int)got, (int)want);
        bad = 1;
    }
}

int main() {
    static float buf[64];
    const void *p = buf;
    const void *odd = reinterpret_cast<const char *>(buf) + 2;
    for (int s = -1; s <= 5; ++s)
        if (rt_status_string((rt_status)s) == nullptr) bad = 1;
    expect(rt_check_create(1, 1, 1, 1), RT_OK, "create minimum");
    expect(rt_check_create(2147483647LL, 65536, 1024, 32), RT_OK, "create maximum");
    expect(rt_check_create(0, 1, 1, 1), RT_EINVAL, "max_n 0");
    expect(rt_check_create(2147483648LL, 1, 1, 1), RT_EINVAL, "max_n 2^31");
    expect(rt_check_create(INT64_MIN, 1, 1, 1), RT_EINVAL, "max_n INT64_MIN");
    expect(rt_check_create(1, 65537, 1, 1), RT_EINVAL, "max_d");
    expect(rt_check_create(1, INT32_MIN, 1, 1), RT_EINVAL, "max_d INT32_MIN");
    expect(rt_check_create(1, 1, 1025, 1), RT_EINVAL, "max_k");
    expect(rt_check_create(1, 1, 1, 33), RT_EINVAL, "max_q");
    expect(rt_check_upload(10, 8, p, 10, 8), RT_OK, "upload");
    expect(rt_check_upload(10, 8, nullptr, 10, 8), RT_EINVAL, "upload null");
    expect(rt_check_upload(10, 8, p, 11, 8), RT_EINVAL, "upload n");
    expect(rt_check_upload(10, 8, p, 10, 9), RT_EINVAL, "upload d");
    expect(rt_check_upload(10, 8, p, INT64_MAX, 8), RT_EINVAL, "upload n huge");
    expect(rt_check_search(8, 4, 10, p, 4, 8, p, p), RT_OK, "search");
    expect(rt_check_search(8, 4, 10, p, 5, 8, p, p), RT_EINVAL, "search q");
    expect(rt_check_search(8, 4, 10, p, 1, 9, p, p), RT_EINVAL, "search k > max_k");
    expect(rt_check_search(8, 4, 5, p, 1, 6, p, p), RT_EINVAL, "search k > n");
    expect(rt_check_search(8, 4, 0, p, 1, 1, p, p), RT_ESTATE, "search nothing resident");
    expect(rt_check_search(8, 4, 10, nullptr, 1, 1, p, p), RT_EINVAL, "search null");
    expect(rt_check_search_metric(8, 4, 10, p, 1, 1, 1, p, p), RT_OK, "metric cosine");
    expect(rt_check_search_metric(8, 4, 10, p, 1, 1, 2, p, p), RT_EINVAL, "metric unknown");
    expect(rt_check_search_metric(8, 4, 10, p, 1, 1, -1, p, p), RT_EINVAL, "metric negative");
    expect(rt_check_select(1024, p, 0, 100, 100, p, p), RT_OK, "select k == n");
    expect(rt_check_select(1024, p, 1, 2147483647LL, 1024, p, p), RT_OK, "select maximum n");
    expect(rt_check_select(1024, p, 2, 100, 10, p, p), RT_EINVAL, "select dtype");
    expect(rt_check_select(1024, odd, 0, 100, 10, p, p), RT_EINVAL, "select misaligned");
    expect(rt_check_select(1024, p, 0, 2147483648LL, 10, p, p), RT_EINVAL, "select n > 2^31 - 1");
    expect(rt_check_select(1024, p, 0, 0, 1, p, p), RT_EINVAL, "select n 0");
    expect(rt_check_select(1024, p, 0, 10, 11, p, p), RT_EINVAL, "select k > n");
    expect(rt_check_select(8, p, 0, 100, 9, p, p), RT_EINVAL, "select k > max_k");
    if (!bad) printf("ok\n");
    return bad;
}
