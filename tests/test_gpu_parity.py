"""Parity of the HIP path with the CPU oracle at sizes the oracle finishes in
seconds (several tiles, ragged tails, every kernel variant), plus edge cases.

Float retrieval follows rules R1-R4 (gpu_util.check_retrieval); integer and
exact-arithmetic cases are compared bit for bit, in order."""
import numpy as np
import pytest

import oracle
from gpu_util import check_exact_topk_property, check_retrieval
import workloads
from top_search_resident_amd import ResidentTopK, ResidentTopKError

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

MAX_N, MAX_D, MAX_K, MAX_Q = 200_000, 3072, 1024, 32


@pytest.fixture(scope="module")
def eng():
    assert torch.cuda.is_available(), "a GPU is required for the parity tests"
    e = ResidentTopK(MAX_N, MAX_D, MAX_K, MAX_Q, device=0)
    yield e
    e.close()


def _search(eng, corpus, queries, k):
    eng.upload_corpus_rowmajor(corpus)
    q = torch.from_numpy(np.ascontiguousarray(queries)).cuda()
    idx, sc = eng.search_resident(q, k)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), sc.cpu().numpy()


def _check_against_oracle(eng, corpus, queries, k):
    g_idx, g_sc = _search(eng, corpus, queries, k)
    o_idx, o_sc = oracle.search(corpus, queries, k)
    for qi in range(queries.shape[0]):
        check_retrieval(g_idx[qi], g_sc[qi], o_idx[qi], o_sc[qi], corpus, queries[qi], oracle)
    return g_idx, g_sc, o_idx, o_sc


# Shapes that exercise every scoring variant: group widths 64/32/16/1 and
# loads-per-lane 1/2/3/4/6/8 on the vector path, the scalar path for d % 4 != 0
# and for d > 2048, ragged row counts, and list sizes 64..1024.
@pytest.mark.parametrize("n,d,k", [
    (10_000, 384, 8), (12_345, 1024, 8), (12_345, 1024, 100), (7_001, 768, 32), (3_333, 128, 64),
    (5_000, 256, 65), (4_099, 1536, 128), (2_050, 2048, 129), (9_999, 4, 7), (1_000, 12, 3),
    (6_000, 100, 16), (3_001, 3000, 10), (20_000, 64, 256), (30_000, 96, 512), (40_000, 384, 1024),
    (1, 384, 1), (5, 8, 5), (63, 32, 63), (64, 1024, 64), (65, 768, 65), (1_000, 384, 1_000),
])
def test_single_query_gaussian(eng, n, d, k):
    corpus = workloads.gaussian_rows(n, d, config_id=100 + d % 97, stream=0)
    q = workloads.gaussian_rows(1, d, config_id=100 + d % 97, stream=1)
    _check_against_oracle(eng, corpus, q, k)


@pytest.mark.parametrize("n,d,k", [(20_000, 768, 32), (5_000, 100, 40), (3_000, 1024, 1024)])
def test_exact_arithmetic_is_bit_exact(eng, n, d, k):
    """Small-integer inputs make every fp32 dot product exact; the answer must then
    equal the oracle's in indices and scores, including the order of exact ties."""
    corpus = workloads.small_int_matrix(n, d, config_id=7, stream=d)
    q = workloads.small_int_matrix(3, d, config_id=7, stream=d + 1)
    for qi in range(3):
        g_idx, g_sc = _search(eng, corpus, q[qi:qi + 1], k)
        o_idx, o_sc = oracle.search(corpus, q[qi:qi + 1], k)
        assert np.array_equal(g_idx, o_idx), (qi, g_idx[0, :10], o_idx[0, :10])
        assert np.array_equal(g_sc.astype(np.float64), o_sc), qi


def test_duplicate_rows_tie_by_index(eng):
    """Identical rows anywhere in the corpus get bit-identical scores, so the lower
    index wins the tie exactly as in the oracle."""
    n, d, k = 50_000, 1024, 32
    corpus = workloads.gaussian_rows(n, d, config_id=11)
    q = workloads.gaussian_rows(1, d, config_id=11, stream=1)
    best = int(np.argmax(corpus.astype(np.float64) @ q[0].astype(np.float64)))
    rng = np.random.default_rng(3)
    for pos in rng.choice(n, 20, replace=False):
        corpus[pos] = corpus[best]
    g_idx, g_sc = _search(eng, corpus, q, k)
    dup = sorted(set(np.nonzero((corpus == corpus[best]).all(axis=1))[0].tolist()))
    assert list(g_idx[0, :len(dup)]) == dup
    assert np.unique(g_sc[0, :len(dup)]).size == 1
    o_idx, o_sc = oracle.search(corpus, q, k)
    check_retrieval(g_idx[0], g_sc[0], o_idx[0], o_sc[0], corpus, q[0], oracle)


def test_planted_near_ties(eng):
    """Mid-scale recipe at reduced size: 0.5% of rows planted around the query
    anchor, so the k-th boundary sits inside a dense cluster."""
    corpus, qs = workloads.retrieval_inputs("c2_50k_768", queries=6)
    for k in (8, 32):
        _check_against_oracle(eng, corpus, qs, k)


@pytest.mark.parametrize("q,d,k,n", [(2, 768, 100, 20_011), (7, 1024, 8, 20_011), (32, 768, 1024, 20_011),
                                     (32, 384, 100, 20_011), (5, 100, 20, 20_011), (3, 2048, 16, 20_011),
                                     (32, 1024, 1, 20_011), (4, 512, 64, 20_011), (9, 256, 33, 65),
                                     (3, 768, 20, 20), (32, 768, 31, 31), (6, 384, 7, 33)])
def test_batched_queries(eng, q, d, k, n):
    """Batches go through the MFMA scorers when d % 4 == 0 and d <= 1024 (the
    direct-load kernel for d in {256, 384, 512, 768} and n >= 32, with a
    ragged last tile loaded from row n - 32), else through the vector path
    once per query."""
    corpus = workloads.gaussian_rows(n, d, config_id=55, stream=0)
    qs = workloads.gaussian_rows(q, d, config_id=55, stream=1)
    _check_against_oracle(eng, corpus, qs, k)


def test_batched_exact_arithmetic(eng):
    corpus = workloads.small_int_matrix(9_000, 256, config_id=8)
    qs = workloads.small_int_matrix(32, 256, config_id=8, stream=1)
    g_idx, g_sc = _search(eng, corpus, qs, 200)
    o_idx, o_sc = oracle.search(corpus, qs, 200)
    assert np.array_equal(g_idx, o_idx)
    assert np.array_equal(g_sc.astype(np.float64), o_sc)


@pytest.mark.parametrize("n,k", [(20_000, 1024), (100_000, 129), (70_000, 700), (200_000, 64)])
def test_batched_large_k_all_equal_scores(eng, n, k):
    """Every score equal: every tile maximum reaches the bound, so the kept
    scores (and, for n > 131072, the tile list) overflow LDS and the exact
    whole-row selection must return indices 0..k-1."""
    d = 64
    corpus = np.zeros((n, d), np.float32)
    corpus[:, 0] = 1.0
    qs = np.zeros((4, d), np.float32)
    qs[:, 0] = np.array([0.5, 0.25, 2.0, 1.0], np.float32)
    g_idx, g_sc = _search(eng, corpus, qs, k)
    for qi in range(4):
        assert list(g_idx[qi]) == list(range(k)), qi
        assert np.all(g_sc[qi] == qs[qi, 0])


def test_batched_large_k_ties_and_tail(eng):
    """Exact integer ties crowding the k-th score, then ordinary Gaussian rows on
    the next call."""
    corpus = workloads.small_int_matrix(30_000, 32, lo=-1, hi=1, config_id=9)
    qs = workloads.small_int_matrix(8, 32, lo=-1, hi=1, config_id=9, stream=1)
    for k in (1024, 300):
        g_idx, g_sc = _search(eng, corpus, qs, k)
        o_idx, o_sc = oracle.search(corpus, qs, k)
        assert np.array_equal(g_idx, o_idx), k
        assert np.array_equal(g_sc.astype(np.float64), o_sc), k
    gauss = workloads.gaussian_rows(50_000, 256, config_id=10)
    gq = workloads.gaussian_rows(8, 256, config_id=10, stream=1)
    _check_against_oracle(eng, gauss, gq, 500)


def test_batched_fewer_tiles_than_k(eng):
    """n = 1000 rows make 32 tiles, fewer than k: no tile bound, every score kept."""
    corpus = workloads.gaussian_rows(1_000, 256, config_id=21)
    qs = workloads.gaussian_rows(5, 256, config_id=21, stream=1)
    for k in (100, 1000):
        _check_against_oracle(eng, corpus, qs, k)


def test_batched_outlier_tile(eng):
    """One row far above the rest puts the largest tile maximum more than an
    octave above the k-th, outside the first histogram window: the bound comes
    from the two plain digit passes instead."""
    corpus = workloads.gaussian_rows(40_000, 128, config_id=22)
    corpus[12_345] *= 64.0
    qs = workloads.gaussian_rows(6, 128, config_id=22, stream=1)
    qs[:, :] = np.abs(qs)  # every query favours the scaled row's positive entries
    corpus[12_345] = np.abs(corpus[12_345])
    for k in (50, 700):
        g_idx, _, o_idx, _ = _check_against_oracle(eng, corpus, qs, k)
        assert np.all(g_idx[:, 0] == 12_345)


def test_batched_ragged_last_tile(eng):
    """The best rows sit in the last, partial tile (n = 32 m + 7): its maximum
    must cover only rows below n."""
    n = 32 * 900 + 7
    corpus = workloads.gaussian_rows(n, 256, config_id=23)
    qs = workloads.gaussian_rows(4, 256, config_id=23, stream=1)
    for qi in range(4):
        corpus[n - 1 - qi] = qs[qi] * np.float32(3.0)
    for k in (1, 10, 130):
        g_idx, _, _, _ = _check_against_oracle(eng, corpus, qs, k)
        assert np.all(g_idx[:, 0] == np.array([n - 1, n - 2, n - 3, n - 4]))


def _same(a, b):
    return np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


def test_deterministic_repeat(eng):
    """Repeated searches give the same indices and score bits: the batch (MFMA
    scorer + tile-bounded selection) and each single query (streaming kernel,
    per-wave lists and the cross-workgroup merge tree, whose arrival order
    varies from call to call)."""
    corpus = workloads.gaussian_rows(60_000, 768, config_id=12)
    qs = workloads.gaussian_rows(4, 768, config_id=12, stream=1)
    a = _search(eng, corpus, qs, 100)
    b = _search(eng, corpus, qs, 100)
    assert _same(a, b), "batched search not deterministic"
    for qi in range(4):
        q1 = torch.from_numpy(qs[qi:qi + 1]).cuda()
        first = None
        for rep in range(10):
            idx, sc = eng.search_resident(q1, 100)
            torch.cuda.synchronize()
            cur = (idx.cpu().numpy(), sc.cpu().numpy())
            if first is None:
                first = cur
            assert _same(first, cur), f"single query {qi} differs on repeat {rep}"


def test_stream_argument(eng):
    corpus = workloads.gaussian_rows(8_000, 384, config_id=13)
    q = workloads.gaussian_rows(1, 384, config_id=13, stream=1)
    eng.upload_corpus_rowmajor(corpus)
    s = torch.cuda.Stream()
    qd = torch.from_numpy(q).cuda()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        idx, sc = eng.search_resident(qd, 8, stream=s)
    s.synchronize()
    o_idx, o_sc = oracle.search(corpus, q, 8)
    check_retrieval(idx.cpu().numpy()[0], sc.cpu().numpy()[0], o_idx[0], o_sc[0], corpus, q[0], oracle)


# ---------------------------------------------------------------- raw top-K

def _select(eng, values, k, offset=0):
    buf = torch.from_numpy(np.ascontiguousarray(values)).cuda()
    view = buf[offset:]
    idx, vals = eng.topk_select(view, k)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), vals.cpu().numpy()


@pytest.mark.parametrize("n,k", [(1, 1), (2, 2), (5, 3), (63, 20), (64, 64), (65, 50), (1_000, 1_000),
                                 (100_003, 20), (1_000_000, 50), (3_000_000, 1024), (777_777, 129)])
def test_topk_int32_matches_oracle(eng, n, k):
    v = workloads.int32_values(n=n, config_id=40 + k % 7)
    g_idx, g_val = _select(eng, v, k)
    o_idx, o_val = oracle.topk(v, k)
    assert np.array_equal(g_idx, o_idx)
    assert np.array_equal(g_val, o_val)


@pytest.mark.parametrize("offset", [1, 2, 3, 5])
def test_topk_int32_misaligned_views(eng, offset):
    v = workloads.int32_values(n=500_000 + offset, config_id=41)
    g_idx, g_val = _select(eng, v, 50, offset=offset)
    o_idx, o_val = oracle.topk(v[offset:], 50)
    assert np.array_equal(g_idx, o_idx)
    assert np.array_equal(g_val, o_val)


def test_topk_int32_special_arrays(eng):
    n = 300_000
    cases = {
        "all_equal": np.full(n, 7, dtype=np.int32),
        "int_min": np.full(n, np.iinfo(np.int32).min, dtype=np.int32),
        "int_max": np.full(n, np.iinfo(np.int32).max, dtype=np.int32),
        "descending": np.arange(n, 0, -1).astype(np.int32),
        "ascending": np.arange(n).astype(np.int32),
        "periodic": (np.arange(n) % 1000).astype(np.int32),
        "two_values": np.where(np.arange(n) % 3 == 0, -1, 1).astype(np.int32),
    }
    for name, v in cases.items():
        for k in (1, 50, 1024):
            g_idx, g_val = _select(eng, v, k)
            o_idx, o_val = oracle.topk(v, k)
            assert np.array_equal(g_idx, o_idx), (name, k)
            assert np.array_equal(g_val, o_val), (name, k)


def test_topk_int32_boundary_ties(eng):
    """Copies of the top-(k+5) values scattered to random positions make the k-th
    boundary an exact tie that only the index can break."""
    rng = np.random.default_rng(5)
    for k in (20, 50):
        v = workloads.int32_values(n=2_000_000, config_id=42)
        top = np.sort(v)[::-1][:k + 5]
        v[rng.choice(v.size, 3 * (k + 5), replace=False)] = np.repeat(top, 3)
        g_idx, g_val = _select(eng, v, k)
        o_idx, o_val = oracle.topk(v, k)
        assert np.array_equal(g_idx, o_idx)
        assert np.array_equal(g_val, o_val)


def test_topk_arrival_tree(eng):
    """Arrays long enough for more workgroups than one merge node takes (256
    workgroups at 5M elements against 128 lists per node for k <= 32 and 64
    for k <= 64), where raw-array selection groups the workgroups by arrival
    order and merges nodes by binned selection.  The cases reach both of the
    binned merge's ends: few candidates (random values), and more than one
    wave can sort (heavy ties, a sorted array whose answer sits in the last
    workgroup), which falls back to pairwise merging."""
    n = 5_000_000
    rng = np.random.default_rng(8)
    cases = {
        "random": workloads.int32_values(n=n, config_id=43),
        "three_values": rng.integers(0, 3, size=n, dtype=np.int32),
        "thousand_values": rng.integers(0, 1000, size=n, dtype=np.int32),
        "ascending": np.arange(n, dtype=np.int32),
        "descending": np.arange(n, 0, -1).astype(np.int32),
    }
    for name, v in cases.items():
        for k in ((20, 32, 33, 50, 64) if name == "random" else (20, 50)):
            o_idx, o_val = oracle.topk(v, k)
            for rep in range(2):  # the second call checks the counters were left at zero
                g_idx, g_val = _select(eng, v, k)
                assert np.array_equal(g_idx, o_idx), (name, k, rep)
                assert np.array_equal(g_val, o_val), (name, k, rep)
    f = rng.standard_normal(n).astype(np.float32)
    for k in (20, 64):
        g_idx, g_val = _select(eng, f, k)
        o_idx, o_val = oracle.topk(f, k)
        assert np.array_equal(g_idx, o_idx), k
        assert np.array_equal(g_val.view(np.uint32), o_val.view(np.uint32)), k


@pytest.mark.parametrize("case", range(16))
def test_topk_tree_boundaries(eng, case):
    """Sizes around the merge tree's shape changes for raw arrays: a workgroup
    streams about 16k elements, a node merges 64 lists for 32 < k <= 64 and
    128 for 16 < k <= 32, and past one node the workgroups are grouped by
    arrival order -- so 1.05M and 2.1M elements are the boundaries, and 4.2M
    reaches the 256-workgroup cap.  Each case draws its size around a
    boundary, a k on either side of 32, a dtype, a value distribution (with
    ties that overflow the binned merge's 64-entry sort) and a misaligned
    start, and must match the oracle bit for bit."""
    rng = np.random.default_rng(1000 + case)
    base = [1_048_576, 2_097_152, 4_194_304, 1_200_000][case % 4]
    n = int(base + rng.integers(-70_000, 70_000))
    k = int(rng.choice([17, 20, 32, 33, 50, 64]))
    offset = int(rng.integers(0, 4))
    dist = case // 4  # 0 uniform, 1 few values, 2 sorted, 3 fp32 Gaussian with duplicates
    if dist == 0:
        v = rng.integers(-(2 ** 31), 2 ** 31, size=n + offset, dtype=np.int64).astype(np.int32)
    elif dist == 1:
        v = rng.integers(0, 5, size=n + offset, dtype=np.int32)
    elif dist == 2:
        v = np.sort(rng.integers(-(2 ** 31), 2 ** 31, size=n + offset, dtype=np.int64)).astype(np.int32)
    else:
        v = rng.standard_normal(n + offset).astype(np.float32)
        v[rng.choice(v.size, 5000, replace=False)] = v[rng.choice(v.size, 5000, replace=False)]
    print(f"[tree boundary] case {case}: n={n} k={k} offset={offset} dist={dist} dtype={v.dtype}", flush=True)
    g_idx, g_val = _select(eng, v, k, offset=offset)
    o_idx, o_val = oracle.topk(v[offset:], k)
    assert np.array_equal(g_idx, o_idx), (case, n, k, offset, dist)
    assert np.array_equal(g_val.view(np.uint32), o_val.view(np.uint32)), (case, n, k, offset, dist)


def test_topk_float32_special_values(eng):
    rng = np.random.default_rng(6)
    v = rng.standard_normal(400_000).astype(np.float32)
    specials = np.array([0.0, -0.0, np.inf, -np.inf, 1e-45, -1e-45, 3.4e38, -3.4e38], dtype=np.float32)
    v[rng.choice(v.size, 4000, replace=False)] = np.tile(specials, 500)
    v[rng.choice(v.size, 2000, replace=False)] = v[rng.choice(v.size, 2000, replace=False)]
    for k in (1, 17, 100, 1024):
        g_idx, g_val = _select(eng, v, k)
        o_idx, o_val = oracle.topk(v, k)
        assert np.array_equal(g_idx, o_idx), k
        assert np.array_equal(g_val.view(np.uint32), o_val.view(np.uint32)), k
    zeros = np.where(np.arange(1000) % 2 == 0, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
    g_idx, g_val = _select(eng, zeros, 10)
    assert list(g_idx) == list(range(10)), "-0.0 must tie +0.0 and fall to the index"
    assert np.array_equal(g_val.view(np.uint32), zeros[:10].view(np.uint32)), "value bits must be preserved"


def test_topk_float32_random(eng):
    v = workloads.float32_values(2_000_003)
    for k in (8, 100, 1000):
        g_idx, g_val = _select(eng, v, k)
        o_idx, o_val = oracle.topk(v, k)
        assert np.array_equal(g_idx, o_idx)
        assert np.array_equal(g_val.view(np.uint32), o_val.view(np.uint32))
        check_exact_topk_property(g_idx, g_val, v)


# ---------------------------------------------------------------- error paths

def test_error_paths():
    e = ResidentTopK(1000, 64, 32, 4, device=0)
    try:
        q = torch.zeros((1, 64), dtype=torch.float32, device="cuda")
        with pytest.raises(ResidentTopKError) as ei:
            e.search_resident(q, 8)  # nothing resident
        assert ei.value.status == 2
        with pytest.raises(ResidentTopKError) as ei:
            e.upload_corpus_rowmajor(np.zeros((1001, 64), np.float32))  # n > max_n
        assert ei.value.status == 1
        e.upload_corpus_rowmajor(np.ones((10, 64), np.float32))
        with pytest.raises(ResidentTopKError):
            e.search_resident(q, 33)  # k > max_k
        with pytest.raises(ResidentTopKError):
            e.search_resident(q, 11)  # k > n
        with pytest.raises(ResidentTopKError):
            e.search_resident(torch.zeros((5, 64), dtype=torch.float32, device="cuda"), 2)  # q > max_q
        idx, sc = e.search_resident(q, 10)  # k == n: a full sort of equal scores
        torch.cuda.synchronize()
        assert list(idx.cpu().numpy()[0]) == list(range(10))
    finally:
        e.close()
    with pytest.raises(ResidentTopKError):
        ResidentTopK(1 << 40, 64, 8, 1)  # beyond the int32 index range


def test_out_of_memory_paths():
    """RT_ENOMEM: limits that pass every check but whose allocation exceeds
    HBM.  rt_engine_create then returns no engine (and leaks nothing: a normal
    engine works afterwards); rt_enable_filtered on an engine whose fp32
    corpus fits but whose reduced-precision copies do not leaves that engine
    working for the plain search."""
    import ctypes
    from top_search_resident_amd import _lib
    lib = _lib.load()
    torch.cuda.empty_cache()
    h = ctypes.c_void_p(12345)
    st = lib.rt_engine_create(2 ** 31 - 1, 65536, 8, 1, 0, ctypes.byref(h))  # a 512 TiB corpus
    assert st == _lib.RT_ENOMEM, st
    assert h.value is None
    with pytest.raises(ResidentTopKError) as ei:
        ResidentTopK(2 ** 31 - 1, 65536, 8, 1)
    assert ei.value.status == _lib.RT_ENOMEM
    free_b, total_b = torch.cuda.mem_get_info()
    # a corpus of ~75% of the free memory: its bf16 copy (half of it) no longer fits
    d = 64
    max_n = min(2 ** 31 - 1, int(0.75 * free_b) // (4 * d))
    with ResidentTopK(max_n, d, 16, 1) as e:
        with pytest.raises(ResidentTopKError) as ei:
            e.enable_filtered()
        assert ei.value.status == _lib.RT_ENOMEM
        corpus = workloads.gaussian_rows(5_000, d, config_id=31)
        q = workloads.gaussian_rows(1, d, config_id=31, stream=1)
        e.upload_corpus_rowmajor(corpus)
        idx, sc = e.search_resident(torch.from_numpy(q).cuda(), 16)
        torch.cuda.synchronize()
        o_idx, o_sc = oracle.search(corpus, q, 16)
        check_retrieval(idx.cpu().numpy()[0], sc.cpu().numpy()[0], o_idx[0], o_sc[0], corpus, q[0], oracle)
        with pytest.raises(ResidentTopKError) as ei:
            e.search_resident_filtered(torch.from_numpy(q).cuda(), 16)  # the filtered search was never enabled
        assert ei.value.status == _lib.RT_ESTATE
    with ResidentTopK(1000, 64, 8, 1) as e:  # everything was released
        e.upload_corpus_rowmajor(np.ones((10, 64), np.float32))
        idx, _ = e.search_resident(torch.ones((1, 64), dtype=torch.float32, device="cuda"), 3)
        torch.cuda.synchronize()
        assert list(idx.cpu().numpy()[0]) == [0, 1, 2]


def test_binding_rejects_bad_buffers():
    """Checks the binding makes before anything is enqueued (the C ABI only sees
    addresses): query width against the resident depth, and output buffers that
    are host memory, non-contiguous, of the wrong dtype or too small."""
    with ResidentTopK(1000, 64, 32, 4, device=0) as e:
        e.upload_corpus_rowmajor(np.ones((100, 64), np.float32))
        q = torch.zeros((1, 64), dtype=torch.float32, device="cuda")
        with pytest.raises(ValueError, match="width"):
            e.search_resident(torch.zeros((1, 32), dtype=torch.float32, device="cuda"), 8)
        with pytest.raises(ValueError, match="width"):
            e.search_resident(torch.zeros((1, 65), dtype=torch.float32, device="cuda"), 8)
        with pytest.raises(TypeError, match="CUDA"):
            e.search_resident(q, 8, out_idx=torch.empty((1, 8), dtype=torch.int32))
        with pytest.raises(TypeError, match="CUDA"):
            e.search_resident(q, 8, out_scores=torch.empty((1, 8), dtype=torch.float32))
        with pytest.raises(TypeError, match="contiguous"):
            e.search_resident(q, 8, out_idx=torch.empty((8, 2), dtype=torch.int32, device="cuda").t())
        with pytest.raises(ValueError, match="needed"):
            e.search_resident(q, 8, out_scores=torch.empty(7, dtype=torch.float32, device="cuda"))
        with pytest.raises(TypeError, match="float32"):
            e.search_resident(q, 8, out_scores=torch.empty(8, dtype=torch.float64, device="cuda"))
        with pytest.raises(ResidentTopKError):
            e.search_resident(q, 0)
        v = torch.arange(100, dtype=torch.int32, device="cuda")
        with pytest.raises(TypeError, match="CUDA"):
            e.topk_select(v, 4, out_values=torch.empty(4, dtype=torch.int32))
        with pytest.raises(TypeError, match="int32"):
            e.topk_select(v, 4, out_values=torch.empty(4, dtype=torch.float32, device="cuda"))
        with pytest.raises(TypeError, match="contiguous"):
            e.topk_select(torch.arange(200, dtype=torch.int32, device="cuda")[::2], 4)
        # the engine still works after every refusal
        idx, _ = e.search_resident(q, 8)
        i2, v2 = e.topk_select(v, 4)
        torch.cuda.synchronize()
        assert list(idx.cpu().numpy()[0]) == list(range(8))
        assert list(i2.cpu().numpy()) == [99, 98, 97, 96]
        # a shared engine follows the resident depth of the corpus it shares
        with e.shared() as s2:
            with pytest.raises(ValueError, match="width"):
                s2.search_resident(torch.zeros((1, 32), dtype=torch.float32, device="cuda"), 8)
            e.upload_corpus_rowmajor(np.ones((50, 32), np.float32))
            s2.search_resident(torch.zeros((1, 32), dtype=torch.float32, device="cuda"), 8)
            torch.cuda.synchronize()


def test_read_probe(eng):
    """rt_read_probe times a plain read of the resident corpus; it rejects bad
    arguments, and the searches after it (it writes into the merge-tree
    scratch) still match the oracle."""
    corpus = workloads.gaussian_rows(150_000, 1024, config_id=13)
    qs = workloads.gaussian_rows(2, 1024, config_id=13, stream=1)
    eng.upload_corpus_rowmajor(corpus)
    ms = eng.read_probe(reps=5)
    nbytes = corpus.nbytes
    print(f"[read probe] {nbytes} B in {ms * 1e3:.1f} us", flush=True)
    assert 0.0 < ms < 50.0
    assert nbytes / (ms * 1e-3) < 8.5e12  # no faster than the HBM peak
    with pytest.raises(ResidentTopKError) as ei:
        eng.read_probe(reps=0)
    assert ei.value.status == 1
    _check_against_oracle(eng, corpus, qs, 64)
    with ResidentTopK(100, 8, 4, 1) as e:
        with pytest.raises(ResidentTopKError) as ei:
            e.read_probe()  # nothing resident
        assert ei.value.status == 2
