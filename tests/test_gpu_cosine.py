"""Parity of the cosine metric (search_resident_metric with RT_METRIC_COSINE)
with the CPU oracle's cosine scores: rows of widely varying length so that the
cosine ranking differs from the inner product's, every scoring variant (vector
shapes, the scalar path, the MFMA batch kernels of compile-time and runtime
depth), zero rows and zero queries (score -inf), and scaled copies of a row
(equal cosines, ties by index)."""
import numpy as np
import pytest

import oracle
from gpu_util import check_retrieval
import workloads
from top_search_resident_amd import ResidentTopK

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

MAX_N, MAX_D, MAX_K, MAX_Q = 100_000, 3072, 1024, 32


@pytest.fixture(scope="module")
def eng():
    assert torch.cuda.is_available(), "a GPU is required for the parity tests"
    e = ResidentTopK(MAX_N, MAX_D, MAX_K, MAX_Q, device=0)
    yield e
    e.close()


def _search(eng, corpus, queries, k, metric="cosine"):
    eng.upload_corpus_rowmajor(corpus)
    q = torch.from_numpy(np.ascontiguousarray(queries)).cuda()
    idx, sc = eng.search_resident(q, k, metric=metric)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), sc.cpu().numpy()


def _check(eng, corpus, queries, k):
    g_idx, g_sc = _search(eng, corpus, queries, k)
    o_idx, o_sc = oracle.search(corpus, queries, k, metric=1)
    for qi in range(queries.shape[0]):
        check_retrieval(g_idx[qi], g_sc[qi], o_idx[qi], o_sc[qi], corpus, queries[qi], oracle, metric="cosine")
    return g_idx, g_sc, o_idx, o_sc


@pytest.mark.parametrize("n,d,k", [
    (12_345, 1024, 100), (7_001, 768, 32), (3_333, 128, 64), (5_000, 100, 40), (9_999, 4, 7),
    (4_099, 1536, 128), (2_050, 2048, 129), (3_001, 3000, 10), (1_000, 13, 5), (40_000, 384, 1024),
    (20_000, 64, 256), (1, 384, 1), (65, 768, 65),
])
def test_cosine_single_query(eng, n, d, k):
    corpus = workloads.scaled_rows(n, d, config_id=300 + d % 89)
    q = workloads.gaussian_rows(1, d, config_id=300 + d % 89, stream=1, normalise=False) * np.float32(2.5)
    _check(eng, corpus, q, k)


def test_cosine_ranking_differs_from_inner_product(eng):
    """On rows of varying length the two metrics pick different rows, and each
    GPU answer matches its own metric's oracle."""
    corpus = workloads.scaled_rows(30_000, 256, config_id=310)
    q = workloads.gaussian_rows(1, 256, config_id=310, stream=1)
    g_cos, _, _, _ = _check(eng, corpus, q, 50)
    g_dot, _ = _search(eng, corpus, q, 50, metric="dot")
    o_dot, _ = oracle.search(corpus, q, 50)
    assert np.array_equal(g_dot, o_dot)
    assert len(set(g_cos[0]) & set(g_dot[0])) < 40


@pytest.mark.parametrize("q,d,k", [(32, 768, 1024), (7, 1024, 8), (2, 256, 100), (32, 384, 64),
                                   (5, 100, 20), (3, 200, 300), (4, 2048, 16)])
def test_cosine_batched(eng, q, d, k):
    """Batches with d % 4 == 0 and d <= 1024 run the MFMA scorer (compile-time
    depths 256/384/768/1024, runtime depth 100/200); d = 2048 runs the vector
    path once per query."""
    n = 20_011
    corpus = workloads.scaled_rows(n, d, config_id=320 + d % 83)
    qs = workloads.scaled_rows(q, d, config_id=320 + d % 83, stream=1)
    _check(eng, corpus, qs, k)


@pytest.mark.parametrize("q", [1, 4])
def test_cosine_zero_rows_and_zero_query(eng, q):
    """Zero rows score -inf: with k above the number of non-zero rows the tail of
    the answer is the lowest-index zero rows.  A zero query scores every row
    -inf, so the answer is rows 0..k-1."""
    n, d = 3_000, 256
    corpus = workloads.scaled_rows(n, d, config_id=330)
    zero = np.random.default_rng(33).choice(n, 2_990, replace=False)
    corpus[zero] = 0.0
    qs = workloads.gaussian_rows(q, d, config_id=330, stream=1)
    k = 20
    g_idx, g_sc, o_idx, _ = _check(eng, corpus, qs, k)
    assert np.array_equal(g_idx, o_idx)
    assert np.all(np.isneginf(g_sc[:, 10:]))
    assert np.array_equal(g_idx[:, 10:], np.tile(np.sort(zero)[:10], (q, 1)))
    zq = np.zeros_like(qs)
    if q > 1:
        zq[1] = qs[1]  # a zero query next to a real one in the same batch
    g_idx, g_sc = _search(eng, corpus, zq, k)
    assert list(g_idx[0]) == list(range(k))
    assert np.all(np.isneginf(g_sc[0]))


@pytest.mark.parametrize("q", [1, 3])
def test_cosine_scaled_copies_tie_by_index(eng, q):
    """A row and its copies scaled by powers of two have bit-identical fp32
    cosines (the scaling is exact in the dot product, the norm and their
    quotient), so they tie and come back in index order, as in the oracle."""
    n, d = 40_000, 768
    corpus = workloads.gaussian_rows(n, d, config_id=340)
    qs = workloads.gaussian_rows(q, d, config_id=340, stream=1)
    best = int(np.argmax(corpus.astype(np.float64) @ qs[0].astype(np.float64)))
    corpus[best] = qs[0] + np.float32(0.5) * corpus[best]
    pos = np.random.default_rng(34).choice(n, 12, replace=False)
    for j, p in enumerate(pos):
        corpus[p] = corpus[best] * np.float32(2.0 ** (j % 7 - 3))
    g_idx, g_sc, o_idx, o_sc = _check(eng, corpus, qs, 32)
    copies = sorted(set(pos.tolist()) | {best})
    assert list(g_idx[0, :len(copies)]) == copies
    assert np.unique(g_sc[0, :len(copies)].view(np.uint32)).size == 1
    assert list(o_idx[0, :len(copies)]) == copies


def test_cosine_extreme_norms(eng):
    """Rows whose lengths span 1e-17 .. 1e17 (and queries of length 1e-10 and
    1e10): cosine is scale-invariant, so the ranking is that of the directions;
    every product stays a normal fp32 number, and the GPU matches the oracle's
    fp64 cosines for single queries and for a batch."""
    n, d = 20_000, 256
    rows = workloads.gaussian_rows(n, d, config_id=320)
    rng = np.random.default_rng(320)
    rows *= (10.0 ** rng.uniform(-17, 17, size=n)).astype(np.float32)[:, None]
    for qscale in (1e-10, 1.0, 1e10):
        q = workloads.gaussian_rows(3, d, config_id=320, stream=1) * np.float32(qscale)
        for qi in range(3):
            _check(eng, rows, q[qi:qi + 1], 50)
        _check(eng, rows, q, 50)  # a batch (matrix-core kernel)


def test_cosine_underflowing_norm_product_ranks_last(eng):
    """The documented range limit: the cosine's denominator is the fp32 product
    |q| |x|; for a row with |x| = 1e-30 and a query with |q| = 1e-20 it
    underflows to 0 and the row scores -inf like a zero row (below every
    finite cosine, ties by index), while rows of normal length rank by their
    cosines."""
    n, d, k = 1_000, 128, 1_000
    rows = workloads.gaussian_rows(n, d, config_id=321)
    tiny = np.arange(0, n, 7)
    rows[tiny] *= np.float32(1e-30)
    q = workloads.gaussian_rows(1, d, config_id=321, stream=1) * np.float32(1e-20)
    g_idx, g_sc = _search(eng, rows, q, k)
    ninf = np.isneginf(g_sc[0])
    assert ninf.sum() == tiny.size
    assert np.array_equal(np.sort(g_idx[0][ninf]), tiny) and np.all(np.diff(g_idx[0][ninf]) > 0)
    assert not np.isinf(g_sc[0][:k - tiny.size]).any()
    normal = np.setdiff1d(np.arange(n), tiny)
    o_idx, o_sc = oracle.search(rows[normal], q, k - tiny.size, metric=1)
    check_retrieval(g_idx[0][:k - tiny.size], g_sc[0][:k - tiny.size], normal[o_idx[0]], o_sc[0],
                    rows, q[0], oracle, metric="cosine")
