"""The batched path of search_resident_filtered: q > 1 queries on an engine with
batch buffers and a depth of 256, 384, 512, 768 or 1024 take one bf16
matrix-core pass for all queries (bounds from the row norms and the query
split into two bf16 parts), per-query thresholds from the maxima of the lower
bounds over 32-row tiles, and the fp32 re-rank of the rows that reach them.
Each query's answer must be the plain single-query scan's answer bit for bit
(indices, order and score bits) and meet the oracle acceptance rules.  Cases:
every compile-time depth, batches of 2 to 32 queries, k from 1 to n, fewer
tiles than k (no threshold: every row re-ranked), a ragged last tile, planted
near-ties, exact integer ties, zero and huge queries, a smaller batch after a
larger one on the same buffers, k above 256 (per-query candidate lists),
lists longer than the in-LDS sort, and a depth that falls back to the
per-query first pass."""
import numpy as np
import pytest

import oracle
from gpu_util import check_retrieval
import workloads
from top_search_resident_amd import ResidentTopK

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

MAX_N, MAX_D, MAX_K, MAX_Q = 120_000, 1024, 1024, 32


@pytest.fixture(scope="module")
def eng():
    assert torch.cuda.is_available(), "a GPU is required for the parity tests"
    e = ResidentTopK(MAX_N, MAX_D, MAX_K, MAX_Q, device=0)
    e.enable_filtered()
    yield e
    e.close()


def _both(eng, corpus, queries, k, upload=True):
    """The filtered batch against the plain single-query search of each query."""
    if upload:
        eng.upload_corpus_rowmajor(corpus)
    q = torch.from_numpy(np.ascontiguousarray(queries)).cuda()
    print(f"[filtered batch] n={corpus.shape[0]} d={corpus.shape[1]} q={q.shape[0]} k={k}", flush=True)
    b_idx, b_sc = eng.search_resident_filtered(q, k)
    plain = [eng.search_resident(q[i:i + 1], k) for i in range(q.shape[0])]
    torch.cuda.synchronize()
    a_idx = np.concatenate([p[0].cpu().numpy() for p in plain])
    a_sc = np.concatenate([p[1].cpu().numpy() for p in plain])
    b_idx, b_sc = b_idx.cpu().numpy(), b_sc.cpu().numpy()
    assert np.array_equal(a_idx, b_idx), (a_idx[:, :8], b_idx[:, :8])
    assert np.array_equal(a_sc.view(np.uint32), b_sc.view(np.uint32))
    return b_idx, b_sc


def _with_oracle(eng, corpus, queries, k, check=None):
    g_idx, g_sc = _both(eng, corpus, queries, k)
    sel = range(queries.shape[0]) if check is None else check
    o_idx, o_sc = oracle.search(corpus, queries[list(sel)], k)
    for j, qi in enumerate(sel):
        check_retrieval(g_idx[qi], g_sc[qi], o_idx[j], o_sc[j], corpus, queries[qi], oracle)


@pytest.mark.parametrize("n,d,q,k", [
    (20_011, 768, 32, 100), (20_011, 1024, 32, 8), (40_000, 384, 17, 64), (30_000, 512, 8, 200),
    (9_000, 256, 32, 1024), (100_000, 768, 32, 32), (65, 768, 2, 65), (33, 512, 5, 5), (3_201, 1024, 32, 1),
    (20, 512, 3, 5), (31, 256, 32, 31), (1, 768, 4, 1), (1_000, 1024, 7, 40),
])
def test_batched_filtered_equals_plain(eng, n, d, q, k):
    corpus = workloads.gaussian_rows(n, d, config_id=700 + d % 97)
    qs = workloads.gaussian_rows(q, d, config_id=700 + d % 97, stream=1)
    _with_oracle(eng, corpus, qs, k, check=range(min(q, 6)))


def test_batched_filtered_planted_near_ties(eng):
    corpus, qs = workloads.retrieval_inputs("c2_100k_768", queries=32)
    for k in (8, 32):
        _with_oracle(eng, corpus, qs, k, check=range(4))


def test_batched_filtered_unnormalised(eng):
    corpus = workloads.scaled_rows(50_000, 1024, config_id=711, sigma=2.0)
    qs = workloads.gaussian_rows(12, 1024, config_id=711, stream=1, normalise=False)
    qs *= np.exp(np.linspace(-6.0, 6.0, 12)).astype(np.float32)[:, None]
    _with_oracle(eng, corpus, qs, 40, check=(0, 5, 11))


def test_batched_filtered_integer_ties(eng):
    """Exact integer scores (entries in [-1, 1]): wide bounds against the score
    spacing, dense ties at the k-th score; the answer is the oracle's exactly."""
    corpus = workloads.small_int_matrix(30_000, 256, lo=-1, hi=1, config_id=712)
    qs = workloads.small_int_matrix(32, 256, lo=-1, hi=1, config_id=712, stream=1)
    for k in (50, 700):
        g_idx, g_sc = _both(eng, corpus, qs, k)
        o_idx, o_sc = oracle.search(corpus, qs, k)
        assert np.array_equal(g_idx, o_idx), k
        assert np.array_equal(g_sc.astype(np.float64), o_sc), k


def test_batched_filtered_all_equal_rows(eng):
    """Every row the same: every bound interval overlaps T, so every row is
    re-ranked and ties go to the lower index."""
    corpus = np.tile(workloads.gaussian_rows(1, 512, config_id=713), (5_000, 1))
    qs = workloads.gaussian_rows(4, 512, config_id=713, stream=1)
    g_idx, _ = _both(eng, corpus, qs, 300)
    assert np.all(g_idx == np.arange(300)[None, :])


def test_batched_filtered_zero_and_huge_queries(eng):
    """A zero query (all scores 0, ties by index); a query whose element rounds
    to infinity in bf16 (its bounds are unknown, so every row is re-ranked); a
    query of values around 1e-30."""
    corpus = workloads.gaussian_rows(12_000, 768, config_id=714)
    qs = workloads.gaussian_rows(6, 768, config_id=714, stream=1)
    qs[1] = 0.0
    qs[3, 7] = np.float32(3.4e38)
    qs[4] *= np.float32(1e-30)
    g_idx, g_sc = _both(eng, corpus, qs, 20)
    assert np.array_equal(g_idx[1], np.arange(20))
    _with_oracle(eng, corpus, qs[[0, 2, 4, 5]], 20)


@pytest.mark.parametrize("k", [257, 512, 1024])
def test_batched_filtered_large_k(eng, k):
    """k above 256: the re-rank appends every row at or above T to a per-query
    list and sorts the list."""
    corpus = workloads.gaussian_rows(MAX_N, 768, config_id=717)
    qs = workloads.gaussian_rows(32, 768, config_id=717, stream=1)
    _with_oracle(eng, corpus, qs, k, check=(0, 31))


def test_batched_filtered_long_candidate_lists(eng):
    """More candidates than the in-LDS sort holds (8192): equal rows put all
    20000 rows at T, integer scores tie over 8192 rows at the top; the
    k-th largest candidate is found by a radix select over the list first."""
    corpus = np.tile(workloads.gaussian_rows(1, 512, config_id=718), (20_000, 1))
    qs = workloads.gaussian_rows(3, 512, config_id=718, stream=1)
    g_idx, _ = _both(eng, corpus, qs, 600)
    assert np.all(g_idx == np.arange(600)[None, :])
    corpus = workloads.small_int_matrix(MAX_N, 256, lo=-1, hi=1, config_id=719)
    qs = workloads.small_int_matrix(8, 256, lo=-1, hi=1, config_id=719, stream=1)
    qs[:, 2:] = 0  # scores in [-2, 2]: over 8192 rows tie at the top score
    g_idx, g_sc = _both(eng, corpus, qs, 1000)
    o_idx, o_sc = oracle.search(corpus, qs, 1000)
    assert np.array_equal(g_idx, o_idx)
    assert np.array_equal(g_sc.astype(np.float64), o_sc)


def test_batched_filtered_smaller_batch_after_larger(eng):
    corpus = workloads.gaussian_rows(60_000, 768, config_id=715)
    qs = workloads.gaussian_rows(32, 768, config_id=715, stream=1)
    _both(eng, corpus, qs, 100)
    _both(eng, corpus, qs[:3] * np.float32(-1.0), 10, upload=False)
    _both(eng, corpus, qs[5:7], 500, upload=False)


def test_batched_filtered_other_depth_falls_back(eng):
    """d = 640 has no matrix-core bound kernel: the per-query first pass runs."""
    corpus = workloads.gaussian_rows(8_000, 640, config_id=716)
    qs = workloads.gaussian_rows(4, 640, config_id=716, stream=1)
    _with_oracle(eng, corpus, qs, 10)
