"""search_resident_filtered with the cosine metric: for each query the answer
must be the plain single-query cosine scan's bit for bit (indices, order and
score bits) and meet the oracle's acceptance rules, through the bf16 and the
fp8 first passes, at every depth they cover, k from 1 to n, rows of very
different lengths, zero rows and zero queries (-inf scores), scaled copies
that tie exactly, batches (one segment per query) and the plain fallback."""
import numpy as np
import pytest

import oracle
from gpu_util import check_retrieval
import workloads
from top_search_resident_amd import ResidentTopK

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

MAX_N, MAX_D, MAX_K, MAX_Q = 120_000, 2048, 1024, 4


@pytest.fixture(scope="module")
def eng():
    assert torch.cuda.is_available(), "a GPU is required for the parity tests"
    e = ResidentTopK(MAX_N, MAX_D, MAX_K, MAX_Q, device=0)
    e.enable_filtered()
    yield e
    e.close()


def _plain(eng, q, k):
    out_i, out_s = [], []
    for i in range(q.shape[0]):
        pi, ps = eng.search_resident(q[i:i + 1], k, metric="cosine")
        torch.cuda.synchronize()
        out_i.append(pi.cpu().numpy()[0])
        out_s.append(ps.cpu().numpy()[0])
    return np.stack(out_i), np.stack(out_s)


def _both(eng, corpus, queries, k, storage, path=None, upload=True):
    """The filtered cosine search (the whole batch at once) against the plain
    single-query cosine scans."""
    if upload:
        eng.upload_corpus_rowmajor(corpus)
    eng.set_filter_storage(storage)
    q = torch.from_numpy(np.ascontiguousarray(queries)).cuda()
    print(f"[filtered cosine] n={corpus.shape[0]} d={corpus.shape[1]} q={q.shape[0]} k={k} {storage}", flush=True)
    fi, fs = eng.search_resident_filtered(q, k, metric="cosine")
    torch.cuda.synchronize()
    assert eng.filter_path_used() == (path or storage)
    b_idx, b_sc = fi.cpu().numpy(), fs.cpu().numpy()
    a_idx, a_sc = _plain(eng, q, k)
    assert np.array_equal(a_idx, b_idx), (a_idx[:, :8], b_idx[:, :8])
    assert np.array_equal(a_sc.view(np.uint32), b_sc.view(np.uint32))
    return b_idx, b_sc


def _with_oracle(eng, corpus, queries, k, storage):
    g_idx, g_sc = _both(eng, corpus, queries, k, storage)
    o_idx, o_sc = oracle.search(corpus, queries, k, metric=1)
    for qi in range(queries.shape[0]):
        check_retrieval(g_idx[qi], g_sc[qi], o_idx[qi], o_sc[qi], corpus, queries[qi], oracle, metric="cosine")
    return g_idx, g_sc, o_idx, o_sc


@pytest.mark.parametrize("storage", ["bf16", "fp8"])
@pytest.mark.parametrize("n,d,k,q", [
    (100_000, 1024, 8, 1), (100_000, 1024, 100, 2), (50_000, 768, 32, 3), (12_345, 384, 64, 1),
    (7_001, 256, 1, 2), (4_099, 1536, 129, 1), (2_050, 2048, 1024, 1), (65, 512, 65, 4),
])
def test_filtered_cosine_equals_plain(eng, storage, n, d, k, q):
    corpus = workloads.scaled_rows(n, d, config_id=900 + d % 97, sigma=1.0)
    qs = workloads.gaussian_rows(q, d, config_id=900 + d % 97, stream=1, normalise=False) * np.float32(3.0)
    _with_oracle(eng, corpus, qs, k, storage)


@pytest.mark.parametrize("storage", ["bf16", "fp8"])
def test_filtered_cosine_zero_rows_and_zero_query(eng, storage):
    """Zero rows score -inf; with k above the number of non-zero rows the tail is
    the lowest-index zero rows.  A zero query scores every row -inf."""
    n, d = 3_000, 256
    corpus = workloads.scaled_rows(n, d, config_id=930)
    zero = np.random.default_rng(93).choice(n, 2_990, replace=False)
    corpus[zero] = 0.0
    qs = workloads.gaussian_rows(2, d, config_id=930, stream=1)
    g_idx, g_sc, o_idx, _ = _with_oracle(eng, corpus, qs, 20, storage)
    assert np.array_equal(g_idx, o_idx)
    assert np.all(np.isneginf(g_sc[:, 10:]))
    zq = qs.copy()
    zq[0] = 0.0
    g_idx, g_sc = _both(eng, corpus, zq, 20, storage, upload=False)
    assert list(g_idx[0]) == list(range(20))
    assert np.all(np.isneginf(g_sc[0]))


@pytest.mark.parametrize("storage", ["bf16", "fp8"])
def test_filtered_cosine_scaled_copies_tie_by_index(eng, storage):
    n, d = 40_000, 768
    corpus = workloads.gaussian_rows(n, d, config_id=940)
    qs = workloads.gaussian_rows(1, d, config_id=940, stream=1)
    best = int(np.argmax(corpus.astype(np.float64) @ qs[0].astype(np.float64)))
    corpus[best] = qs[0] + np.float32(0.5) * corpus[best]
    pos = np.random.default_rng(94).choice(n, 12, replace=False)
    for j, p in enumerate(pos):
        corpus[p] = corpus[best] * np.float32(2.0 ** (j % 7 - 3))
    g_idx, g_sc, o_idx, _ = _with_oracle(eng, corpus, qs, 32, storage)
    copies = sorted(set(pos.tolist()) | {best})
    assert list(g_idx[0, :len(copies)]) == copies
    assert list(o_idx[0, :len(copies)]) == copies


def test_filtered_cosine_planted_near_ties(eng):
    corpus, qs = workloads.retrieval_inputs("c2_100k_768", queries=3)
    for storage in ("bf16", "fp8"):
        _with_oracle(eng, corpus, qs, 32, storage)


@pytest.mark.parametrize("metric", ["dot", "cosine"])
def test_plain_fallback_is_the_single_query_scan(eng, metric):
    """A depth the filtered passes do not cover (d % 8 != 0) runs the plain scan
    one query at a time: each answer is the single-query scan's, also in a
    batch."""
    corpus = workloads.gaussian_rows(20_000, 100, config_id=950)
    qs = workloads.gaussian_rows(3, 100, config_id=950, stream=1)
    eng.upload_corpus_rowmajor(corpus)
    q = torch.from_numpy(qs).cuda()
    fi, fs = eng.search_resident_filtered(q, 50, metric=metric)
    torch.cuda.synchronize()
    assert eng.filter_path_used() == "plain"
    for i in range(3):
        pi, ps = eng.search_resident(q[i:i + 1], 50, metric=metric)
        torch.cuda.synchronize()
        assert np.array_equal(fi.cpu().numpy()[i], pi.cpu().numpy()[0])
        assert np.array_equal(fs.cpu().numpy()[i].view(np.uint32), ps.cpu().numpy()[0].view(np.uint32))


def test_bad_metric(eng):
    q = torch.zeros((1, 256), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        eng.search_resident_filtered(q, 4, metric="l2")


def test_filtered_cosine_batch_long_wave_ranges():
    """A cosine batch of 32 queries over 200,000 rows of depth 256 takes the
    single-query passes with one segment per query.  On a 256-CU part that is
    64 waves per query of 3,125 rows each, so the fp8 pass writes each wave's
    bounds in two bursts (its LDS gather holds 2,048 rows)."""
    n, d, k, q = 200_000, 256, 10, 32
    e = ResidentTopK(n, d, 64, q, device=0)
    try:
        e.enable_filtered()
        corpus = workloads.gaussian_rows(n, d, config_id=931)
        qs = workloads.gaussian_rows(q, d, config_id=931, stream=1)
        g_idx, g_sc = _both(e, corpus, qs, k, "fp8")
        o_idx, o_sc = oracle.search(corpus, qs[:3], k, metric=1)
        for qi in range(3):
            check_retrieval(g_idx[qi], g_sc[qi], o_idx[qi], o_sc[qi], corpus, qs[qi], oracle, metric="cosine")
    finally:
        e.close()
