"""The fp8 first pass of search_resident_filtered (set_filter_storage("fp8")):
rows stored as e4m3 codes with a power-of-two scale per row, a certified bound
from each row's stored rounding error, and the fp32 re-rank of the rows that
reach the threshold.  The answer must be the plain single-query scan's bit for
bit (indices, order and score bits) and meet the oracle acceptance rules, on
every depth the pass covers, k from 1 to n, planted near-ties, exact integer
ties (exact in e4m3 after scaling), all-equal rows, zero rows and queries,
rows of very different lengths, huge and tiny values, and a corpus with a
value that is not finite (the plain scan runs)."""
import numpy as np
import pytest

import oracle
from gpu_util import check_retrieval
import workloads
from top_search_resident_amd import ResidentTopK

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

MAX_N, MAX_D, MAX_K, MAX_Q = 120_000, 2048, 1024, 1


@pytest.fixture(scope="module")
def eng():
    assert torch.cuda.is_available(), "a GPU is required for the parity tests"
    e = ResidentTopK(MAX_N, MAX_D, MAX_K, MAX_Q, device=0)
    e.enable_filtered()
    e.set_filter_storage("fp8")
    yield e
    e.close()


def _both(eng, corpus, queries, k, upload=True, path="fp8"):
    """The filtered search against the plain search, query by query."""
    if upload:
        eng.upload_corpus_rowmajor(corpus)
    q = torch.from_numpy(np.ascontiguousarray(queries)).cuda()
    print(f"[filtered fp8] n={corpus.shape[0]} d={corpus.shape[1]} q={q.shape[0]} k={k}", flush=True)
    b_idx, b_sc, a_idx, a_sc = [], [], [], []
    for i in range(q.shape[0]):
        fi, fs = eng.search_resident_filtered(q[i:i + 1], k)
        torch.cuda.synchronize()
        assert eng.filter_path_used() == path
        pi, ps = eng.search_resident(q[i:i + 1], k)
        torch.cuda.synchronize()
        b_idx.append(fi.cpu().numpy()[0]), b_sc.append(fs.cpu().numpy()[0])
        a_idx.append(pi.cpu().numpy()[0]), a_sc.append(ps.cpu().numpy()[0])
    a_idx, a_sc, b_idx, b_sc = map(np.stack, (a_idx, a_sc, b_idx, b_sc))
    assert np.array_equal(a_idx, b_idx), (a_idx[:, :8], b_idx[:, :8])
    assert np.array_equal(a_sc.view(np.uint32), b_sc.view(np.uint32))
    return b_idx, b_sc


def _with_oracle(eng, corpus, queries, k):
    g_idx, g_sc = _both(eng, corpus, queries, k)
    o_idx, o_sc = oracle.search(corpus, queries, k)
    for qi in range(queries.shape[0]):
        check_retrieval(g_idx[qi], g_sc[qi], o_idx[qi], o_sc[qi], corpus, queries[qi], oracle)


@pytest.mark.parametrize("n,d,k", [
    (100_000, 1024, 8), (100_000, 1024, 100), (50_000, 768, 32), (12_345, 384, 64), (7_001, 256, 1),
    (4_099, 1536, 129), (2_050, 2048, 1024), (30_000, 512, 256), (65, 768, 65), (1, 512, 1),
])
def test_fp8_filtered_equals_plain(eng, n, d, k):
    corpus = workloads.gaussian_rows(n, d, config_id=800 + d % 89)
    q = workloads.gaussian_rows(2, d, config_id=800 + d % 89, stream=1)
    _with_oracle(eng, corpus, q, k)


def test_fp8_planted_near_ties(eng):
    corpus, qs = workloads.retrieval_inputs("c2_100k_768", queries=3)
    for k in (8, 32):
        _with_oracle(eng, corpus, qs, k)


def test_fp8_rows_of_different_lengths(eng):
    corpus = workloads.scaled_rows(60_000, 1024, config_id=810, sigma=2.0)
    q = workloads.gaussian_rows(2, 1024, config_id=810, stream=1, normalise=False) * np.float32(7.0)
    _with_oracle(eng, corpus, q, 50)


def test_fp8_integer_ties_and_all_equal(eng):
    """Small integers are exact in e4m3 after scaling (zero rounding error), so
    the bounds are the summation terms only; ties crowd the k-th score."""
    corpus = workloads.small_int_matrix(40_000, 512, config_id=811)
    q = workloads.small_int_matrix(2, 512, config_id=811, stream=1)
    for k in (100, 1000):
        g_idx, g_sc = _both(eng, corpus, q, k)
        o_idx, o_sc = oracle.search(corpus, q, k)
        assert np.array_equal(g_idx, o_idx)
        assert np.array_equal(g_sc.astype(np.float64), o_sc)
    same = np.tile(workloads.gaussian_rows(1, 768, config_id=812), (3_000, 1))
    g_idx, _ = _both(eng, same, workloads.gaussian_rows(1, 768, config_id=812, stream=1), 200)
    assert np.array_equal(g_idx[0], np.arange(200))


def test_fp8_zero_rows_and_query(eng):
    corpus = workloads.gaussian_rows(9_000, 256, config_id=813)
    corpus[::7] = 0.0
    q = workloads.gaussian_rows(2, 256, config_id=813, stream=1)
    q[1] = 0.0
    g_idx, _ = _both(eng, corpus, q, 30)
    assert np.array_equal(g_idx[1], np.arange(30))


def test_fp8_huge_and_tiny_values(eng):
    """Rows scaled by 1e30 and by 1e-38 (the scale stops at 2^-126, so small
    codes become e4m3 subnormals or zero: the stored error covers them), and
    rows with a few huge entries next to small ones."""
    corpus = workloads.gaussian_rows(20_000, 768, config_id=814, normalise=False)
    corpus[:5_000] *= np.float32(1e30)
    corpus[5_000:10_000] *= np.float32(1e-38)
    corpus[10_000:12_000, :3] *= np.float32(1e6)
    q = workloads.gaussian_rows(2, 768, config_id=814, stream=1)
    _both(eng, corpus, q, 40)
    _with_oracle(eng, corpus[10_000:], q, 40)


def test_fp8_nonfinite_corpus_runs_the_plain_scan(eng):
    corpus = workloads.gaussian_rows(5_000, 512, config_id=815)
    corpus[17, 3] = np.float32(np.inf)
    q = workloads.gaussian_rows(1, 512, config_id=815, stream=1)
    _both(eng, corpus, q, 10, path="plain")


def test_storage_choice():
    """"auto" runs the plain scan for one query over a small corpus, "bf16" and
    "fp8" force their passes; a depth without an fp8 pass falls back to bf16;
    unknown names are rejected."""
    with ResidentTopK(4_000, 640, 64, 1) as e:
        e.enable_filtered()
        corpus = workloads.gaussian_rows(4_000, 512, config_id=816)
        q = workloads.gaussian_rows(1, 512, config_id=816, stream=1)
        e.upload_corpus_rowmajor(corpus)
        qd = torch.from_numpy(q).cuda()
        assert e.filter_path_used() is None
        e.search_resident_filtered(qd, 5)
        torch.cuda.synchronize()
        assert e.filter_path_used() == "plain"
        e.set_filter_storage("fp8")
        e.search_resident_filtered(qd, 5)
        torch.cuda.synchronize()
        assert e.filter_path_used() == "fp8"
        e.set_filter_storage("bf16")
        e.search_resident_filtered(qd, 5)
        torch.cuda.synchronize()
        assert e.filter_path_used() == "bf16"
        e.set_filter_storage("fp8")
        e.upload_corpus_rowmajor(workloads.gaussian_rows(4_000, 640, config_id=816))
        e.search_resident_filtered(torch.from_numpy(workloads.gaussian_rows(1, 640, config_id=816, stream=1)).cuda(), 5)
        torch.cuda.synchronize()
        assert e.filter_path_used() == "bf16"
        with pytest.raises(ValueError):
            e.set_filter_storage("fp4")
