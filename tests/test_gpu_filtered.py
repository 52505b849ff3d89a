"""The bf16-filtered exact search (search_resident_filtered): its answer must be
the plain fp32 search's answer bit for bit (indices, order and scores) and meet
the oracle acceptance rules, on shapes that exercise every lane-group layout of
both passes, on inputs where many rows crowd the k-th score (planted near-ties,
exact integer ties, all-equal rows, where the second pass has to re-score many
or all rows), on zero rows and queries, on batches, on engines sharing a
corpus, and on a corpus with values that overflow bf16 (plain-scan fallback), and the default
storage choice, which runs the plain scan for one query over a small corpus."""
import numpy as np
import pytest

import oracle
from gpu_util import check_retrieval
import workloads
from top_search_resident_amd import ResidentTopK

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

MAX_N, MAX_D, MAX_K, MAX_Q = 120_000, 2048, 1024, 8


@pytest.fixture(scope="module")
def eng():
    assert torch.cuda.is_available(), "a GPU is required for the parity tests"
    e = ResidentTopK(MAX_N, MAX_D, MAX_K, MAX_Q, device=0)
    e.enable_filtered()
    e.set_filter_storage("bf16")  # the default would run the plain scan for a single query on these sizes
    yield e
    e.close()


def _both(eng, corpus, queries, k, upload=True):
    """Filtered answers for all queries at once, checked against the plain
    single-query search of each query (the fp32 streaming scan; a plain batch
    would take the MFMA path, whose fp32 sums are ordered differently)."""
    if upload:
        eng.upload_corpus_rowmajor(corpus)
    q = torch.from_numpy(np.ascontiguousarray(queries)).cuda()
    b_idx, b_sc = eng.search_resident_filtered(q, k)
    plain = [eng.search_resident(q[i:i + 1], k) for i in range(q.shape[0])]
    torch.cuda.synchronize()
    a_idx = np.concatenate([p[0].cpu().numpy() for p in plain])
    a_sc = np.concatenate([p[1].cpu().numpy() for p in plain])
    b_idx, b_sc = b_idx.cpu().numpy(), b_sc.cpu().numpy()
    assert np.array_equal(a_idx, b_idx), (a_idx[:, :8], b_idx[:, :8])
    assert np.array_equal(a_sc.view(np.uint32), b_sc.view(np.uint32))
    return b_idx, b_sc


def _with_oracle(eng, corpus, queries, k):
    g_idx, g_sc = _both(eng, corpus, queries, k)
    o_idx, o_sc = oracle.search(corpus, queries, k)
    for qi in range(queries.shape[0]):
        check_retrieval(g_idx[qi], g_sc[qi], o_idx[qi], o_sc[qi], corpus, queries[qi], oracle)


@pytest.mark.parametrize("n,d,k", [
    (100_000, 1024, 8), (100_000, 1024, 100), (50_000, 768, 32), (12_345, 384, 64), (7_001, 128, 1),
    (9_999, 8, 5), (4_099, 1536, 129), (2_050, 2048, 1024), (30_000, 96, 256), (65, 768, 65), (1, 64, 1),
    (20_000, 40, 7), (5_000, 264, 17),
])
def test_filtered_equals_plain(eng, n, d, k):
    corpus = workloads.gaussian_rows(n, d, config_id=500 + d % 91)
    q = workloads.gaussian_rows(1, d, config_id=500 + d % 91, stream=1)
    _with_oracle(eng, corpus, q, k)


def test_filtered_unnormalised_rows(eng):
    corpus = workloads.scaled_rows(60_000, 512, config_id=510, sigma=2.0)
    q = workloads.gaussian_rows(2, 512, config_id=510, stream=1, normalise=False) * np.float32(7.0)
    _with_oracle(eng, corpus, q, 50)


def test_filtered_planted_near_ties(eng):
    corpus, qs = workloads.retrieval_inputs("c2_100k_768", queries=5)
    for k in (8, 32):
        _with_oracle(eng, corpus, qs, k)


def test_filtered_integer_ties_and_all_equal(eng):
    """Exact integer scores: bounds are wide against the score spacing, so many
    rows reach the threshold; all-equal rows: every row does."""
    corpus = workloads.small_int_matrix(40_000, 64, config_id=520)
    q = workloads.small_int_matrix(3, 64, config_id=520, stream=1)
    for k in (10, 300):
        g_idx, g_sc = _both(eng, corpus, q, k)
        o_idx, o_sc = oracle.search(corpus, q, k)
        assert np.array_equal(g_idx, o_idx)
        assert np.array_equal(g_sc.astype(np.float64), o_sc)
    flat = np.ones((30_000, 32), np.float32)
    g_idx, _ = _both(eng, flat, np.ones((1, 32), np.float32), 100)
    assert list(g_idx[0]) == list(range(100))


def test_filtered_zero_rows_and_query(eng):
    corpus = workloads.gaussian_rows(20_000, 256, config_id=530)
    corpus[::3] = 0.0
    q = workloads.gaussian_rows(2, 256, config_id=530, stream=1)
    _with_oracle(eng, corpus, q, 40)
    g_idx, g_sc = _both(eng, corpus, np.zeros((1, 256), np.float32), 20)
    assert list(g_idx[0]) == list(range(20)) and np.all(g_sc == 0)


def test_filtered_batch(eng):
    corpus = workloads.gaussian_rows(80_000, 768, config_id=540)
    qs = workloads.gaussian_rows(8, 768, config_id=540, stream=1)
    _with_oracle(eng, corpus, qs, 100)


def test_filtered_bf16_overflow_falls_back(eng):
    """A value beyond the largest bf16 makes the copy unusable for bounds: the
    call must still return the plain answer."""
    corpus = workloads.gaussian_rows(10_000, 128, config_id=550)
    corpus[777, 5] = np.float32(3.4e38)
    q = workloads.gaussian_rows(1, 128, config_id=550, stream=1)
    q[0, 5] = 0.0
    _both(eng, corpus, q, 16)


def test_filtered_worst_case_rounding(eng):
    """Every element of row 700 sits halfway between two bf16 values, with the
    rounding lowering every product (bf16 score 15.625, fp32 score 15.875, a
    shortfall of 2^-8 of sum |x q|); row 300 is exact in bf16 and scores 15.8125.
    A bound on the bf16 rounding below 2^-8 would exclude row 700, the answer."""
    d = 64
    corpus = workloads.gaussian_rows(5_000, d, config_id=580)
    corpus[700, :40] = 1 + 2.0 ** -8
    corpus[700, 40:] = -(1 + 3 * 2.0 ** -8)
    corpus[300] = 253 / 1024
    corpus[1200, :40] = -(1 + 2.0 ** -8)      # same construction, lowest scores
    corpus[1200, 40:] = 1 + 3 * 2.0 ** -8
    q = np.ones((1, d), np.float32)
    for k in (1, 2, 5):
        g_idx, g_sc = _both(eng, corpus, q, k, upload=(k == 1))
        assert g_idx[0, 0] == 700 and g_sc[0, 0] == np.float32(15.875)
        if k > 1:
            assert g_idx[0, 1] == 300 and g_sc[0, 1] == np.float32(15.8125)
    o_idx, o_sc = oracle.search(corpus, q, 5)
    check_retrieval(g_idx[0], g_sc[0], o_idx[0], o_sc[0], corpus, q[0], oracle)


def test_filtered_nonfinite_bf16_sum(eng):
    """Row 7 is (v, -v, 0, ...) with 3 v finite in fp32 while 3 bf16(v)
    overflows: its bf16 sum is inf + (-inf) = NaN, its fp32 score 0.  A NaN sum
    bounds nothing; the row must still be re-scored and the rest ranked."""
    d = 8
    v = np.float32(10913 * 2.0 ** 113)           # rounds up to 171 2^119 in bf16
    assert np.isfinite(np.float32(3) * v)
    corpus = workloads.gaussian_rows(3_000, d, config_id=590)
    corpus[7] = 0.0
    corpus[7, 0], corpus[7, 1] = v, -v
    q = np.zeros((1, d), np.float32)
    q[0, :2] = 3.0
    q[0, 2:] = 0.5
    for k in (1, 3, 40):
        _with_oracle(eng, corpus, q, k)


def test_filtered_zero_query_overflowing_row_norm(eng):
    """A row whose L2 norm overflows fp32 (inf) with a zero query: the bound's
    product 0 x inf is NaN; every score is 0 and ties go to the lowest indices."""
    d = 16
    corpus = workloads.gaussian_rows(2_000, d, config_id=595)
    corpus[1, :3] = np.float32(3.0e38)
    g_idx, g_sc = _both(eng, corpus, np.zeros((1, d), np.float32), 10)
    assert list(g_idx[0]) == list(range(10)) and np.all(g_sc == 0)


def test_filtered_shared_engines():
    corpus = workloads.gaussian_rows(50_000, 1024, config_id=560)
    qs = workloads.gaussian_rows(4, 1024, config_id=560, stream=1)
    with ResidentTopK(50_000, 1024, 128, 1) as a:
        a.upload_corpus_rowmajor(corpus)
        b = a.shared()
        b.enable_filtered()  # builds the shared bf16 copy from the resident corpus
        a.enable_filtered()  # only a's own scratch: the copy exists
        qd = torch.from_numpy(qs).cuda()
        o_idx, o_sc = oracle.search(corpus, qs, 64)
        for qi in range(4):
            for e in (a, b):
                i, s = e.search_resident_filtered(qd[qi:qi + 1], 64)
                torch.cuda.synchronize()
                check_retrieval(i.cpu().numpy()[0], s.cpu().numpy()[0], o_idx[qi], o_sc[qi], corpus, qs[qi], oracle)
        b.close()


def test_filtered_needs_enable():
    from top_search_resident_amd import ResidentTopKError
    with ResidentTopK(1000, 64, 8, 1) as e:
        e.upload_corpus_rowmajor(workloads.gaussian_rows(1000, 64, config_id=570))
        q = torch.zeros((1, 64), dtype=torch.float32, device="cuda")
        with pytest.raises(ResidentTopKError) as ei:
            e.search_resident_filtered(q, 4)
        assert ei.value.status == 2


def test_filtered_auto_small_corpus_runs_the_plain_scan():
    """Under the default storage choice a single query over a small corpus runs
    the plain scan (the two passes cost more there); a batch still takes a
    filtered path; a corpus above the threshold takes the fp8 pass.  Every
    answer is the single-query scan's, bit for bit."""
    with ResidentTopK(60_000, 1024, 64, 4) as e:
        e.enable_filtered()
        for n, want in ((20_000, "plain"), (60_000, "fp8")):  # 20.5M and 61.4M elements; threshold 46.1M
            corpus = workloads.gaussian_rows(n, 1024, config_id=580)
            qs = workloads.gaussian_rows(4, 1024, config_id=580, stream=1)
            e.upload_corpus_rowmajor(corpus)
            qd = torch.from_numpy(qs).cuda()
            for i in range(2):
                fi, fs = e.search_resident_filtered(qd[i:i + 1], 32)
                torch.cuda.synchronize()
                assert e.filter_path_used() == want, (n, e.filter_path_used())
                pi, ps = e.search_resident(qd[i:i + 1], 32)
                torch.cuda.synchronize()
                assert np.array_equal(fi.cpu().numpy(), pi.cpu().numpy())
                assert np.array_equal(fs.cpu().numpy().view(np.uint32), ps.cpu().numpy().view(np.uint32))
            bi, bs = e.search_resident_filtered(qd, 32)
            torch.cuda.synchronize()
            assert e.filter_path_used() == "bf16_matrix"
            for i in range(4):
                pi, ps = e.search_resident(qd[i:i + 1], 32)
                torch.cuda.synchronize()
                assert np.array_equal(bi.cpu().numpy()[i], pi.cpu().numpy()[0])
                assert np.array_equal(bs.cpu().numpy()[i].view(np.uint32), ps.cpu().numpy()[0].view(np.uint32))
