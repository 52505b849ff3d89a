"""The five workloads at full size, in the launch configuration the benchmark
times.  The oracle checks a sample of queries in full (R1-R4); the other queries
are checked row by row (returned scores against the oracle's fp64 scores of the
same rows), for sortedness and distinctness, and -- on a further sample -- for
completeness against the oracle's scores of every row.  The raw int32 top-K is
checked exactly: against the oracle once, and by rank counting for every K."""
import numpy as np
import pytest

import oracle
from gpu_util import REL_TOL, SCALE_FLOOR, check_exact_topk_property, check_retrieval, cs_bound
import workloads
from top_search_resident_amd import ResidentTopK

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _sorted_distinct(idx, sc):
    assert np.unique(idx).size == idx.size
    for j in range(idx.size - 1):
        assert sc[j] > sc[j + 1] or (sc[j] == sc[j + 1] and idx[j] < idx[j + 1])


def _row_scores_match(idx, sc, corpus, q):
    rows = corpus[idx.astype(np.int64)]
    o = oracle.scores(rows, q)
    den = np.maximum(np.abs(o), SCALE_FLOOR * cs_bound(rows, q))
    assert np.all(np.abs(sc.astype(np.float64) - o) <= REL_TOL * den)


def _complete(idx, sc, corpus, q):
    """No row left out has an oracle score above the k-th returned row's oracle
    score by more than the tolerance (R3 without a sort)."""
    o_all = oracle.scores(corpus, q)
    mask = np.ones(corpus.shape[0], dtype=bool)
    mask[idx] = False
    o_k = o_all[idx].min()
    assert o_all[mask].max() <= o_k + REL_TOL * abs(o_k)


def _run_sequential(eng, qdev, k):
    out_i = np.empty((qdev.shape[0], k), np.int32)
    out_s = np.empty((qdev.shape[0], k), np.float32)
    for qi in range(qdev.shape[0]):
        i, s = eng.search_resident(qdev[qi:qi + 1], k)
        out_i[qi], out_s[qi] = i.cpu().numpy()[0], s.cpu().numpy()[0]
    return out_i, out_s


@pytest.mark.parametrize("name,n_full,n_complete", [
    ("c1_10k_384", 1, 1), ("c2_50k_768", 40, 200), ("c2_100k_768", 40, 200), ("c3_1m_1024", 3, 12)])
def test_single_query_workloads(name, n_full, n_complete):
    w = workloads.WORKLOADS[name]
    print(f"[fullsize] {name}: generating inputs", flush=True)
    corpus, qs = workloads.retrieval_inputs(name)
    n, d = corpus.shape
    with ResidentTopK(n, d, max(w["ks"]), 1) as eng:
        eng.upload_corpus_rowmajor(corpus)
        qdev = torch.from_numpy(qs).cuda()
        kmax = max(w["ks"])
        o_idx, o_sc = oracle.search(corpus, qs[:n_full], kmax)
        for k in w["ks"]:
            print(f"[fullsize] {name}: {qs.shape[0]} sequential queries at k={k}", flush=True)
            g_idx, g_sc = _run_sequential(eng, qdev, k)
            for qi in range(qs.shape[0]):
                _sorted_distinct(g_idx[qi], g_sc[qi])
            for qi in range(0, qs.shape[0], max(1, qs.shape[0] // 100)):
                _row_scores_match(g_idx[qi], g_sc[qi], corpus, qs[qi])
            for qi in range(n_full):
                check_retrieval(g_idx[qi], g_sc[qi], o_idx[qi, :k], o_sc[qi, :k], corpus, qs[qi], oracle)
            step = max(1, qs.shape[0] // n_complete)
            for qi in range(0, qs.shape[0], step)[:n_complete]:
                _complete(g_idx[qi], g_sc[qi], corpus, qs[qi])
            if name == "c2_100k_768" or name == "c3_1m_1024":
                # the filtered search as the benchmark's leg runs it (the engine
                # chooses the fp8 first pass at these sizes): the same answers,
                # bit for bit, on a sample of the queries
                eng.enable_filtered()
                for qi in range(0, qs.shape[0], max(1, qs.shape[0] // 50)):
                    f_idx, f_sc = eng.search_resident_filtered(qdev[qi:qi + 1], k)
                    torch.cuda.synchronize()
                    assert eng.filter_path_used() == "fp8"
                    assert np.array_equal(f_idx.cpu().numpy()[0], g_idx[qi]), (name, k, qi)
                    assert np.array_equal(f_sc.cpu().numpy()[0].view(np.uint32), g_sc[qi].view(np.uint32))


def test_c3_repeat_is_bit_identical():
    """One query at the large single-query size, repeated 50 times at each K:
    the merge tree's workgroups arrive in a different order on every call, yet
    the indices and score bits must not change (the order is the comparator's,
    decided on the device, with no float sum across workgroups)."""
    name = "c3_1m_1024"
    print(f"[fullsize] {name} repeat: generating inputs", flush=True)
    corpus, qs = workloads.retrieval_inputs(name, queries=2)
    n, d = corpus.shape
    ks = workloads.WORKLOADS[name]["ks"]
    with ResidentTopK(n, d, max(ks), 1) as eng:
        eng.upload_corpus_rowmajor(corpus)
        qdev = torch.from_numpy(qs).cuda()
        for k in ks:
            outs = []
            for rep in range(50):
                outs.append(eng.search_resident(qdev[:1], k))
            torch.cuda.synchronize()
            i0, s0 = outs[0][0].cpu().numpy(), outs[0][1].cpu().numpy()
            for rep, (i, s) in enumerate(outs[1:], 1):
                assert np.array_equal(i.cpu().numpy(), i0), (k, rep)
                assert np.array_equal(s.cpu().numpy().view(np.uint32), s0.view(np.uint32)), (k, rep)
        o_idx, o_sc = oracle.search(corpus, qs[:1], max(ks))
        check_retrieval(i0[0], s0[0], o_idx[0, :max(ks)], o_sc[0, :max(ks)], corpus, qs[0], oracle)


def test_int32_1e8():
    print("[fullsize] c4_1e8_int32: generating inputs", flush=True)
    v = workloads.int32_values()
    vdev = torch.from_numpy(v).cuda()
    ks = workloads.WORKLOADS["c4_1e8_int32"]["ks"]
    with ResidentTopK(1, 1, max(ks), 1) as eng:
        res = {}
        for k in ks:
            i, x = eng.topk_select(vdev, k)
            torch.cuda.synchronize()
            res[k] = (i.cpu().numpy(), x.cpu().numpy())
            check_exact_topk_property(res[k][0], res[k][1], v)
        print("[fullsize] c4_1e8_int32: oracle full sort", flush=True)
        o_idx, o_val = oracle.topk(v, max(ks))
        for k in ks:
            assert np.array_equal(res[k][0], o_idx[:k])
            assert np.array_equal(res[k][1], o_val[:k])


def test_batched_500k():
    name = "c5_q32_500k_768"
    w = workloads.WORKLOADS[name]
    print(f"[fullsize] {name}: generating inputs", flush=True)
    corpus, qs = workloads.retrieval_inputs(name)
    n, d = corpus.shape
    with ResidentTopK(n, d, max(w["ks"]), 32) as eng:
        eng.upload_corpus_rowmajor(corpus)
        qdev = torch.from_numpy(qs).cuda()
        res = {}
        for k in w["ks"]:
            i, s = eng.search_resident(qdev, k)
            torch.cuda.synchronize()
            res[k] = (i.cpu().numpy(), s.cpu().numpy())
        print(f"[fullsize] {name}: oracle for 32 queries", flush=True)
        o_idx, o_sc = oracle.search(corpus, qs, max(w["ks"]))
        for k in w["ks"]:
            for qi in range(qs.shape[0]):
                check_retrieval(res[k][0][qi], res[k][1][qi], o_idx[qi, :k], o_sc[qi, :k], corpus, qs[qi], oracle)
        # the same batch through the bf16 matrix-core filter (the benchmark's
        # filtered leg): every query's answer is the single-query scan's, bit
        # for bit, and passes the oracle rules
        print(f"[fullsize] {name}: filtered batch", flush=True)
        eng.enable_filtered()
        for k in w["ks"]:
            f_idx, f_sc = eng.search_resident_filtered(qdev, k)
            plain = [eng.search_resident(qdev[qi:qi + 1], k) for qi in range(qs.shape[0])]
            torch.cuda.synchronize()
            p_idx = np.concatenate([p[0].cpu().numpy() for p in plain])
            p_sc = np.concatenate([p[1].cpu().numpy() for p in plain])
            f_idx, f_sc = f_idx.cpu().numpy(), f_sc.cpu().numpy()
            assert np.array_equal(f_idx, p_idx), k
            assert np.array_equal(f_sc.view(np.uint32), p_sc.view(np.uint32)), k
            for qi in range(qs.shape[0]):
                check_retrieval(f_idx[qi], f_sc[qi], o_idx[qi, :k], o_sc[qi, :k], corpus, qs[qi], oracle)


def test_cosine_1m():
    """The cosine metric at the large single-query size, rows rescaled by
    log-normal factors (so each row's norm matters), in the launch configuration
    the benchmark times with --metric cosine."""
    name = "c3_1m_1024"
    print(f"[fullsize] {name} cosine: generating inputs", flush=True)
    corpus, qs = workloads.retrieval_inputs(name, queries=24)
    rng = np.random.default_rng(77)
    corpus *= np.exp(rng.standard_normal(corpus.shape[0])).astype(np.float32)[:, None]
    qs *= np.float32(3.0)
    n, d = corpus.shape
    ks = workloads.WORKLOADS[name]["ks"]
    with ResidentTopK(n, d, max(ks), 1) as eng:
        eng.upload_corpus_rowmajor(corpus)
        qdev = torch.from_numpy(qs).cuda()
        print(f"[fullsize] {name} cosine: oracle for 2 queries", flush=True)
        o_idx, o_sc = oracle.search(corpus, qs[:2], max(ks), metric=1)
        for k in ks:
            for qi in range(qs.shape[0]):
                i, s = eng.search_resident(qdev[qi:qi + 1], k, metric="cosine")
                g_idx, g_sc = i.cpu().numpy()[0], s.cpu().numpy()[0]
                _sorted_distinct(g_idx, g_sc)
                o_rows = oracle.cosine_scores(corpus[g_idx.astype(np.int64)], qs[qi])
                assert np.all(np.abs(g_sc.astype(np.float64) - o_rows) <= REL_TOL * np.maximum(np.abs(o_rows), 0.01))
                if qi < 2:
                    check_retrieval(g_idx, g_sc, o_idx[qi, :k], o_sc[qi, :k], corpus, qs[qi], oracle,
                                    metric="cosine")
