"""Concurrent searches on engines that share one resident corpus
(rt_engine_create_shared): several engines, each on its own stream, issue
searches and selects without synchronising in between; every answer must match
the CPU oracle and the same search run alone.  Also the shared corpus's
lifetime and an upload through a sharing engine."""
import numpy as np
import pytest

import oracle
from gpu_util import check_exact_topk_property, check_retrieval
import workloads
from top_search_resident_amd import ResidentTopK

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _host(t):
    return t.cpu().numpy()


def test_concurrent_single_queries_on_streams():
    corpus, qs = workloads.retrieval_inputs("c2_50k_768", queries=24)
    n, d = corpus.shape
    ks = (8, 32, 100, 1)
    with ResidentTopK(n, d, 128, 1) as parent:
        parent.upload_corpus_rowmajor(corpus)
        engines = [parent.shared(max_k=128, max_q=1) for _ in range(4)]
        streams = [torch.cuda.Stream() for _ in range(4)]
        qdev = torch.from_numpy(qs).cuda()
        torch.cuda.synchronize()
        results = []
        for r in range(6):
            for e, (eng, s) in enumerate(zip(engines, streams)):
                qi = r * 4 + e
                k = ks[e]
                with torch.cuda.stream(s):
                    idx, sc = eng.search_resident(qdev[qi:qi + 1], k, stream=s)
                results.append((qi, k, idx, sc))
        torch.cuda.synchronize()
        o_idx, o_sc = oracle.search(corpus, qs, max(ks))
        for qi, k, idx, sc in results:
            g_idx, g_sc = _host(idx)[0], _host(sc)[0]
            check_retrieval(g_idx, g_sc, o_idx[qi, :k], o_sc[qi, :k], corpus, qs[qi], oracle)
            a_idx, a_sc = parent.search_resident(qdev[qi:qi + 1], k)
            torch.cuda.synchronize()
            assert np.array_equal(_host(a_idx)[0], g_idx), (qi, k)
            assert np.array_equal(_host(a_sc)[0].view(np.uint32), g_sc.view(np.uint32)), (qi, k)
        for eng in engines:
            eng.close()


def test_concurrent_batch_cosine_and_select():
    """A batched (MFMA) search, a cosine search and a raw int32 top-K run at the
    same time on three engines sharing one corpus."""
    corpus = workloads.scaled_rows(30_000, 256, config_id=400)
    qs = workloads.gaussian_rows(16, 256, config_id=400, stream=1)
    vals = workloads.int32_values(n=3_000_000, config_id=401)
    with ResidentTopK(30_000, 256, 256, 16) as a:
        a.upload_corpus_rowmajor(corpus)
        b = a.shared(max_k=64, max_q=1)
        c = a.shared(max_k=64, max_q=1)
        sa, sb, sc_ = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
        qdev = torch.from_numpy(qs).cuda()
        vdev = torch.from_numpy(vals).cuda()
        torch.cuda.synchronize()
        for _ in range(3):
            with torch.cuda.stream(sa):
                ai, asc = a.search_resident(qdev, 200, stream=sa)
            with torch.cuda.stream(sb):
                bi, bsc = b.search_resident(qdev[3:4], 50, stream=sb, metric="cosine")
            with torch.cuda.stream(sc_):
                ci, cv = c.topk_select(vdev, 64, stream=sc_)
        torch.cuda.synchronize()
        o_idx, o_sc = oracle.search(corpus, qs, 200)
        for qi in range(16):
            check_retrieval(_host(ai)[qi], _host(asc)[qi], o_idx[qi], o_sc[qi], corpus, qs[qi], oracle)
        oc_idx, oc_sc = oracle.search(corpus, qs[3:4], 50, metric=1)
        check_retrieval(_host(bi)[0], _host(bsc)[0], oc_idx[0], oc_sc[0], corpus, qs[3], oracle, metric="cosine")
        r_idx, r_val = oracle.topk(vals, 64)
        assert np.array_equal(_host(ci), r_idx)
        assert np.array_equal(_host(cv), r_val)
        check_exact_topk_property(_host(ci), _host(cv), vals)
        b.close()
        c.close()


def test_shared_corpus_lifetime_and_upload():
    """The corpus outlives the engine that created it while another engine shares
    it, and an upload through one sharing engine is what every sharer searches."""
    c1 = workloads.gaussian_rows(5_000, 128, config_id=402)
    c2 = workloads.gaussian_rows(4_000, 128, config_id=403)
    q = workloads.gaussian_rows(1, 128, config_id=402, stream=1)
    qdev = torch.from_numpy(q).cuda()
    parent = ResidentTopK(5_000, 128, 64, 1)
    parent.upload_corpus_rowmajor(c1)
    child = parent.shared()
    other = child.shared(max_k=16)
    parent.close()  # the corpus stays: two engines still share it
    idx, sc = child.search_resident(qdev, 10)
    torch.cuda.synchronize()
    o_idx, o_sc = oracle.search(c1, q, 10)
    check_retrieval(_host(idx)[0], _host(sc)[0], o_idx[0], o_sc[0], c1, q[0], oracle)
    assert child.info()["resident_n"] == 5_000
    other.upload_corpus_rowmajor(c2)  # replaces the corpus for both
    assert child.info()["resident_n"] == 4_000
    idx, sc = child.search_resident(qdev, 10)
    torch.cuda.synchronize()
    o_idx, o_sc = oracle.search(c2, q, 10)
    check_retrieval(_host(idx)[0], _host(sc)[0], o_idx[0], o_sc[0], c2, q[0], oracle)
    child.close()
    idx, sc = other.search_resident(qdev, 16)
    torch.cuda.synchronize()
    o_idx, o_sc = oracle.search(c2, q, 16)
    check_retrieval(_host(idx)[0], _host(sc)[0], o_idx[0], o_sc[0], c2, q[0], oracle)
    other.close()
