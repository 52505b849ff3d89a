"""Dynamic batching (rt_batcher_*): single queries submitted from many host
threads are gathered into batched searches.  In exact mode every answer must
equal, bit for bit, the plain single-query scan of the same query (the
filtered batch re-scores with the scan's arithmetic) and pass the oracle
checks; in plain mode the answers pass the oracle checks.  Also: mixed k in one
batch (each request gets the prefix of the batch's top-kmax), the batch sizes
reached, and the error paths."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
from gpu_util import check_retrieval
import workloads
from top_search_resident_amd import Batcher, ResidentTopK, ResidentTopKError

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

KS = (8, 32, 100, 1, 17)


def _single_scan(eng, q, k):
    idx, sc = eng.search_resident(torch.from_numpy(q[None, :]).cuda(), k)
    torch.cuda.synchronize()
    return idx.cpu().numpy()[0], sc.cpu().numpy()[0]


@pytest.mark.parametrize("exact", [True, False])
def test_batcher_many_threads(exact):
    print(f"[batcher] exact={exact}: 50k x 768, 96 queries from 12 threads", flush=True)
    corpus, qs = workloads.retrieval_inputs("c2_50k_768", queries=96)
    n, d = corpus.shape
    with ResidentTopK(n, d, 128, 32) as eng:
        eng.upload_corpus_rowmajor(corpus)
        if exact:
            eng.enable_filtered()
        scan = eng.shared(max_k=128, max_q=1)  # single-query scans, same corpus
        with Batcher(eng, max_batch=32, max_wait_us=3000, exact=exact) as b:
            def one(i):
                return b.search(qs[i], KS[i % len(KS)])
            with ThreadPoolExecutor(12) as ex:
                got = list(ex.map(one, range(len(qs))))
            st = b.stats()
        print(f"[batcher] stats {st}", flush=True)
        assert st["served"] == len(qs) and st["waiting"] == 0
        assert st["batches"] < len(qs) and st["largest_batch"] >= 2, st  # requests were batched
        o_idx, o_sc = oracle.search(corpus, qs, max(KS))
        for i, (idx, sc) in enumerate(got):
            k = KS[i % len(KS)]
            assert idx.shape == (k,) and sc.shape == (k,)
            check_retrieval(idx, sc, o_idx[i][:k], o_sc[i][:k], corpus, qs[i], oracle)
            if exact:
                s_idx, s_sc = _single_scan(scan, qs[i], k)
                assert np.array_equal(idx, s_idx), i
                assert np.array_equal(sc.view(np.uint32), s_sc.view(np.uint32)), i
        scan.close()


def test_batcher_waits_and_errors():
    corpus, qs = workloads.retrieval_inputs("c1_10k_384", queries=8)
    n, d = corpus.shape
    with ResidentTopK(n, d, 64, 8) as eng:
        with pytest.raises(ResidentTopKError) as ei:
            Batcher(eng, max_batch=8, exact=False)  # nothing resident
        assert ei.value.status == 2
        eng.upload_corpus_rowmajor(corpus)
        with pytest.raises(ResidentTopKError) as ei:
            Batcher(eng, max_batch=8, exact=True)  # enable_filtered not called
        assert ei.value.status == 2
        with pytest.raises(ResidentTopKError) as ei:
            Batcher(eng, max_batch=9, exact=False)  # beyond the engine's max_q
        assert ei.value.status == 1
        eng.enable_filtered()
        with Batcher(eng, max_batch=8, max_wait_us=0) as b:
            with pytest.raises(ResidentTopKError):
                b.submit(qs[0], 65)  # k > max_k
            with pytest.raises(ValueError):
                b.submit(qs[0][:10], 8)  # wrong depth
            handles = [b.submit(qs[i], 8) for i in range(8)]  # submitted before any wait
            out = [b.wait(h) for h in handles]
            with pytest.raises(ResidentTopKError):
                b.wait(handles[0])  # already waited for
            o_idx, o_sc = oracle.search(corpus, qs, 8)
            for i, (idx, sc) in enumerate(out):
                check_retrieval(idx, sc, o_idx[i], o_sc[i], corpus, qs[i], oracle)
