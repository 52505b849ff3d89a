"""Dynamic batching (rt_batcher_*): single queries submitted from many host
threads are gathered into batched searches.  In exact mode every answer must
equal, bit for bit, the plain single-query scan of the same query (the
filtered batch re-scores with the scan's arithmetic) and pass the oracle
checks; in plain mode the answers pass the oracle checks.  Also: mixed k in one
batch (each request gets the prefix of the batch's top-kmax), k above 256 (the
filtered batch's candidate lists), requests whose handles are dropped or still
queued when the batcher or its engine closes, the batch sizes reached, and the
error paths."""
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


def test_batcher_large_k_exact():
    """k up to 1024 in exact mode: the batch re-ranks through per-query
    candidate lists, and every answer is still the single-query scan's."""
    ks = (1024, 8, 300, 257, 64)
    print("[batcher] 100k x 768, 40 queries, k up to 1024", flush=True)
    corpus = workloads.gaussian_rows(100_000, 768, config_id=720)
    qs = workloads.gaussian_rows(40, 768, config_id=720, stream=1)
    with ResidentTopK(100_000, 768, 1024, 32) as eng:
        eng.upload_corpus_rowmajor(corpus)
        eng.enable_filtered()
        scan = eng.shared(max_k=1024, max_q=1)
        with Batcher(eng, max_batch=16, max_wait_us=3000) as b:
            with ThreadPoolExecutor(8) as ex:
                got = list(ex.map(lambda i: b.search(qs[i], ks[i % len(ks)]), range(len(qs))))
            assert b.stats()["largest_batch"] >= 2
        for i, (idx, sc) in enumerate(got):
            s_idx, s_sc = _single_scan(scan, qs[i], ks[i % len(ks)])
            assert np.array_equal(idx, s_idx), i
            assert np.array_equal(sc.view(np.uint32), s_sc.view(np.uint32)), i
        o_idx, o_sc = oracle.search(corpus, qs[:3], 1024)
        for i in range(3):
            k = ks[i % len(ks)]
            check_retrieval(got[i][0], got[i][1], o_idx[i][:k], o_sc[i][:k], corpus, qs[i], oracle)
        scan.close()


def test_batcher_dropped_and_pending_requests():
    """Handles dropped without wait() and requests still queued at close: the
    batcher keeps their arrays alive, close() serves them, and closing the
    engine closes its batcher first."""
    import gc
    corpus, qs = workloads.retrieval_inputs("c1_10k_384", queries=16)
    n, d = corpus.shape
    o_idx, o_sc = oracle.search(corpus, qs, 8)
    eng = ResidentTopK(n, d, 64, 16)
    eng.upload_corpus_rowmajor(corpus)
    eng.enable_filtered()
    b = Batcher(eng, max_batch=16, max_wait_us=200_000)  # long wait: requests stay queued
    for i in range(4):
        b.submit(qs[i], 8)  # handle dropped at once
    gc.collect()
    kept = [b.submit(qs[i], 8) for i in range(4, 16)]
    b.close()  # serves all 16, then frees the batcher
    for i, (_, idx, sc, _) in zip(range(4, 16), kept):
        check_retrieval(idx, sc, o_idx[i], o_sc[i], corpus, qs[i], oracle)
    with pytest.raises(ResidentTopKError):
        b.wait(kept[0])  # the batcher is closed
    b2 = Batcher(eng, max_batch=16, max_wait_us=200_000)
    h = b2.submit(qs[0], 8)
    eng.close()  # closes b2 first, which serves the queued request
    check_retrieval(h[1], h[2], o_idx[0], o_sc[0], corpus, qs[0], oracle)
