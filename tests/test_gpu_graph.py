"""HIP graph capture of the hot path: each entry point is captured once into a
torch.cuda.CUDAGraph on fixed buffers and replayed several times, with new
inputs copied into the captured input buffer before each replay and the
engine's own eager calls in between.  Every replay must equal the eager call
on the same input bit for bit (indices, order and score bits), and the eager
calls must still be right afterwards (the merge tree's counters, which each
call leaves at zero, are shared by both).  Covers the single-query scan, the
fp32 matrix-core batch, the filtered search (single query and batched, k below
and above 256) and the raw-array selection, with an engine and without one
(topk_select_noalloc, meant for callers under capture)."""
import numpy as np
import pytest

import oracle
from gpu_util import check_retrieval
import workloads
from top_search_resident_amd import ResidentTopK, topk_select_noalloc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

N, D, MAX_K, MAX_Q = 60_000, 768, 1024, 8
REPLAYS = 4


@pytest.fixture(scope="module")
def eng():
    assert torch.cuda.is_available(), "a GPU is required for the graph tests"
    e = ResidentTopK(N, D, MAX_K, MAX_Q, device=0)
    corpus = workloads.gaussian_rows(N, D, config_id=990)
    e.upload_corpus_rowmajor(corpus)
    e.enable_filtered()
    e.set_filter_storage("bf16")  # a single filtered query takes both passes at this size
    e._corpus = corpus
    yield e
    e.close()


def _capture(fn):
    """fn() enqueues the work on torch's current stream; returns the graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("mode,q,k", [
    ("plain", 1, 8), ("plain", 1, 100), ("plain", 8, 32), ("plain", 8, 1024),
    ("filtered", 1, 32), ("filtered", 8, 100), ("filtered", 8, 1024),
])
def test_search_graph_replays(eng, mode, q, k):
    print(f"[graph] {mode} q={q} k={k}", flush=True)
    qs = workloads.gaussian_rows(q * (REPLAYS + 1), D, config_id=991 + k, stream=1)
    q_static = torch.from_numpy(qs[:q]).cuda()
    oi = torch.empty((q, k), dtype=torch.int32, device="cuda")
    os_ = torch.empty((q, k), dtype=torch.float32, device="cuda")
    search = eng.search_resident if mode == "plain" else eng.search_resident_filtered
    g = _capture(lambda: search(q_static, k, oi, os_))
    for r in range(REPLAYS):
        batch = torch.from_numpy(qs[r * q:(r + 1) * q]).cuda()
        q_static.copy_(batch)
        g.replay()
        torch.cuda.synchronize()
        got_i, got_s = oi.cpu().numpy(), os_.cpu().numpy()
        ei, es = search(batch, k)  # eager, between replays
        torch.cuda.synchronize()
        assert np.array_equal(got_i, ei.cpu().numpy()), (mode, r)
        assert np.array_equal(got_s.view(np.uint32), es.cpu().numpy().view(np.uint32)), (mode, r)
        if r == 0:
            o_idx, o_sc = oracle.search(eng._corpus, qs[:1], k)
            check_retrieval(got_i[0], got_s[0], o_idx[0], o_sc[0], eng._corpus, qs[0], oracle)


@pytest.mark.parametrize("dtype,noalloc", [("int32", False), ("float32", False), ("int32", True),
                                           ("float32", True)])
def test_topk_select_graph_replays(eng, dtype, noalloc):
    print(f"[graph] topk_select {dtype} noalloc={noalloc}", flush=True)
    n, k = 3_000_001, 50
    rng = np.random.default_rng(992)
    if dtype == "int32":
        host = [rng.integers(-2**31, 2**31, n, dtype=np.int64).astype(np.int32) for _ in range(REPLAYS)]
    else:
        host = [rng.standard_normal(n).astype(np.float32) for _ in range(REPLAYS)]
    v_static = torch.from_numpy(host[0]).cuda()
    oi = torch.empty(k, dtype=torch.int32, device="cuda")
    ov = torch.empty(k, dtype=v_static.dtype, device="cuda")
    if noalloc:
        g = _capture(lambda: topk_select_noalloc(v_static, k, oi, ov))
    else:
        g = _capture(lambda: eng.topk_select(v_static, k, oi, ov))
    for r in range(REPLAYS):
        v_static.copy_(torch.from_numpy(host[r]).cuda())
        g.replay()
        torch.cuda.synchronize()
        got_i, got_v = oi.cpu().numpy(), ov.cpu().numpy()
        ei, ev = eng.topk_select(v_static, k)
        torch.cuda.synchronize()
        assert np.array_equal(got_i, ei.cpu().numpy()), r
        assert np.array_equal(got_v.view(np.uint32), ev.cpu().numpy().view(np.uint32)), r
        o_idx, o_val = oracle.topk(host[r], k)
        assert np.array_equal(got_i, o_idx), r
        assert np.array_equal(got_v.view(np.uint32), np.asarray(o_val, dtype=got_v.dtype).view(np.uint32)), r
