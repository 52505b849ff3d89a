"""Seeded random shapes against the oracle: corpus sizes from 1 row to a few
hundred thousand, depths that do and do not fit the fast lane-group shapes
(4 .. 1024, including 100 and 1000), batches of 1 .. 32 queries, k from 1 to
1024 (capped at n), both metrics, duplicate rows, and the filtered search
(which must equal the single-query scan bit for bit); and raw int32/fp32
arrays from 1 to 6M elements with k up to 1024, ties, sorted runs and
misaligned starts (bit-exact).  Each case prints its parameters first."""
import numpy as np
import pytest

import oracle
from gpu_util import check_retrieval
from top_search_resident_amd import ResidentTopK

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

KS = (1, 5, 8, 32, 33, 64, 100, 257, 1024)
DEPTHS = (4, 8, 12, 64, 100, 128, 256, 384, 512, 768, 1000, 1024)


@pytest.mark.parametrize("case", range(40))
def test_random_search_shapes(case):
    rng = np.random.default_rng(5000 + case)
    d = int(rng.choice(DEPTHS))
    n = int(np.exp(rng.uniform(0.0, np.log(min(300_000, 4e7 / d)))))
    q = int(rng.choice([1, 1, 1, 2, 5, 32]))
    k = int(min(n, rng.choice(KS)))
    metric = "cosine" if rng.random() < 0.3 else "dot"
    filtered = d % 8 == 0 and rng.random() < 0.5
    storage = ("auto", "bf16", "fp8")[case % 3]  # first pass of a single-query filtered search
    print(f"[random search] case {case}: n={n} d={d} q={q} k={k} {metric} filtered={filtered} {storage}",
          flush=True)
    x = rng.standard_normal((n, d)).astype(np.float32)
    x /= np.linalg.norm(x, axis=1, keepdims=True).astype(np.float32) + np.float32(1e-30)
    if rng.random() < 0.3:  # duplicate rows: exact score ties
        x[rng.integers(0, n, n // 10)] = x[rng.integers(0, n, n // 10)]
    qs = rng.standard_normal((q, d)).astype(np.float32)
    with ResidentTopK(n, d, 1024, 32) as eng:
        eng.upload_corpus_rowmajor(x)
        qd = torch.from_numpy(qs).cuda()
        if filtered:
            eng.enable_filtered()
            eng.set_filter_storage(storage)
            gi, gs = eng.search_resident_filtered(qd, k, metric=metric)
            ref = [eng.search_resident(qd[i:i + 1], k, metric=metric) for i in range(q)]
        else:
            gi, gs = eng.search_resident(qd, k, metric=metric)
            ref = None
        torch.cuda.synchronize()
        gi, gs = gi.cpu().numpy(), gs.cpu().numpy()
        if ref is not None:
            for i in range(q):
                assert np.array_equal(gi[i], ref[i][0].cpu().numpy()[0]), i
                assert np.array_equal(gs[i].view(np.uint32), ref[i][1].cpu().numpy()[0].view(np.uint32)), i
    o_idx, o_sc = oracle.search(x, qs, k, 1 if metric == "cosine" else 0)
    for i in range(q):
        check_retrieval(gi[i], gs[i], o_idx[i], o_sc[i], x, qs[i], oracle, metric=metric)


@pytest.mark.parametrize("case", range(40))
def test_random_select_shapes(case):
    rng = np.random.default_rng(6000 + case)
    n = int(np.exp(rng.uniform(0.0, np.log(6e6))))
    k = int(min(n, rng.choice([1, 2, 7, 9, 16, 17, 31, 33, 63, 65, 100, 129, 257, 700, 1024])))
    off = int(rng.integers(0, 4))
    dist = int(rng.integers(0, 5))
    if dist == 0:
        v = rng.integers(-(2 ** 31), 2 ** 31, size=n + off, dtype=np.int64).astype(np.int32)
    elif dist == 1:
        v = rng.integers(-3, 3, size=n + off, dtype=np.int32)
    elif dist == 2:
        v = np.sort(rng.integers(-(2 ** 31), 2 ** 31, size=n + off, dtype=np.int64)).astype(np.int32)
        if rng.random() < 0.5:
            v = v[::-1].copy()
    elif dist == 3:
        v = rng.standard_normal(n + off).astype(np.float32)
    else:
        v = np.round(rng.standard_normal(n + off) * 4).astype(np.float32)
    print(f"[random select] case {case}: n={n} k={k} offset={off} dist={dist} dtype={v.dtype}", flush=True)
    with ResidentTopK(1, 1, 1024, 1) as eng:
        buf = torch.from_numpy(np.ascontiguousarray(v)).cuda()
        gi, gv = eng.topk_select(buf[off:], k)
        torch.cuda.synchronize()
        gi, gv = gi.cpu().numpy(), gv.cpu().numpy()
    oi, ov = oracle.topk(v[off:], k)
    assert np.array_equal(gi, oi)
    assert np.array_equal(gv.view(np.uint32), ov.view(np.uint32))
