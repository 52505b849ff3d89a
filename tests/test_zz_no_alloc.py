"""topk_select_noalloc (no engine, no allocation: the kernels' scratch is a
static device array per GPU) against topk_select through the C ABI: the same
indices and value bits, on two calls in a row, the second with a smaller
input, for int32 and fp32 arrays, and against the oracle."""
import ctypes

import numpy as np
import pytest

import oracle
import workloads
from top_search_resident_amd import ResidentTopK, ResidentTopKError, _lib, topk_select_noalloc

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _raw_noalloc(values, k):
    """Call the C entry point directly with torch-owned buffers."""
    lib = _lib.load()
    oi = torch.empty(k, dtype=torch.int32, device="cuda")
    ov = torch.empty(k, dtype=values.dtype, device="cuda")
    dt = _lib.RT_DTYPE_INT32 if values.dtype == torch.int32 else _lib.RT_DTYPE_FLOAT32
    st = lib.topk_select_noalloc(ctypes.c_void_p(values.data_ptr()), dt, int(values.numel()), int(k),
                                 ctypes.c_void_p(oi.data_ptr()), ctypes.c_void_p(ov.data_ptr()),
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == _lib.RT_OK, st
    return oi, ov


def _same(a, b):
    return (np.array_equal(a[0].cpu().numpy(), b[0].cpu().numpy()) and
            np.array_equal(a[1].cpu().numpy().view(np.uint32), b[1].cpu().numpy().view(np.uint32)))


@pytest.mark.parametrize("k_big,k_small", [(50, 20), (1024, 100), (300, 7)])
def test_noalloc_matches_topk_select_twice(k_big, k_small):
    big = torch.from_numpy(workloads.int32_values(n=3_000_000, config_id=60)).cuda()
    small = torch.from_numpy(workloads.int32_values(n=123_457, config_id=61)).cuda()
    with ResidentTopK(1, 1, 1024, 1) as eng:
        ref_big = eng.topk_select(big, k_big)
        ref_small = eng.topk_select(small, k_small)
        got_big = _raw_noalloc(big, k_big)
        got_small = _raw_noalloc(small, k_small)  # second call, smaller input
        torch.cuda.synchronize()
    assert _same(got_big, ref_big), "first call differs from topk_select"
    assert _same(got_small, ref_small), "second (smaller) call differs from topk_select"
    o_idx, o_val = oracle.topk(small.cpu().numpy(), k_small)
    assert np.array_equal(got_small[0].cpu().numpy(), o_idx)
    assert np.array_equal(got_small[1].cpu().numpy(), o_val)


def test_noalloc_float_and_edges():
    rng = np.random.default_rng(9)
    v = rng.standard_normal(1_000_003).astype(np.float32)
    v[rng.choice(v.size, 64, replace=False)] = np.float32(-0.0)
    v[rng.choice(v.size, 8, replace=False)] = np.inf
    buf = torch.from_numpy(v).cuda()
    with ResidentTopK(1, 1, 1024, 1) as eng:
        for off, k in ((0, 1024), (3, 33), (1, 1)):
            view = buf[off:]
            ref = eng.topk_select(view, k)
            got = topk_select_noalloc(view, k)
            torch.cuda.synchronize()
            assert _same(got, ref), (off, k)
            o_idx, o_val = oracle.topk(v[off:], k)
            assert np.array_equal(got[0].cpu().numpy(), o_idx)
            assert np.array_equal(got[1].cpu().numpy().view(np.uint32), o_val.view(np.uint32))
    # tiny arrays (one workgroup) and k == n
    t = torch.tensor([5, -1, 5, 7], dtype=torch.int32, device="cuda")
    i, x = topk_select_noalloc(t, 4)
    torch.cuda.synchronize()
    assert list(i.cpu().numpy()) == [3, 0, 2, 1] and list(x.cpu().numpy()) == [7, 5, 5, -1]


def test_noalloc_rejects_bad_arguments():
    lib = _lib.load()
    t = torch.zeros(16, dtype=torch.int32, device="cuda")
    oi = torch.empty(8, dtype=torch.int32, device="cuda")
    p = ctypes.c_void_p
    s = p(torch.cuda.current_stream().cuda_stream)
    assert lib.topk_select_noalloc(p(t.data_ptr()), 0, 16, 1025, p(oi.data_ptr()), p(oi.data_ptr()), s) == 1
    assert lib.topk_select_noalloc(p(t.data_ptr()), 0, 16, 17, p(oi.data_ptr()), p(oi.data_ptr()), s) == 1
    assert lib.topk_select_noalloc(p(t.data_ptr()), 2, 16, 4, p(oi.data_ptr()), p(oi.data_ptr()), s) == 1
    assert lib.topk_select_noalloc(p(t.data_ptr() + 2), 0, 8, 4, p(oi.data_ptr()), p(oi.data_ptr()), s) == 1
    assert lib.topk_select_noalloc(p(0), 0, 16, 4, p(oi.data_ptr()), p(oi.data_ptr()), s) == 1
    with pytest.raises(ResidentTopKError):
        topk_select_noalloc(t, 0)
    with pytest.raises(TypeError):
        topk_select_noalloc(t.cpu(), 4)
    i, x = topk_select_noalloc(t, 4)  # still works after the refusals
    torch.cuda.synchronize()
    assert list(i.cpu().numpy()) == [0, 1, 2, 3]
