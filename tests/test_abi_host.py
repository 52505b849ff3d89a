"""The C-ABI library on the host (no GPU): it loads, exports every symbol the
header declares, and its host-side argument checks follow the documented rules."""
import ctypes
import os
import re

import pytest

from top_search_resident_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "resident_topk.h")
OK, EINVAL, ESTATE = _lib.RT_OK, _lib.RT_EINVAL, _lib.RT_ESTATE
P = ctypes.c_void_p(0x1000)      # a non-null pointer value (never dereferenced by the checks)
NULL = ctypes.c_void_p(0)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([A-Za-z_][A-Za-z0-9_]*)\s*\(", text)) -
                  {"defined", "extern", "if", "sizeof"})


def test_header_and_binding_agree():
    assert sorted(_lib.EXPORTS) == _declared_functions()


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for s in range(5):
        assert lib.rt_status_string(s)
    assert b"unknown" in lib.rt_status_string(99)


def test_check_create(lib):
    assert lib.rt_check_create(1_000_000, 1024, 1024, 32) == OK
    assert lib.rt_check_create(0, 8, 8, 1) == EINVAL
    assert lib.rt_check_create(2 ** 31, 8, 8, 1) == EINVAL
    assert lib.rt_check_create(10, 0, 8, 1) == EINVAL
    assert lib.rt_check_create(10, 65537, 8, 1) == EINVAL
    assert lib.rt_check_create(10, 8, 0, 1) == EINVAL
    assert lib.rt_check_create(10, 8, 1025, 1) == EINVAL
    assert lib.rt_check_create(10, 8, 8, 0) == EINVAL
    assert lib.rt_check_create(10, 8, 8, 33) == EINVAL


def test_check_upload(lib):
    assert lib.rt_check_upload(100, 64, P, 100, 64) == OK
    assert lib.rt_check_upload(100, 64, NULL, 100, 64) == EINVAL
    assert lib.rt_check_upload(100, 64, P, 101, 64) == EINVAL   # N > max_n
    assert lib.rt_check_upload(100, 64, P, 100, 65) == EINVAL   # D > max_d
    assert lib.rt_check_upload(100, 64, P, 0, 64) == EINVAL


def test_check_search(lib):
    assert lib.rt_check_search(128, 32, 1000, P, 1, 8, P, P) == OK
    assert lib.rt_check_search(128, 32, 1000, P, 32, 128, P, P) == OK
    assert lib.rt_check_search(128, 32, 8, P, 1, 8, P, P) == OK        # k == n: full sort
    assert lib.rt_check_search(128, 32, 7, P, 1, 8, P, P) == EINVAL    # k > n
    assert lib.rt_check_search(128, 32, 0, P, 1, 8, P, P) == ESTATE    # nothing resident
    assert lib.rt_check_search(128, 32, 1000, P, 1, 129, P, P) == EINVAL
    assert lib.rt_check_search(128, 32, 1000, P, 1, 0, P, P) == EINVAL
    assert lib.rt_check_search(128, 32, 1000, P, 33, 8, P, P) == EINVAL
    assert lib.rt_check_search(128, 32, 1000, P, 0, 8, P, P) == EINVAL
    for args in ((NULL, P, P), (P, NULL, P), (P, P, NULL)):
        assert lib.rt_check_search(128, 32, 1000, args[0], 1, 8, args[1], args[2]) == EINVAL


def test_check_search_metric(lib):
    for metric in (_lib.RT_METRIC_DOT, _lib.RT_METRIC_COSINE):
        assert lib.rt_check_search_metric(128, 32, 1000, P, 1, 8, metric, P, P) == OK
        assert lib.rt_check_search_metric(128, 32, 7, P, 1, 8, metric, P, P) == EINVAL   # k > n
        assert lib.rt_check_search_metric(128, 32, 0, P, 1, 8, metric, P, P) == ESTATE   # nothing resident
        assert lib.rt_check_search_metric(128, 32, 1000, NULL, 1, 8, metric, P, P) == EINVAL
    for metric in (-1, 2, 99):
        assert lib.rt_check_search_metric(128, 32, 1000, P, 1, 8, metric, P, P) == EINVAL


def test_check_select(lib):
    assert lib.rt_check_select(64, P, 0, 1000, 50, P, P) == OK
    assert lib.rt_check_select(64, P, 1, 1000, 50, P, P) == OK
    assert lib.rt_check_select(64, P, 2, 1000, 50, P, P) == EINVAL            # dtype
    assert lib.rt_check_select(64, ctypes.c_void_p(0x1002), 0, 1000, 50, P, P) == EINVAL  # misaligned
    assert lib.rt_check_select(64, P, 0, 49, 50, P, P) == EINVAL              # k > n
    assert lib.rt_check_select(64, P, 0, 1000, 65, P, P) == EINVAL            # k > max_k
    assert lib.rt_check_select(64, P, 0, 2 ** 31, 50, P, P) == EINVAL         # int32 indices
    assert lib.rt_check_select(64, NULL, 0, 1000, 50, P, P) == EINVAL


def test_entry_points_reject_null_engine(lib):
    assert lib.upload_corpus_rowmajor(NULL, P, 10, 4) == EINVAL
    assert lib.search_resident(NULL, P, 1, 1, P, P, NULL) == EINVAL
    assert lib.search_resident_metric(NULL, P, 1, 1, 1, P, P, NULL) == EINVAL
    assert lib.search_resident_filtered(NULL, P, 1, 1, P, P, NULL) == EINVAL
    assert lib.rt_enable_filtered(NULL) == EINVAL
    assert lib.topk_select(NULL, P, 0, 10, 1, P, P, NULL) == EINVAL
    assert lib.rt_profile_enable(NULL, 1) == EINVAL
    assert lib.rt_last_hip_error(NULL) == 0
    out = ctypes.c_void_p()
    assert lib.rt_engine_create(0, 8, 8, 1, 0, ctypes.byref(out)) == EINVAL and not out.value
    assert lib.rt_engine_create_shared(NULL, 8, 1, ctypes.byref(out)) == EINVAL and not out.value
    lib.rt_engine_destroy(NULL)  # ignored
    b = ctypes.c_void_p()
    assert lib.rt_batcher_create(NULL, 8, 100, 1, ctypes.byref(b)) == EINVAL and not b.value
    assert lib.rt_batcher_create(P, 8, 100, 1, None) == EINVAL
    assert lib.rt_batcher_create(P, 8, -1, 1, ctypes.byref(b)) == EINVAL and not b.value   # negative wait
    assert lib.rt_batcher_create(P, 8, 100, 2, ctypes.byref(b)) == EINVAL and not b.value  # exact is 0 or 1
    t = ctypes.c_uint64(0)
    assert lib.rt_batcher_submit(NULL, P, 1, P, P, ctypes.byref(t)) == EINVAL
    assert lib.rt_batcher_wait(NULL, 1) == EINVAL
    assert lib.rt_batcher_stats(NULL, (ctypes.c_int64 * 4)()) == EINVAL
    lib.rt_batcher_destroy(NULL)  # ignored


def test_binding_rejects_bad_tensors_on_the_host():
    """The binding passes only addresses to the C ABI, so it must refuse, before
    any call, a buffer a kernel cannot use: a host tensor, the wrong dtype, a
    non-contiguous view or one too small, and queries whose width is not the
    resident depth."""
    torch = pytest.importorskip("torch")
    import top_search_resident_amd as pkg
    ok = torch.empty(8, dtype=torch.int32)
    with pytest.raises(TypeError, match="CUDA"):
        pkg._check_tensor(ok, "out_idx", torch.int32, 8, 0)          # host memory
    with pytest.raises(TypeError, match="int32"):
        pkg._check_tensor(torch.empty(8, dtype=torch.float32), "out_idx", torch.int32, 8, 0)
    with pytest.raises(TypeError, match="torch tensor"):
        pkg._check_tensor(ok.numpy(), "out_idx", torch.int32, 8, 0)
    with pytest.raises(TypeError, match="CUDA"):
        pkg._check_queries(torch.zeros((2, 16)), 16, 0)
    with pytest.raises(ValueError, match=r"\[q, d\]"):
        pkg._check_queries(torch.zeros((2, 4, 4)), 16, 0)
