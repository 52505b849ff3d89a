"""ctypes loader for libresident_topk.so (the HIP library built for gfx950).

Loading fails loudly when the library is missing: there is no CPU fallback.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libresident_topk.so")

RT_OK, RT_EINVAL, RT_ESTATE, RT_ENOMEM, RT_EHIP = 0, 1, 2, 3, 4
RT_DTYPE_INT32, RT_DTYPE_FLOAT32 = 0, 1
RT_METRIC_DOT, RT_METRIC_COSINE = 0, 1

# Every symbol include/resident_topk.h declares.
EXPORTS = (
    "rt_engine_create", "rt_engine_create_shared", "rt_engine_destroy", "upload_corpus_rowmajor", "search_resident",
    "search_resident_metric", "rt_enable_filtered", "search_resident_filtered", "topk_select", "rt_status_string", "rt_last_hip_error", "rt_profile_enable",
    "rt_profile_read", "rt_engine_info", "rt_check_create", "rt_check_upload",
    "rt_check_search", "rt_check_search_metric", "rt_check_select", "rt_filter_bounds",
    "rt_filter_bounds_batched", "rt_filter_bounds_fp8", "rt_set_filter_storage", "rt_filter_path_used",
    "rt_read_probe", "search_resident_filtered_metric", "topk_select_noalloc", "rt_cosine_score",
    "rt_filter_cosine_bounds", "rt_batcher_create", "rt_batcher_submit", "rt_batcher_wait", "rt_batcher_stats",
    "rt_batcher_destroy",
)

_lib = None


class ResidentTopKError(RuntimeError):
    def __init__(self, status, what, hip_error=0):
        self.status = status
        self.hip_error = hip_error
        msg = f"{what}: {status_string(status)} (status {status})"
        if hip_error:
            msg += f", hipError {hip_error}"
        super().__init__(msg)


def library_path():
    return LIBRARY


def load():
    """Load (once) and return the ctypes handle of libresident_topk.so."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY):
        raise ImportError(
            f"{LIBRARY} is not built; run __graft_entry__.build() (hipcc --offload-arch=gfx950)")
    lib = ctypes.CDLL(LIBRARY)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    sig = {
        "rt_engine_create": ([i64, i32, i32, i32, i32, ctypes.POINTER(vp)], ctypes.c_int),
        "rt_engine_create_shared": ([vp, i32, i32, ctypes.POINTER(vp)], ctypes.c_int),
        "rt_engine_destroy": ([vp], None),
        "upload_corpus_rowmajor": ([vp, vp, i64, i32], ctypes.c_int),
        "search_resident": ([vp, vp, i32, i32, vp, vp, vp], ctypes.c_int),
        "search_resident_metric": ([vp, vp, i32, i32, i32, vp, vp, vp], ctypes.c_int),
        "rt_enable_filtered": ([vp], ctypes.c_int),
        "search_resident_filtered": ([vp, vp, i32, i32, vp, vp, vp], ctypes.c_int),
        "search_resident_filtered_metric": ([vp, vp, i32, i32, i32, vp, vp, vp], ctypes.c_int),
        "topk_select": ([vp, vp, i32, i64, i32, vp, vp, vp], ctypes.c_int),
        "topk_select_noalloc": ([vp, i32, i64, i32, vp, vp, vp], ctypes.c_int),
        "rt_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "rt_last_hip_error": ([vp], i32),
        "rt_profile_enable": ([vp, i32], ctypes.c_int),
        "rt_profile_read": ([vp, ctypes.POINTER(ctypes.c_float)], ctypes.c_int),
        "rt_read_probe": ([vp, i32, vp, ctypes.POINTER(ctypes.c_float)], ctypes.c_int),
        "rt_engine_info": ([vp, ctypes.POINTER(i64)], ctypes.c_int),
        "rt_check_create": ([i64, i32, i32, i32], ctypes.c_int),
        "rt_check_upload": ([i64, i32, vp, i64, i32], ctypes.c_int),
        "rt_check_search": ([i32, i32, i64, vp, i32, i32, vp, vp], ctypes.c_int),
        "rt_check_search_metric": ([i32, i32, i64, vp, i32, i32, i32, vp, vp], ctypes.c_int),
        "rt_check_select": ([i32, vp, i32, i64, i32, vp, vp], ctypes.c_int),
        "rt_filter_bounds": ([i32, ctypes.POINTER(ctypes.c_float)], ctypes.c_int),
        "rt_filter_bounds_batched": ([i32, ctypes.POINTER(ctypes.c_float)], ctypes.c_int),
        "rt_filter_bounds_fp8": ([i32, ctypes.POINTER(ctypes.c_float)], ctypes.c_int),
        "rt_set_filter_storage": ([vp, i32], ctypes.c_int),
        "rt_filter_path_used": ([vp], ctypes.c_int32),
        "rt_cosine_score": ([ctypes.c_float, ctypes.c_float, ctypes.c_float], ctypes.c_float),
        "rt_filter_cosine_bounds": ([i32, ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                     ctypes.POINTER(ctypes.c_float)], ctypes.c_int),
        "rt_batcher_create": ([vp, i32, i32, i32, ctypes.POINTER(vp)], ctypes.c_int),
        "rt_batcher_submit": ([vp, vp, i32, vp, vp, ctypes.POINTER(ctypes.c_uint64)], ctypes.c_int),
        "rt_batcher_wait": ([vp, ctypes.c_uint64], ctypes.c_int),
        "rt_batcher_stats": ([vp, ctypes.POINTER(i64)], ctypes.c_int),
        "rt_batcher_destroy": ([vp], None),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def status_string(status):
    try:
        return load().rt_status_string(int(status)).decode()
    except ImportError:
        return str(status)


def filter_bounds(d):
    """(cb, delta) of search_resident_filtered's single-query bound at depth d
    (host-only)."""
    out = (ctypes.c_float * 2)()
    st = load().rt_filter_bounds(int(d), out)
    if st != RT_OK:
        raise ResidentTopKError(st, "rt_filter_bounds")
    return float(out[0]), float(out[1])


def filter_bounds_fp8(d):
    """(cr, cx, delta) of the fp8 first pass's bound at depth d (host-only)."""
    out = (ctypes.c_float * 3)()
    st = load().rt_filter_bounds_fp8(int(d), out)
    if st != RT_OK:
        raise ResidentTopKError(st, "rt_filter_bounds_fp8")
    return float(out[0]), float(out[1]), float(out[2])


def filter_bounds_batched(d):
    """(cr, cx, delta) of the batched first pass's bound at depth d (host-only)."""
    out = (ctypes.c_float * 3)()
    st = load().rt_filter_bounds_batched(int(d), out)
    if st != RT_OK:
        raise ResidentTopKError(st, "rt_filter_bounds_batched")
    return float(out[0]), float(out[1]), float(out[2])
