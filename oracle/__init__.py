"""CPU oracle for exact resident top-K -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this package.  The product path (``top_search_resident_amd``)
never imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (see its header for the definitions and
the passages of the pages they follow); this module only marshals numpy arrays
through ctypes.  Every function here is pinned by ``tests/test_oracle_pins.py``
against facts that do not come from the oracle itself (exact rational brute
force, closed forms, invariants, a library sort, hand-worked fixtures).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_c_i64 = ctypes.c_int64
_ptr = ctypes.c_void_p


def _ptr_of(a):
    return ctypes.c_void_p(a.ctypes.data)


class Oracle:
    """ctypes view of one compiled oracle library (the real one, or a mutant
    copy built by the mutation tests)."""

    def __init__(self, path=None):
        if path is None:
            path = _build.LIBRARY
            if not os.path.exists(path):
                _build.build(quiet=True)
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_scores.argtypes = [_ptr, _c_i64, _c_i64, _ptr, _ptr]
        lib.oracle_search.argtypes = [_ptr, _c_i64, _c_i64, _ptr, _c_i64, _c_i64, _ptr, _ptr]
        lib.oracle_cosine_scores.argtypes = [_ptr, _c_i64, _c_i64, _ptr, _ptr]
        lib.oracle_search_metric.argtypes = [_ptr, _c_i64, _c_i64, _ptr, _c_i64, _c_i64, ctypes.c_int32,
                                             _ptr, _ptr]
        lib.oracle_topk_i32.argtypes = [_ptr, _c_i64, _c_i64, _ptr, _ptr]
        lib.oracle_topk_f32.argtypes = [_ptr, _c_i64, _c_i64, _ptr, _ptr]
        for f in (lib.oracle_scores, lib.oracle_search, lib.oracle_topk_i32, lib.oracle_topk_f32,
                  lib.oracle_cosine_scores, lib.oracle_search_metric):
            f.restype = ctypes.c_int
        self.lib = lib

    def num_threads(self):
        return int(self.lib.oracle_num_threads())

    def scores(self, corpus, query):
        """fp64 inner products of every corpus row with one query, shape (n,)."""
        corpus = np.ascontiguousarray(corpus, dtype=np.float32)
        query = np.ascontiguousarray(query, dtype=np.float32).reshape(-1)
        n, d = corpus.shape
        if query.shape[0] != d:
            raise ValueError("query length must equal corpus width")
        out = np.empty(n, dtype=np.float64)
        rc = self.lib.oracle_scores(_ptr_of(corpus), n, d, _ptr_of(query), _ptr_of(out))
        if rc:
            raise RuntimeError(f"oracle_scores failed ({rc})")
        return out

    def cosine_scores(self, corpus, query):
        """fp64 cosine similarity of every corpus row with one query, shape (n,);
        -inf where a norm is zero."""
        corpus = np.ascontiguousarray(corpus, dtype=np.float32)
        query = np.ascontiguousarray(query, dtype=np.float32).reshape(-1)
        n, d = corpus.shape
        if query.shape[0] != d:
            raise ValueError("query length must equal corpus width")
        out = np.empty(n, dtype=np.float64)
        rc = self.lib.oracle_cosine_scores(_ptr_of(corpus), n, d, _ptr_of(query), _ptr_of(out))
        if rc:
            raise RuntimeError(f"oracle_cosine_scores failed ({rc})")
        return out

    def search(self, corpus, queries, k, metric=0):
        """Exact top-k for each query; metric 0 = inner product, 1 = cosine.

        Returns (idx int32 [q, k], score float64 [q, k]), best-first, ties by
        lower index."""
        corpus = np.ascontiguousarray(corpus, dtype=np.float32)
        queries = np.ascontiguousarray(queries, dtype=np.float32)
        if queries.ndim == 1:
            queries = queries.reshape(1, -1)
        n, d = corpus.shape
        q = queries.shape[0]
        if queries.shape[1] != d:
            raise ValueError("query width must equal corpus width")
        idx = np.empty((q, k), dtype=np.int32)
        sc = np.empty((q, k), dtype=np.float64)
        if metric == 0:
            rc = self.lib.oracle_search(_ptr_of(corpus), n, d, _ptr_of(queries), q, k,
                                        _ptr_of(idx), _ptr_of(sc))
        else:
            rc = self.lib.oracle_search_metric(_ptr_of(corpus), n, d, _ptr_of(queries), q, k, int(metric),
                                               _ptr_of(idx), _ptr_of(sc))
        if rc:
            raise RuntimeError(f"oracle_search failed ({rc})")
        return idx, sc

    def topk(self, values, k):
        """K largest of a 1-D int32 or float32 array, ties to lower index.

        Returns (idx int32 [k], values [k] with the input's dtype and bits)."""
        values = np.ascontiguousarray(values)
        n = values.shape[0]
        idx = np.empty(k, dtype=np.int32)
        if values.dtype == np.int32:
            out = np.empty(k, dtype=np.int32)
            rc = self.lib.oracle_topk_i32(_ptr_of(values), n, k, _ptr_of(idx), _ptr_of(out))
        elif values.dtype == np.float32:
            out = np.empty(k, dtype=np.float32)
            rc = self.lib.oracle_topk_f32(_ptr_of(values), n, k, _ptr_of(idx), _ptr_of(out))
        else:
            raise TypeError("oracle topk takes int32 or float32 arrays")
        if rc:
            raise RuntimeError(f"oracle_topk failed ({rc})")
        return idx, out


_default = None


def default():
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def scores(corpus, query):
    return default().scores(corpus, query)


def search(corpus, queries, k, metric=0):
    return default().search(corpus, queries, k, metric)


def cosine_scores(corpus, query):
    return default().cosine_scores(corpus, query)


def topk(values, k):
    return default().topk(values, k)


def num_threads():
    return default().num_threads()
