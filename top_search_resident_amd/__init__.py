"""top_search_resident_amd -- exact resident top-K retrieval on AMD MI355X (gfx950).

A thin binding over the C ABI of ``libresident_topk.so`` (include/resident_topk.h).
It only marshals arguments: every step of the search runs in the library's HIP
kernels.  PyTorch supplies device memory and streams.  Importing the package does
not load the library; constructing an engine does, and fails loudly if the HIP
library is not built.

    eng = ResidentTopK(max_n=1_000_000, max_d=1024, max_k=128, max_q=32)
    eng.upload_corpus_rowmajor(corpus)              # once; host or device fp32 [n, d]
    idx, scores = eng.search_resident(queries, k)   # device fp32 [q, d] -> [q, k] each
    idx, vals = eng.topk_select(values, k)          # device int32/fp32 [n] -> [k] each
"""
import ctypes
import threading
import weakref

from . import _lib
from ._lib import ResidentTopKError, RT_DTYPE_FLOAT32, RT_DTYPE_INT32, RT_METRIC_COSINE, RT_METRIC_DOT

__all__ = ["ResidentTopK", "ResidentTopKError", "Batcher", "topk_select_noalloc"]


_torch_module = None


def _torch():
    global _torch_module
    if _torch_module is None:
        import torch
        _torch_module = torch
    return _torch_module


def _check(status, what, eng=None):
    if status != _lib.RT_OK:
        hip = _lib.load().rt_last_hip_error(eng) if eng else 0
        raise ResidentTopKError(status, what, hip)


def _check_tensor(t, name, dtype, min_numel, device):
    """Raise before anything is enqueued unless `t` is a contiguous CUDA tensor
    of `dtype` on cuda:`device` with at least `min_numel` elements: the C ABI
    receives only its address, and a kernel writing through a host address or
    past the end of a buffer faults the GPU."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    dev = t.get_device()  # -1 for a host tensor; one call instead of is_cuda and device.index
    if dev != device:
        if dev < 0:
            raise TypeError(f"{name} must be a CUDA tensor")
        raise ValueError(f"{name} is on {t.device}, the engine on cuda:{device}")
    if not t.is_contiguous():
        raise TypeError(f"{name} must be contiguous")
    if t.numel() < min_numel:
        raise ValueError(f"{name} holds {t.numel()} elements, {min_numel} needed")


def _check_queries(queries, d, device):
    """A contiguous fp32 CUDA tensor [q, d] (or [d]) on the engine's device whose
    width is the resident depth d (the C ABI reads q * d floats)."""
    torch = _torch()
    if not isinstance(queries, torch.Tensor):
        raise TypeError("queries must be a torch tensor")
    if queries.dim() == 1:
        queries = queries.view(1, -1)
    if queries.dim() != 2:
        raise ValueError("queries must be [q, d] or [d]")
    _check_tensor(queries, "queries", torch.float32, 0, device)
    if d is not None and queries.shape[1] != d:
        raise ValueError(f"queries have width {queries.shape[1]}, the resident corpus depth {d}")
    return queries


_raw_stream = None


def _stream_handle(stream, device):
    """The HIP stream to enqueue on: `stream`, or the current stream of
    `device`.  torch.cuda.current_stream() builds a Stream object, which costs
    ~2.7 us per call on MI355X hosts (most of this binding's per-call time);
    torch's own raw accessor returns the same handle in ~0.1 us."""
    global _raw_stream
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream)
    torch = _torch()
    if _raw_stream is None:
        _raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", False)
    if _raw_stream:
        return ctypes.c_void_p(_raw_stream(device))
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def topk_select_noalloc(values, k, out_idx=None, out_values=None, stream=None):
    """topk_select without an engine: the library allocates nothing (its kernels'
    scratch is a static device array per GPU).  values: a contiguous int32 or
    float32 CUDA tensor on the current device.  Returns (idx int32 [k], values
    [k]) on the device, best-first.  Calls overlapping on one GPU race on the
    shared array."""
    torch = _torch()
    lib = _lib.load()
    if not isinstance(values, torch.Tensor) or values.dtype not in (torch.int32, torch.float32):
        raise TypeError("topk_select_noalloc takes int32 or float32 tensors")
    dev = torch.cuda.current_device()
    _check_tensor(values, "values", values.dtype, 1, dev)
    k = int(k)
    if k < 1:
        raise ResidentTopKError(_lib.RT_EINVAL, f"k = {k}")
    if out_idx is None:
        out_idx = torch.empty(k, dtype=torch.int32, device=values.device)
    if out_values is None:
        out_values = torch.empty(k, dtype=values.dtype, device=values.device)
    _check_tensor(out_idx, "out_idx", torch.int32, k, dev)
    _check_tensor(out_values, "out_values", values.dtype, k, dev)
    dt = RT_DTYPE_INT32 if values.dtype == torch.int32 else RT_DTYPE_FLOAT32
    st = lib.topk_select_noalloc(ctypes.c_void_p(values.data_ptr()), dt, int(values.numel()), k,
                                 ctypes.c_void_p(out_idx.data_ptr()), ctypes.c_void_p(out_values.data_ptr()),
                                 _stream_handle(stream, dev))
    _check(st, "topk_select_noalloc")
    return out_idx, out_values


class ResidentTopK:
    """One engine: owns all device memory for a resident corpus of up to
    max_n x max_d fp32 rows, top-k up to max_k, batches up to max_q queries."""

    def __init__(self, max_n, max_d, max_k=128, max_q=1, device=0, _share=None):
        self._lib = _lib.load()
        self._h = ctypes.c_void_p()
        if _share is None:
            st = self._lib.rt_engine_create(int(max_n), int(max_d), int(max_k), int(max_q), int(device),
                                            ctypes.byref(self._h))
            _check(st, "rt_engine_create")
        else:
            st = self._lib.rt_engine_create_shared(_share._h, int(max_k), int(max_q), ctypes.byref(self._h))
            _check(st, "rt_engine_create_shared")
        self.device = int(device)
        self.max_n, self.max_d, self.max_k, self.max_q = int(max_n), int(max_d), int(max_k), int(max_q)
        # Resident depth, shared by every engine that shares the corpus (an
        # upload through any of them changes it for all); None before an upload.
        self._res = _share._res if _share is not None else {"d": None}
        self._batchers = weakref.WeakSet()  # closed before this engine is

    def shared(self, max_k=None, max_q=None):
        """A new engine that searches this engine's resident corpus (no copy) with
        scratch memory of its own, so the two can search concurrently on
        different streams.  The corpus stays allocated until every engine that
        shares it is closed."""
        return ResidentTopK(self.max_n, self.max_d, self.max_k if max_k is None else max_k,
                            self.max_q if max_q is None else max_q, self.device, _share=self)

    # -- lifecycle ---------------------------------------------------------
    def close(self):
        for b in list(getattr(self, "_batchers", ())):
            b.close()  # a batcher's dispatcher thread uses this engine
        if getattr(self, "_h", None) and self._h.value:
            self._lib.rt_engine_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _lib_resident_d(self):
        out = (ctypes.c_int64 * 7)()
        _check(self._lib.rt_engine_info(self._h, out), "rt_engine_info")
        return int(out[5]) or None

    def _outputs(self, q, k, out_idx, out_val, val_dtype, name_val, like):
        torch = _torch()
        if k < 1:
            raise ResidentTopKError(_lib.RT_EINVAL, f"k = {k}")
        if out_idx is None:
            out_idx = torch.empty((q, k) if q else (k,), dtype=torch.int32, device=like.device)
        if out_val is None:
            out_val = torch.empty((q, k) if q else (k,), dtype=val_dtype, device=like.device)
        n = max(q, 1) * k
        _check_tensor(out_idx, "out_idx", torch.int32, n, self.device)
        _check_tensor(out_val, name_val, val_dtype, n, self.device)
        return out_idx, out_val

    def info(self):
        out = (ctypes.c_int64 * 7)()
        _check(self._lib.rt_engine_info(self._h, out), "rt_engine_info")
        keys = ("max_n", "max_d", "max_k", "max_q", "resident_n", "resident_d", "device")
        return dict(zip(keys, [int(v) for v in out]))

    # -- the three calls ----------------------------------------------------
    def upload_corpus_rowmajor(self, corpus):
        """Copy an [n, d] fp32 row-major corpus (numpy array or torch tensor, host
        or device) into the engine; synchronous."""
        if hasattr(corpus, "data_ptr"):
            torch = _torch()
            if corpus.dtype != torch.float32 or not corpus.is_contiguous() or corpus.dim() != 2:
                raise TypeError("corpus must be a contiguous 2-D float32 tensor")
            ptr, (n, d) = corpus.data_ptr(), tuple(corpus.shape)
        else:
            import numpy as np
            if corpus.dtype != np.float32 or corpus.ndim != 2 or not corpus.flags.c_contiguous:
                raise TypeError("corpus must be a C-contiguous 2-D float32 array")
            ptr, (n, d) = corpus.ctypes.data, corpus.shape
        st = self._lib.upload_corpus_rowmajor(self._h, ctypes.c_void_p(ptr), int(n), int(d))
        # the library's state decides: a rejected upload keeps the previous
        # corpus, a failed copy leaves none
        self._res["d"] = self._lib_resident_d()
        _check(st, "upload_corpus_rowmajor", self._h)
        self._keep = corpus  # not needed after the synchronous copy; kept only until the next upload

    def search_resident(self, queries, k, out_idx=None, out_scores=None, stream=None, metric="dot"):
        """Exact top-k by inner product (metric="dot") or cosine similarity
        (metric="cosine").  queries: device fp32 [q, d] or [d].
        Returns (idx int32 [q, k], scores fp32 [q, k]) on the device, best-first;
        enqueued on `stream` (default: torch's current stream on the engine's device)."""
        torch = _torch()
        metrics = {"dot": RT_METRIC_DOT, "cosine": RT_METRIC_COSINE}
        if metric not in metrics:
            raise ValueError(f"metric must be one of {sorted(metrics)}")
        queries = _check_queries(queries, self._res["d"], self.device)
        q = queries.shape[0]
        out_idx, out_scores = self._outputs(q, int(k), out_idx, out_scores, torch.float32, "out_scores", queries)
        st = self._lib.search_resident_metric(self._h, ctypes.c_void_p(queries.data_ptr()), int(q), int(k),
                                              metrics[metric], ctypes.c_void_p(out_idx.data_ptr()),
                                              ctypes.c_void_p(out_scores.data_ptr()),
                                              _stream_handle(stream, self.device))
        _check(st, "search_resident", self._h)
        return out_idx, out_scores

    def enable_filtered(self):
        """Allocate the bf16 copy of the corpus and this engine's scratch for
        search_resident_filtered (once, at set-up)."""
        _check(self._lib.rt_enable_filtered(self._h), "rt_enable_filtered", self._h)

    _STORAGE = {"auto": 0, "bf16": 1, "fp8": 2}
    _PATHS = {0: None, 1: "plain", 2: "bf16", 3: "fp8", 4: "bf16_matrix"}

    def set_filter_storage(self, storage):
        """First pass of a single-query filtered search: "auto" (the plain scan
        below ~46M corpus elements, where two passes cost more than they save,
        fp8 from there on), "bf16" or "fp8".  The answers are the same."""
        if storage not in self._STORAGE:
            raise ValueError(f"storage must be one of {sorted(self._STORAGE)}")
        _check(self._lib.rt_set_filter_storage(self._h, self._STORAGE[storage]), "rt_set_filter_storage", self._h)

    def filter_path_used(self):
        """What the last search_resident_filtered call ran: "plain", "bf16",
        "fp8", "bf16_matrix" (a batch), or None."""
        return self._PATHS.get(int(self._lib.rt_filter_path_used(self._h)))

    def search_resident_filtered(self, queries, k, out_idx=None, out_scores=None, stream=None, metric="dot"):
        """Exact top-k by inner product (metric="dot") or cosine similarity
        (metric="cosine") -- for each query, the answer search_resident gives
        for that query alone -- that reads a reduced-precision copy of the
        corpus first and the fp32 rows only where their certified score bounds
        reach a certified threshold.  An inner-product batch runs one bf16
        matrix-core first pass for all of its queries."""
        torch = _torch()
        metrics = {"dot": RT_METRIC_DOT, "cosine": RT_METRIC_COSINE}
        if metric not in metrics:
            raise ValueError(f"metric must be one of {sorted(metrics)}")
        queries = _check_queries(queries, self._res["d"], self.device)
        q = queries.shape[0]
        out_idx, out_scores = self._outputs(q, int(k), out_idx, out_scores, torch.float32, "out_scores", queries)
        st = self._lib.search_resident_filtered_metric(self._h, ctypes.c_void_p(queries.data_ptr()), int(q), int(k),
                                                       metrics[metric], ctypes.c_void_p(out_idx.data_ptr()),
                                                       ctypes.c_void_p(out_scores.data_ptr()),
                                              _stream_handle(stream, self.device))
        _check(st, "search_resident_filtered", self._h)
        return out_idx, out_scores

    def topk_select(self, values, k, out_idx=None, out_values=None, stream=None):
        """Top-k of a raw device int32/fp32 1-D tensor, ties to the lower position.
        Returns (idx int32 [k], values [k]) on the device, best-first."""
        torch = _torch()
        if values.dtype == torch.int32:
            dt = RT_DTYPE_INT32
        elif values.dtype == torch.float32:
            dt = RT_DTYPE_FLOAT32
        else:
            raise TypeError("topk_select takes int32 or float32 tensors")
        _check_tensor(values, "values", values.dtype, 1, self.device)
        values = values.view(-1)
        out_idx, out_values = self._outputs(0, int(k), out_idx, out_values, values.dtype, "out_values", values)
        st = self._lib.topk_select(self._h, ctypes.c_void_p(values.data_ptr()), dt, int(values.numel()),
                                   int(k), ctypes.c_void_p(out_idx.data_ptr()),
                                   ctypes.c_void_p(out_values.data_ptr()), _stream_handle(stream, self.device))
        _check(st, "topk_select", self._h)
        return out_idx, out_values

    # -- measurement -----------------------------------------------------------
    def profile(self, on=True):
        _check(self._lib.rt_profile_enable(self._h, 1 if on else 0), "rt_profile_enable")

    def profile_read(self):
        """Device durations (ms) of the last call: (the whole call, its first
        kernel when it ran more than one -- the batched scoring kernel, or the
        first pass of a filtered search -- else 0, the rest).  The stream must
        have finished."""
        out = (ctypes.c_float * 3)()
        _check(self._lib.rt_profile_read(self._h, out), "rt_profile_read", self._h)
        return float(out[0]), float(out[1]), float(out[2])

    def read_probe(self, reps=20, stream=None):
        """Average device time (ms) of one plain streaming read of the resident
        fp32 corpus (rt_read_probe): the read ceiling that the scan is measured
        against.  Synchronises the stream; replaces the last profile."""
        out = ctypes.c_float(0.0)
        _check(self._lib.rt_read_probe(self._h, int(reps), _stream_handle(stream, self.device),
                                       ctypes.byref(out)),
               "rt_read_probe", self._h)
        return float(out.value)


class Batcher:
    """Dynamic batching of single-query searches from many threads
    (rt_batcher_*): submissions that arrive within `max_wait_us` of each other
    run as one batched search of up to `max_batch` queries on `engine`, which
    the batcher uses alone until it is closed (take engine.shared() for other
    work on the same corpus).  exact=True (the default) runs the batched
    filtered search -- every answer equals the plain single-query scan's, bit
    for bit -- and needs engine.enable_filtered() first; exact=False runs the
    plain batched search (fp32 matrix cores)."""

    def __init__(self, engine, max_batch=32, max_wait_us=200, exact=True):
        self._lib = engine._lib
        self._engine = engine  # keeps the engine open while the batcher uses it
        self._h = ctypes.c_void_p()
        st = self._lib.rt_batcher_create(engine._h, int(max_batch), int(max_wait_us), 1 if exact else 0,
                                         ctypes.byref(self._h))
        _check(st, "rt_batcher_create", engine._h)
        self.d = engine._res["d"]
        # Output (and query) arrays of every request not yet waited for: the
        # dispatcher thread writes the answers into them, so they must outlive
        # the request even if the caller drops its handle.
        self._pending = {}
        self._lock = threading.Lock()
        engine._batchers.add(self)

    def submit(self, query, k):
        """Queue one query (host fp32 [d], numpy or CPU tensor).  Returns a
        handle for wait()."""
        import numpy as np
        if hasattr(query, "data_ptr"):
            if query.device.type != "cpu":
                raise TypeError("Batcher.submit takes host queries (numpy or CPU tensor)")
            query = query.numpy()
        q = np.ascontiguousarray(query, dtype=np.float32).reshape(-1)
        if q.shape[0] != self.d:
            raise ValueError(f"query has {q.shape[0]} values, the corpus depth is {self.d}")
        k = int(k)
        if k < 1:
            raise ResidentTopKError(_lib.RT_EINVAL, f"k = {k}")
        idx = np.empty(k, dtype=np.int32)
        sc = np.empty(k, dtype=np.float32)
        ticket = ctypes.c_uint64(0)
        st = self._lib.rt_batcher_submit(self._h, q.ctypes.data, k, idx.ctypes.data, sc.ctypes.data,
                                         ctypes.byref(ticket))
        _check(st, "rt_batcher_submit")
        handle = (int(ticket.value), idx, sc, q)
        with self._lock:
            self._pending[handle[0]] = handle
        return handle

    def wait(self, handle):
        """Block until the request completes; returns (idx int32 [k], scores
        fp32 [k]) as numpy arrays, best-first."""
        ticket, idx, sc, _ = handle
        st = self._lib.rt_batcher_wait(self._h, ctypes.c_uint64(ticket))
        with self._lock:  # once wait returns, nothing writes to this request's arrays
            self._pending.pop(ticket, None)
        _check(st, "rt_batcher_wait")
        return idx, sc

    def search(self, query, k):
        """submit() + wait(): one blocking search, batched with whatever other
        threads submit meanwhile."""
        return self.wait(self.submit(query, k))

    def stats(self):
        out = (ctypes.c_int64 * 4)()
        _check(self._lib.rt_batcher_stats(self._h, out), "rt_batcher_stats")
        return dict(zip(("batches", "served", "largest_batch", "waiting"), [int(v) for v in out]))

    def close(self):
        """Serves every request still queued (their handles' arrays receive the
        answers), then frees the batcher; wait() is not available afterwards.
        No other thread may be inside submit() or wait() meanwhile."""
        if getattr(self, "_h", None) and self._h.value:
            self._lib.rt_batcher_destroy(self._h)
            self._h = ctypes.c_void_p()
        if getattr(self, "_pending", None):
            with self._lock:
                self._pending.clear()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
