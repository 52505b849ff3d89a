"""Seeded synthetic inputs for exact resident top-K.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no scoring, no ordering, no selection).  The tests feed the
same arrays to the HIP path and to the CPU oracle, and the benchmark uses the
same recipes.

Recipe (all generators are numpy PCG64 seeded from SeedSequence([1, config,
stream, chunk]); base seed 1 as in "GPU-Resident Top-K for Agentic RAG",
section 5, which benchmarks seeded Gaussian, L2-normalised embeddings):

* embeddings: iid N(0,1) fp32 entries, each row divided by its L2 norm computed
  in fp64, then cast back to fp32;
* near-tie planting (the mid-scale sweep): an anchor query q0 is drawn; a seeded
  0.5% subset of corpus rows is replaced by normalise(q0 + 0.01 z); query 0 is
  q0 and later queries are normalise(q0 + 0.01 z');
* raw int32 arrays: uniform over [-2^31, 2^31); a seeded 1% of positions are
  overwritten with the value found at another uniformly drawn position, which
  creates exact ties.

Large arrays are generated in fixed row chunks, each with its own child seed,
so the result does not depend on the number of worker threads.
"""
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

BASE_SEED = 1
STREAM_CORPUS, STREAM_QUERIES, STREAM_PLANT_POS, STREAM_PLANT_NOISE, STREAM_DUP = 0, 1, 2, 3, 4
CHUNK_ROWS = 8192

# The five workloads.  Sizes follow the benchmark configurations of the pages'
# method (resident retrieval at several corpus sizes, a raw int32 top-K, and a
# batched large-K retrieval).
WORKLOADS = {
    "c1_10k_384": dict(config_id=1, n=10_000, d=384, ks=(8,), queries=1, kind="retrieval"),
    "c2_50k_768": dict(config_id=2, n=50_000, d=768, ks=(8, 32), queries=1000, kind="retrieval",
                       planted_fraction=0.005, planted_sigma=0.01),
    "c2_100k_768": dict(config_id=2, n=100_000, d=768, ks=(8, 32), queries=1000, kind="retrieval",
                        planted_fraction=0.005, planted_sigma=0.01),
    "c3_1m_1024": dict(config_id=3, n=1_000_000, d=1024, ks=(8, 32, 100), queries=1000,
                       kind="retrieval"),
    "c4_1e8_int32": dict(config_id=4, n=100_000_000, ks=(20, 50), kind="int32",
                         dup_fraction=0.01),
    "c5_q32_500k_768": dict(config_id=5, n=500_000, d=768, ks=(100, 1024), queries=32,
                            kind="retrieval", batch=32),
}


def _rng(config_id, stream, chunk=0):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [BASE_SEED, int(config_id), int(stream), int(chunk)])))


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normalise_rows(x):
    """Divide each row by its fp64 L2 norm; returns fp32 (input generation only)."""
    x64 = np.asarray(x, dtype=np.float64)
    norms = np.sqrt(np.einsum("ij,ij->i", x64, x64))
    norms[norms == 0.0] = 1.0
    return (x64 / norms[:, None]).astype(np.float32)


def gaussian_rows(n, d, config_id, stream=STREAM_CORPUS, normalise=True, out=None):
    """n x d fp32 rows, iid N(0,1), optionally L2-normalised, chunk-seeded."""
    if out is None:
        out = np.empty((n, d), dtype=np.float32)
    chunks = [(c, c * CHUNK_ROWS, min(n, (c + 1) * CHUNK_ROWS)) for c in range((n + CHUNK_ROWS - 1) // CHUNK_ROWS)]

    def work(item):
        c, lo, hi = item
        block = _rng(config_id, stream, c).standard_normal((hi - lo, d), dtype=np.float32)
        out[lo:hi] = normalise_rows(block) if normalise else block

    if len(chunks) > 1:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, chunks))
    else:
        for item in chunks:
            work(item)
    return out


def scaled_rows(n, d, config_id, stream=STREAM_CORPUS, sigma=1.0):
    """n x d fp32 rows: iid N(0,1) entries, each row multiplied by its own
    log-normal factor exp(sigma * N(0,1)), so row lengths vary widely (inputs for
    the cosine metric, whose ranking then differs from the inner product's)."""
    rows = gaussian_rows(n, d, config_id, stream, normalise=False)
    scale = np.exp(sigma * _rng(config_id, stream, 1 << 20).standard_normal(n)).astype(np.float32)
    rows *= scale[:, None]
    return rows


def retrieval_inputs(name, n=None, d=None, queries=None):
    """(corpus fp32 [n, d], queries fp32 [q, d]) for a retrieval workload.

    ``n``/``d``/``queries`` override the workload's sizes (smaller parity cases
    keep the same distribution and planting recipe)."""
    w = WORKLOADS[name]
    n = w["n"] if n is None else n
    d = w["d"] if d is None else d
    q = w["queries"] if queries is None else queries
    cid = w["config_id"]
    corpus = gaussian_rows(n, d, cid, STREAM_CORPUS)
    frac = w.get("planted_fraction")
    if frac:
        sigma = w["planted_sigma"]
        qrng = _rng(cid, STREAM_QUERIES)
        q0 = normalise_rows(qrng.standard_normal((1, d), dtype=np.float32))[0]
        m = int(round(frac * n))
        pos = _rng(cid, STREAM_PLANT_POS).choice(n, size=m, replace=False)
        noise = _rng(cid, STREAM_PLANT_NOISE).standard_normal((m, d), dtype=np.float32)
        corpus[pos] = normalise_rows(q0[None, :].astype(np.float64) + sigma * noise.astype(np.float64))
        qs = np.empty((q, d), dtype=np.float32)
        qs[0] = q0
        if q > 1:
            z = qrng.standard_normal((q - 1, d), dtype=np.float32)
            qs[1:] = normalise_rows(q0[None, :].astype(np.float64) + sigma * z.astype(np.float64))
    else:
        qs = gaussian_rows(q, d, cid, STREAM_QUERIES)
    return corpus, qs


def int32_values(n=None, dup_fraction=None, config_id=4):
    """Uniform int32 over [-2^31, 2^31) with a fraction of positions overwritten by
    the value at another uniformly drawn position (exact duplicates)."""
    w = WORKLOADS["c4_1e8_int32"]
    n = w["n"] if n is None else n
    dup_fraction = w["dup_fraction"] if dup_fraction is None else dup_fraction
    vals = _rng(config_id, STREAM_CORPUS).integers(-(2 ** 31), 2 ** 31, size=n, dtype=np.int32)
    m = int(round(dup_fraction * n))
    if m:
        drng = _rng(config_id, STREAM_DUP)
        # distinct targets in draw order (oversample, then keep the first m unique)
        cand = drng.integers(0, n, size=m + m // 8 + 16, dtype=np.int64)
        _, first = np.unique(cand, return_index=True)
        targets = cand[np.sort(first)][:m]
        if targets.shape[0] < m:  # pragma: no cover - tiny n
            targets = drng.choice(n, size=m, replace=False)
        sources = drng.integers(0, n, size=targets.shape[0], dtype=np.int64)
        vals[targets] = vals[sources].copy()
    return vals


def float32_values(n, config_id=6, stream=STREAM_CORPUS):
    """iid N(0,1) fp32 values (raw-array float top-K cases)."""
    return _rng(config_id, stream).standard_normal(n, dtype=np.float32)


def small_int_matrix(n, d, lo=-3, hi=3, config_id=7, stream=STREAM_CORPUS):
    """Integer-valued fp32 matrix with entries in [lo, hi].  With entries in
    [-3, 3] every partial dot product is an integer of magnitude <= 9*D, exact in
    fp32 while 9*D < 2^24, which makes ties exact."""
    return _rng(config_id, stream).integers(lo, hi + 1, size=(n, d)).astype(np.float32)
