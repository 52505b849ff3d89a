"""Helpers shared by the GPU parity tests: the acceptance rules for float
retrieval and exact top-K, applied to HIP results against the CPU oracle."""
import numpy as np

REL_TOL = 1e-4  # float retrieval: scores within 1e-4 relative of the oracle
# Relative error is ill-conditioned for scores near 0, which any fp32 dot product
# carries with an absolute error of its own.  The relative denominator is
# therefore floored at 1% of the Cauchy-Schwarz bound |x| |q| of that row's
# score (1e-6 absolute for unit vectors).  At the workloads' k-th scores
# (>= 0.09 for unit vectors) the floor never binds.
SCALE_FLOOR = 0.01


def _rel_ok(g, o, tol=REL_TOL, scale=None):
    """|g - o| <= tol * max(|o|, SCALE_FLOOR * scale); infinite values (the
    cosine metric's -inf for a zero norm) must be equal."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    den = np.abs(o)
    if scale is not None:
        den = np.maximum(den, SCALE_FLOOR * scale)
    with np.errstate(invalid="ignore"):
        close = np.abs(g - o) <= tol * np.maximum(den, 1e-30)
    inf = np.isinf(g) | np.isinf(o)
    return np.where(inf, g == o, close)


def cs_bound(rows, query):
    """|x| |q| for each row (fp64): the largest |score| the row can have."""
    return np.linalg.norm(rows.astype(np.float64), axis=1) * np.linalg.norm(query.astype(np.float64))


def oracle_scores(oracle_mod, rows, query, metric="dot"):
    """The oracle's fp64 scores of `rows` for one query under `metric`."""
    if metric == "cosine":
        return oracle_mod.cosine_scores(rows, query)
    return oracle_mod.scores(rows, query)


def score_scale(rows, query, metric="dot"):
    """Largest |score| each row can have: |x| |q| for the inner product, 1 for
    cosine."""
    if metric == "cosine":
        return np.ones(rows.shape[0])
    return cs_bound(rows, query)


def check_retrieval(g_idx, g_sc, o_idx, o_sc, corpus, query, oracle_mod, tol=REL_TOL, metric="dot"):
    """Float retrieval acceptance for one query under `metric` ("dot" or
    "cosine").

    R1  the GPU list is sorted under the comparator on its own fp32 scores;
    R2  each GPU score is within tol of the oracle's score of the same row and
        of the oracle's score at the same rank;
    R3  rows in the symmetric difference of the two index sets have oracle
        scores within tol of the oracle's k-th score (boundary near-ties);
    R4  indices are distinct and in range.
    """
    g_idx = np.asarray(g_idx).astype(np.int64)
    g_sc = np.asarray(g_sc).astype(np.float32)
    k = o_idx.shape[0]
    n = corpus.shape[0]
    assert g_idx.shape == (k,) and g_sc.shape == (k,)
    # R4
    assert np.all((g_idx >= 0) & (g_idx < n)), "index out of range"
    assert np.unique(g_idx).size == k, "duplicate indices"
    # R1
    for j in range(k - 1):
        a, b = g_sc[j], g_sc[j + 1]
        assert a > b or (a == b and g_idx[j] < g_idx[j + 1]), f"not sorted at {j}"
    # R2
    o_of_g = oracle_scores(oracle_mod, corpus[g_idx], query, metric)
    scale_g = score_scale(corpus[g_idx], query, metric)
    scale_o = score_scale(corpus[o_idx.astype(np.int64)], query, metric)
    assert np.all(_rel_ok(g_sc.astype(np.float64), o_of_g, tol, scale_g)), \
        "score differs from the oracle's score of that row"
    assert np.all(_rel_ok(g_sc.astype(np.float64), o_sc, tol, np.maximum(scale_g, scale_o))), \
        "score differs from the oracle's score at that rank"
    # R3
    diff = np.setxor1d(g_idx, o_idx.astype(np.int64))
    if diff.size:
        o_k = o_sc[-1]
        o_diff = oracle_scores(oracle_mod, corpus[diff], query, metric)
        assert np.all(_rel_ok(o_diff, np.full_like(o_diff, o_k), tol, scale_o[-1])), \
            f"index sets differ away from the k-th boundary: {diff[:8]}"


def check_exact_topk_property(g_idx, g_val, values):
    """Exactness of a raw top-k from properties that pin it uniquely: the list is
    sorted under the comparator, indices are distinct and hold the returned
    values, and exactly k-1 elements of the whole array beat the k-th entry."""
    g_idx = np.asarray(g_idx).astype(np.int64)
    g_val = np.asarray(g_val)
    k = g_idx.shape[0]
    v = values
    assert np.unique(g_idx).size == k
    assert np.array_equal(v[g_idx].view(np.uint32), g_val.view(np.uint32))
    if v.dtype == np.float32:
        key = v.astype(np.float64)
        gk = g_val.astype(np.float64)
    else:
        key = v.astype(np.int64)
        gk = g_val.astype(np.int64)
    for j in range(k - 1):
        assert gk[j] > gk[j + 1] or (gk[j] == gk[j + 1] and g_idx[j] < g_idx[j + 1]), j
    last_v, last_i = gk[-1], g_idx[-1]
    better = np.count_nonzero(key > last_v) + np.count_nonzero(key[:last_i] == last_v)
    assert better == k - 1, f"{better} elements beat the k-th entry (expected {k - 1})"
