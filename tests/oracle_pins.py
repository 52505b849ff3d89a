"""Pins for the CPU oracle: facts that do not come from the oracle itself.

Each check takes an ``oracle.Oracle`` instance and raises AssertionError when
the oracle disagrees with something the pages or the mathematics fix:

* exact rational arithmetic (``fractions.Fraction``) and brute-force rank
  counting on tiny inputs -- pins the inner product and the ordering rule;
* closed forms (one-hot corpus, query contained in the corpus, all-equal,
  monotone arrays) -- pin the direction of the order and the tie rule;
* a library routine (numpy ``lexsort`` on int64-widened keys) for the raw int32
  top-K;
* hand-worked fixtures in ``tests/golden/hand_worked.json``;
* invariants (sortedness, distinctness, completeness), permutation invariance,
  and the exactness of the two-stage (per-block then merge) decomposition;
* cosine mode: exact rationals on integer vectors with integer norms, scale
  invariance, the zero-norm rule, and a 50-digit decimal evaluation.

``tests/test_oracle_mutants.py`` plants plausible mistakes in copies of the
oracle and checks that at least one of these pins fails for each.
"""
from fractions import Fraction
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_worked.json")
INT32_MIN, INT32_MAX = -(2 ** 31), 2 ** 31 - 1


def _better(sa, ia, sb, ib):
    """The pages' comparator, stated once more for the brute-force checks."""
    return sa > sb or (sa == sb and ia < ib)


def _exact_dot(row, q):
    return sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(row, q)), Fraction(0))


# ------------------------------------------------------------------ scoring

def pin_scores_exact_rational(o, seed=11):
    """fp64 scores lie within the fp64 summation bound of the exact rational
    inner product (every fp32*fp32 product is exact in fp64)."""
    rng = np.random.default_rng(seed)
    for n, d in ((40, 7), (17, 1), (9, 33)):
        corpus = rng.standard_normal((n, d)).astype(np.float32)
        q = rng.standard_normal(d).astype(np.float32)
        got = o.scores(corpus, q)
        for i in range(n):
            exact = _exact_dot(corpus[i], q)
            mag = sum(abs(float(a) * float(b)) for a, b in zip(corpus[i], q))
            bound = d * 2.0 ** -52 * mag + 1e-300
            assert abs(Fraction(got[i]) - exact) <= Fraction(bound), (n, d, i, got[i], float(exact))


def pin_search_rank_counting(o, seed=12):
    """On tiny random inputs the oracle's order equals the order obtained by
    counting, with exact rationals, how many rows beat each row."""
    rng = np.random.default_rng(seed)
    for n, d in ((48, 6), (31, 3), (5, 11)):
        corpus = rng.standard_normal((n, d)).astype(np.float32)
        q = rng.standard_normal(d).astype(np.float32)
        exact = [_exact_dot(corpus[i], q) for i in range(n)]
        rank = [sum(1 for j in range(n) if _better(exact[j], j, exact[i], i)) for i in range(n)]
        by_rank = [None] * n
        for i, r in enumerate(rank):
            by_rank[r] = i
        for k in (1, 2, n // 2 or 1, n):
            idx, sc = o.search(corpus, q[None, :], k)
            assert list(idx[0]) == by_rank[:k], (n, d, k, list(idx[0]), by_rank[:k])
            for r in range(k):
                assert abs(Fraction(sc[0, r]) - exact[by_rank[r]]) <= Fraction(1e-12), (n, d, k, r)


def pin_search_integer_ties(o, seed=13):
    """Integer-valued inputs make every score exact and produce many exact ties;
    the oracle must return exactly the rows of rank 0..k-1 (rank = number of
    rows that beat it under the comparator), with exact scores."""
    rng = np.random.default_rng(seed)
    for n, d in ((300, 16), (64, 2), (257, 5)):
        corpus = rng.integers(-3, 4, size=(n, d)).astype(np.float32)
        q = rng.integers(-3, 4, size=d).astype(np.float32)
        s = corpus.astype(np.int64) @ q.astype(np.int64)
        ii = np.arange(n)
        beats = (s[:, None] > s[None, :]) | ((s[:, None] == s[None, :]) & (ii[:, None] < ii[None, :]))
        rank = beats.sum(axis=0)
        order = np.empty(n, dtype=np.int64)
        order[rank] = ii
        for k in (1, 7, n):
            idx, sc = o.search(corpus, q[None, :], k)
            assert np.array_equal(idx[0], order[:k]), (n, d, k)
            assert np.array_equal(sc[0], s[order[:k]].astype(np.float64)), (n, d, k)


def pin_onehot_closed_form(o, seed=14):
    """Corpus = identity: score of row i is q[i] exactly.  With q[i] = (n - p[i]) / n
    for a permutation p, the row of rank r is the i with p[i] = r."""
    rng = np.random.default_rng(seed)
    for n in (64, 37):
        p = rng.permutation(n)
        q = ((n - p) / n).astype(np.float32)
        corpus = np.eye(n, dtype=np.float32)
        inv = np.argsort(p)  # inv[r] = i with p[i] = r
        for k in (1, 5, n):
            idx, sc = o.search(corpus, q[None, :], k)
            assert np.array_equal(idx[0], inv[:k]), (n, k)
            assert np.array_equal(sc[0], q[inv[:k]].astype(np.float64)), (n, k)


def pin_query_in_corpus(o, seed=15):
    """A unit-norm query that is itself a corpus row scores ~1 there and ranks
    first (every other unit row scores < 1 by Cauchy-Schwarz)."""
    rng = np.random.default_rng(seed)
    n, d = 2000, 64
    corpus = rng.standard_normal((n, d))
    corpus /= np.linalg.norm(corpus, axis=1, keepdims=True)
    corpus = corpus.astype(np.float32)
    j = 1234
    idx, sc = o.search(corpus, corpus[j][None, :], 3)
    assert idx[0, 0] == j
    assert abs(sc[0, 0] - 1.0) < 1e-6
    assert sc[0, 1] < sc[0, 0]


# ------------------------------------------------------------------ raw top-K

def pin_topk_i32_lexsort(o, seed=16):
    """Raw int32 top-K equals numpy lexsort on int64-widened (-value, index)."""
    rng = np.random.default_rng(seed)
    n = 200_000
    v = rng.integers(INT32_MIN, INT32_MAX + 1, size=n, dtype=np.int64)
    v[rng.integers(0, n, 50)] = INT32_MAX
    v[rng.integers(0, n, 50)] = INT32_MIN
    dup = rng.integers(0, n, 2000)
    v[dup] = v[rng.integers(0, n, 2000)]
    v = v.astype(np.int32)
    order = np.lexsort((np.arange(n), -v.astype(np.int64)))
    for k in (1, 20, 50, 1024):
        idx, vals = o.topk(v, k)
        assert np.array_equal(idx, order[:k]), k
        assert np.array_equal(vals, v[order[:k]]), k


def pin_topk_i32_special(o):
    n = 1000
    idx, _ = o.topk(np.full(n, 7, dtype=np.int32), 10)
    assert np.array_equal(idx, np.arange(10)), "all-equal must return the lowest indices"
    idx, _ = o.topk(np.arange(n, 0, -1).astype(np.int32), 10)
    assert np.array_equal(idx, np.arange(10)), "descending array: first k positions"
    idx, _ = o.topk(np.arange(n).astype(np.int32), 10)
    assert np.array_equal(idx, np.arange(n - 1, n - 11, -1)), "ascending array: last k positions"
    idx, vals = o.topk(np.full(n, INT32_MIN, dtype=np.int32), 3)
    assert np.array_equal(idx, [0, 1, 2]) and np.all(vals == INT32_MIN)
    v = np.array([INT32_MIN, -1, 0, 1, INT32_MAX], dtype=np.int32)
    idx, _ = o.topk(v, 5)
    assert np.array_equal(idx, [4, 3, 2, 1, 0]), "int32 extremes must order without overflow"


def pin_topk_f32_lexsort(o, seed=17):
    """Raw fp32 top-K on values without signed zeros equals lexsort on fp64."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(100_000).astype(np.float32)
    v[rng.integers(0, v.size, 500)] = v[rng.integers(0, v.size, 500)]
    order = np.lexsort((np.arange(v.size), -v.astype(np.float64)))
    for k in (1, 33, 1024):
        idx, vals = o.topk(v, k)
        assert np.array_equal(idx, order[:k]), k
        assert np.array_equal(vals.view(np.uint32), v[order[:k]].view(np.uint32)), k


# ------------------------------------------------------------------ golden

def pin_golden(o, path=GOLDEN):
    with open(path) as f:
        g = json.load(f)
    for case in g["retrieval"]:
        corpus = np.array(case["corpus"], dtype=np.float32)
        q = np.array(case["query"], dtype=np.float32)
        idx, sc = o.search(corpus, q[None, :], case["k"])
        assert list(idx[0]) == case["expected_idx"], case["note"]
        assert list(sc[0]) == [float(x) for x in case["expected_score"]], case["note"]
    for case in g["topk_int32"]:
        v = np.array(case["values"], dtype=np.int64).astype(np.int32)
        idx, vals = o.topk(v, case["k"])
        assert list(idx) == case["expected_idx"], case["note"]
        assert np.array_equal(vals, v[case["expected_idx"]])
    for case in g["topk_float32"]:
        v = np.array([float(x) for x in case["values"]], dtype=np.float32)
        idx, vals = o.topk(v, case["k"])
        assert list(idx) == case["expected_idx"], case["note"]
        assert np.array_equal(vals.view(np.uint32), v[case["expected_idx"]].view(np.uint32)), \
            "returned values must keep their own bits (e.g. the sign of -0.0)"


# ------------------------------------------------------------------ invariants

def check_topk_invariants(idx, scores, all_scores):
    """Sorted under the comparator, distinct, in range, and every row left out
    is beaten by the k-th returned pair."""
    n = all_scores.shape[0]
    k = idx.shape[0]
    assert np.all((idx >= 0) & (idx < n))
    assert np.unique(idx).size == k
    assert np.array_equal(scores, all_scores[idx])
    for r in range(k - 1):
        assert _better(scores[r], idx[r], scores[r + 1], idx[r + 1]), r
    mask = np.ones(n, dtype=bool)
    mask[idx] = False
    rest = np.nonzero(mask)[0]
    sk, ik = scores[-1], idx[-1]
    bad = (all_scores[rest] > sk) | ((all_scores[rest] == sk) & (rest < ik))
    assert not bad.any(), "a left-out row beats the k-th returned row"


def pin_invariants(o, seed=18):
    rng = np.random.default_rng(seed)
    corpus = rng.standard_normal((5000, 24)).astype(np.float32)
    qs = rng.standard_normal((3, 24)).astype(np.float32)
    for k in (1, 10, 100):
        idx, sc = o.search(corpus, qs, k)
        for qi in range(3):
            check_topk_invariants(idx[qi], sc[qi], o.scores(corpus, qs[qi]))
    v = rng.integers(-50, 50, size=20000).astype(np.int32)
    idx, vals = o.topk(v, 300)
    check_topk_invariants(idx, vals.astype(np.int64), v.astype(np.int64))


def pin_permutation_invariance(o, seed=19):
    """Permuting rows and mapping the answer back gives the same rows on
    tie-free data, and the same score sequence when there are ties."""
    rng = np.random.default_rng(seed)
    corpus = rng.standard_normal((3000, 16)).astype(np.float32)
    q = rng.standard_normal(16).astype(np.float32)
    perm = rng.permutation(3000)
    a_idx, a_sc = o.search(corpus, q[None, :], 50)
    b_idx, b_sc = o.search(corpus[perm], q[None, :], 50)
    assert np.array_equal(perm[b_idx[0]], a_idx[0])
    assert np.array_equal(a_sc, b_sc)
    ti = rng.integers(-2, 3, size=(3000, 4)).astype(np.float32)
    tq = rng.integers(-2, 3, size=4).astype(np.float32)
    a_idx, a_sc = o.search(ti, tq[None, :], 200)
    b_idx, b_sc = o.search(ti[perm], tq[None, :], 200)
    assert np.array_equal(a_sc, b_sc)
    v = rng.integers(-5, 5, size=4000).astype(np.int32)
    p2 = rng.permutation(4000)
    ai, av = o.topk(v, 100)
    bi, bv = o.topk(v[p2], 100)
    assert np.array_equal(av, bv)


def pin_two_stage_decomposition(o, seed=20):
    """Top-k of the union of per-block top-k lists equals the global top-k for
    any partition of the rows into blocks (the exactness of per-block partial
    top-K followed by a multi-way merge)."""
    rng = np.random.default_rng(seed)
    n, d, k = 4000, 12, 25
    corpus = rng.integers(-2, 3, size=(n, d)).astype(np.float32)  # tie-heavy
    q = rng.integers(-2, 3, size=d).astype(np.float32)
    g_idx, g_sc = o.search(corpus, q[None, :], k)
    for trial in range(5):
        cuts = np.sort(rng.choice(np.arange(1, n), size=rng.integers(1, 40), replace=False))
        bounds = np.concatenate([[0], cuts, [n]])
        pool = []
        for lo, hi in zip(bounds[:-1], bounds[1:]):
            kk = min(k, hi - lo)
            bi, bs = o.search(corpus[lo:hi], q[None, :], kk)
            pool += [(bs[0, r], lo + bi[0, r]) for r in range(kk)]
        pool.sort(key=lambda t: (-t[0], t[1]))
        assert [i for _, i in pool[:k]] == list(g_idx[0]), trial
        assert [s for s, _ in pool[:k]] == list(g_sc[0]), trial


# ------------------------------------------------------------------ cosine mode

def _norm_vectors():
    """Integer vectors of length 4 whose L2 norms are integers, with every sign
    pattern and a few coordinate orders."""
    base = [(1, 2, 2, 0), (2, 3, 6, 0), (1, 4, 8, 0), (4, 4, 7, 0), (2, 6, 9, 0), (6, 6, 7, 0),
            (3, 4, 12, 0), (0, 0, 0, 5), (1, 1, 1, 1), (2, 2, 1, 4), (0, 3, 4, 0), (2, 4, 5, 6)]
    out = []
    for v in base:
        for signs in ((1, 1, 1, 1), (-1, 1, -1, 1), (1, -1, 1, -1), (-1, -1, -1, -1)):
            for perm in ((0, 1, 2, 3), (3, 2, 1, 0), (1, 3, 0, 2)):
                out.append(tuple(signs[i] * v[perm[i]] for i in range(4)))
    return sorted(set(out))


def pin_cosine_pythagorean_exact(o):
    """Integer vectors with integer norms make the cosine an exact rational
    dot / (|q| |r|); the oracle's fp64 value is its correctly rounded quotient,
    and the order (with its exact ties) is the rank-counting order."""
    vecs = _norm_vectors()
    corpus = np.array(vecs, np.float32)
    norms = [round(float(np.sqrt(sum(x * x for x in v)))) for v in vecs]
    assert all(sum(x * x for x in v) == nv * nv for v, nv in zip(vecs, norms))
    n = len(vecs)
    for qi in (0, 7, 19, 33, 50):
        q = vecs[qi % n]
        nq = norms[qi % n]
        exact = [Fraction(sum(a * b for a, b in zip(v, q)), nv * nq) for v, nv in zip(vecs, norms)]
        got = o.cosine_scores(corpus, np.array(q, np.float32))
        for i in range(n):
            assert got[i] == float(exact[i]), (qi, i, got[i], exact[i])
        rank = [sum(1 for j in range(n) if _better(exact[j], j, exact[i], i)) for i in range(n)]
        by_rank = [None] * n
        for i, r in enumerate(rank):
            by_rank[r] = i
        for k in (1, 5, n):
            idx, _ = o.search(corpus, np.array([q], np.float32), k, metric=1)
            assert list(idx[0]) == by_rank[:k], (qi, k)


def pin_cosine_scale_invariance(o, seed=31):
    """Cosine ignores positive scale: rows and query multiplied by powers of two
    (exact in fp32) give bit-identical scores; a negated row gives the negated
    score."""
    rng = np.random.default_rng(seed)
    corpus = rng.standard_normal((30, 13)).astype(np.float32)
    q = rng.standard_normal(13).astype(np.float32)
    base = o.cosine_scores(corpus, q)
    scale = np.float32(2.0) ** rng.integers(-20, 21, size=30).astype(np.float32)
    scaled = corpus * scale[:, None]
    assert np.array_equal(o.cosine_scores(scaled, q * np.float32(2.0 ** -7)), base)
    assert np.array_equal(o.cosine_scores(-corpus, q), -base)
    assert np.all(np.abs(base) <= 1.0)


def pin_cosine_zero_norms(o):
    """A zero row scores -inf and ranks below every finite score (zero rows among
    themselves by index); a zero query makes every score -inf, so the answer is
    indices 0 .. k-1."""
    corpus = np.array([[0, 0, 0], [1, 0, 0], [0, 0, 0], [-1, 0, 0], [0, 2, 0]], np.float32)
    q = np.array([1, 0, 0], np.float32)
    sc = o.cosine_scores(corpus, q)
    assert sc[0] == -np.inf and sc[2] == -np.inf
    assert list(sc[[1, 3, 4]]) == [1.0, -1.0, 0.0]
    idx, _ = o.search(corpus, q[None, :], 5, metric=1)
    assert list(idx[0]) == [1, 4, 3, 0, 2]
    idx, sc = o.search(corpus, np.zeros((1, 3), np.float32), 3, metric=1)
    assert list(idx[0]) == [0, 1, 2] and np.all(sc == -np.inf)


def pin_cosine_decimal(o, seed=32):
    """On small random inputs the oracle agrees with a 50-digit decimal
    evaluation of dot / (|q| |r|) to within its own fp64 rounding bound."""
    from decimal import Decimal, getcontext
    getcontext().prec = 50
    rng = np.random.default_rng(seed)
    for n, d in ((12, 5), (7, 40)):
        corpus = rng.standard_normal((n, d)).astype(np.float32)
        q = rng.standard_normal(d).astype(np.float32)
        got = o.cosine_scores(corpus, q)
        dq = [Decimal(float(x)) for x in q]
        qn = sum(x * x for x in dq).sqrt()
        for i in range(n):
            dr = [Decimal(float(x)) for x in corpus[i]]
            exact = sum(a * b for a, b in zip(dr, dq)) / (sum(x * x for x in dr).sqrt() * qn)
            assert abs(Decimal(got[i]) - exact) <= Decimal((d + 8) * 2.0 ** -52), (n, d, i)


ALL_PINS = [
    pin_scores_exact_rational,
    pin_search_rank_counting,
    pin_search_integer_ties,
    pin_onehot_closed_form,
    pin_query_in_corpus,
    pin_topk_i32_lexsort,
    pin_topk_i32_special,
    pin_topk_f32_lexsort,
    pin_golden,
    pin_invariants,
    pin_permutation_invariance,
    pin_two_stage_decomposition,
    pin_cosine_pythagorean_exact,
    pin_cosine_scale_invariance,
    pin_cosine_zero_norms,
    pin_cosine_decimal,
]
