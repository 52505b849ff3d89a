"""The cosine bounds of the filtered search, on the host (no GPU).

Reading: with a - e <= acc <= a + e for the plain scan's fp32 inner product acc
and den = fl(|q| |x|) > 0, the plain cosine fl(acc / den) lies in
[lo, hi] = [fl(fl(a - e) / den) - (2^-20 |.| + FLT_MIN), fl(fl(a + e) / den) + (2^-20 |.| + FLT_MIN)]
(each step in fp32, round to nearest: IEEE division is what the GPU's
correctly rounded fp32 division gives), and an overflowed quotient gives the
infinite bound on its side (+inf above, -inf below: the row is kept).  Checked here with numpy's fp32
arithmetic over adversarial values: quotients near the top and the bottom of
the fp32 range (overflow to inf, subnormal results), acc at the ends of its
interval and in between, both signs, and den from subnormal to huge.  Under
correctly rounded division the bounds hold without widening (monotonicity);
the widening is the margin for a division off by several ulps."""
import numpy as np

F32 = np.float32
FLT_MIN = F32(np.finfo(np.float32).tiny)


def _bounds(a, e, den, rel=F32(2.0 ** -20), absolute=FLT_MIN):
    with np.errstate(over="ignore", under="ignore", invalid="ignore"):
        h = F32(F32(a + e) / den)
        l = F32(F32(a - e) / den)
        hi = F32(h + F32(F32(abs(h)) * rel + absolute)) if np.isfinite(h) else F32(np.inf)
        lo = F32(l - F32(F32(abs(l)) * rel + absolute)) if np.isfinite(l) else F32(-np.inf)
    return hi, lo


def _cases(rng, n):
    for _ in range(n):
        den = F32(np.exp(rng.uniform(np.log(1e-44), np.log(3e38))))
        if den <= 0:
            continue
        mag = F32(np.exp(rng.uniform(np.log(1e-45), np.log(3e38))))
        a = F32(mag * rng.choice([-1.0, 1.0]))
        with np.errstate(over="ignore"):
            e = F32(abs(a) * F32(rng.choice([0.0, 2.0 ** -20, 2.0 ** -8, 0.03, 1.0, 4.0])))
        if not np.isfinite(e):  # the kernel gives such a row the bounds (+inf, -inf) before the quotient
            continue
        for t in (0.0, 1.0, -1.0, rng.uniform(-1, 1)):
            with np.errstate(over="ignore", invalid="ignore"):
                acc = F32(a + F32(t) * e)
            if not np.isfinite(acc) or abs(acc - a) > e:  # left the interval when rounded
                continue
            yield a, e, den, acc


def _violations(rel=F32(2.0 ** -20), absolute=FLT_MIN, n=20000):
    rng = np.random.default_rng(2026)
    bad = 0
    for a, e, den, acc in _cases(rng, n):
        with np.errstate(over="ignore", under="ignore"):
            plain = F32(acc / den)
        hi, lo = _bounds(a, e, den, rel, absolute)
        if not (lo <= plain <= hi):
            bad += 1
    return bad


def test_widening_covers_the_divisions():
    assert _violations() == 0


def test_ieee_division_needs_no_widening():
    """acc <= a + e for floats means acc <= fl(a + e) (no float lies between
    fl(a + e) and a + e when rounding to nearest), and correctly rounded
    division is monotone: the bounds hold even without widening."""
    assert _violations(rel=F32(0.0), absolute=F32(0.0)) == 0


def _ulps(x, n, direction):
    for _ in range(n):
        x = np.nextafter(x, F32(direction), dtype=np.float32)
    return x


def test_widening_tolerates_an_inexact_division():
    """The widening is the margin for a division that is not correctly
    rounded: a plain cosine 8 ulps off either way (or any amount below the
    normal range) still lies within the bounds."""
    rng = np.random.default_rng(7)
    for a, e, den, acc in _cases(rng, 5000):
        with np.errstate(over="ignore", under="ignore"):
            plain = F32(acc / den)
        if not np.isfinite(plain):
            continue
        hi, lo = _bounds(a, e, den)
        assert _ulps(plain, 8, np.inf) <= hi and _ulps(plain, 8, -np.inf) >= lo, (a, e, den, acc)
        if abs(plain) < FLT_MIN:
            assert F32(plain + F32(0.99) * FLT_MIN) <= hi and F32(plain - F32(0.99) * FLT_MIN) >= lo


def test_overflow_and_zero():
    # both quotients overflow: the bounds are (+inf, -inf), never NaN
    hi, lo = _bounds(F32(3e38), F32(3e37), F32(1e-3))
    assert np.isposinf(hi) and np.isneginf(lo)
    hi, lo = _bounds(F32(-3e38), F32(0.0), F32(1e-3))
    assert np.isposinf(hi) and np.isneginf(lo)
    hi, lo = _bounds(F32(0.0), F32(0.0), F32(2.0))
    assert hi > 0 > lo


# ---- the library's own code (the function the kernels compile), on the host

def _lib_bounds(lib, known, a, e, qnorm, rn):
    import ctypes
    out = (ctypes.c_float * 2)()
    assert lib.rt_filter_cosine_bounds(int(known), float(a), float(e), float(qnorm), float(rn), out) == 0
    return F32(out[0]), F32(out[1])


def test_library_cosine_bounds_match_the_model():
    """rt_filter_cosine_bounds runs the same cosine_bounds source as the first
    passes of the filtered cosine search; bit for bit it must give the model's
    bounds above on the same adversarial cases (den = qnorm x 1.0 exactly), the
    (-inf, -inf) of a non-positive product of norms, and the untouched
    (+inf, -inf) of an unknown bound."""
    from top_search_resident_amd import _lib
    lib = _lib.load()
    rng = np.random.default_rng(2027)
    n = 0
    for a, e, den, acc in _cases(rng, 5000):
        hi, lo = _lib_bounds(lib, True, a, e, den, 1.0)
        mhi, mlo = _bounds(a, e, den)
        assert hi.tobytes() == mhi.tobytes() and lo.tobytes() == mlo.tobytes(), (a, e, den, hi, mhi, lo, mlo)
        with np.errstate(over="ignore", under="ignore"):
            plain = F32(acc / den)
        assert lo <= plain <= hi
        n += 1
    assert n > 10000
    for qn, rn in ((0.0, 1.0), (1.0, 0.0), (-1.0, 1.0), (1e-30, 1e-30)):  # the last product underflows to 0
        hi, lo = _lib_bounds(lib, True, 0.5, 0.1, qn, rn)
        assert np.isneginf(hi) and np.isneginf(lo), (qn, rn)
    hi, lo = _lib_bounds(lib, False, 0.5, 0.1, 2.0, 3.0)
    assert np.isposinf(hi) and np.isneginf(lo)
    hi, lo = _lib_bounds(lib, True, F32(3e38), F32(3e37), F32(1e-3), 1.0)
    assert np.isposinf(hi) and np.isneginf(lo)


def test_library_cosine_score():
    """rt_cosine_score is the scans' cosine epilogue: fp32 acc / fl(qnorm rnorm),
    -inf when that product is not positive (a zero row, a zero query, or norms
    whose product underflows in fp32)."""
    from top_search_resident_amd import _lib
    lib = _lib.load()
    rng = np.random.default_rng(5)
    for _ in range(2000):
        acc = F32(rng.standard_normal() * 10.0 ** rng.integers(-20, 20))
        qn = F32(abs(rng.standard_normal()) * 10.0 ** rng.integers(-18, 18))
        rn = F32(abs(rng.standard_normal()) * 10.0 ** rng.integers(-18, 18))
        with np.errstate(over="ignore", under="ignore", invalid="ignore"):
            den = F32(qn * rn)
            want = F32(acc / den) if den > 0 else F32(-np.inf)
        got = F32(lib.rt_cosine_score(float(acc), float(qn), float(rn)))
        assert got.tobytes() == want.tobytes() or (np.isnan(got) and np.isnan(want)), (acc, qn, rn, got, want)
    assert np.isneginf(lib.rt_cosine_score(1.0, 0.0, 5.0))
    assert np.isneginf(lib.rt_cosine_score(1e-40, 1e-25, 1e-25))  # |q| |x| underflows: ranked as a zero row
