"""The bound behind the fp8 first pass of search_resident_filtered, on the host
(no GPU).

A row x is stored as e4m3 codes of x / s, s a power of two with max |x| <= 224 s
(the library's rule, also checked here), so x~ = s dec(codes).  The pass
computes a = s (fp32 sum of dec(codes)_j q_j); the single-query scan computes s
= the fp32 dot product of x with q.  The library's constants (cr, cx, delta) =
rt_filter_bounds_fp8(d) must give
    |a - s| <= |q| (cr |x - x~| + cx |x|) + delta max(|q|, 1) max(s, 1)
for the fp32 sums in any order.  The e4m3 rounding here is torch's float ->
float8_e4m3fn conversion (round to nearest, ties to even), a library routine
independent of the HIP code; the library measures |x - x~| from its own stored
codes, so the bound holds whatever rounding the hardware conversion uses.
The worst case is built by hand: every element halfway between two e4m3
values and rounding down, so a falls short by exactly |x - x~| |q|: half of cr
fails it."""
from fractions import Fraction

import numpy as np
import pytest

import workloads
from top_search_resident_amd import _lib

torch = pytest.importorskip("torch")


def _scale(x):
    """The library's per-row scale: the power of two 2^k with max |x| <= 224 2^k
    (k >= -126; 1 for a zero row)."""
    mx = float(np.max(np.abs(x.astype(np.float64))))
    if mx == 0.0:
        return 1.0
    k = int(np.ceil(np.log2(mx / 224.0)))
    while 224.0 * 2.0 ** (k - 1) >= mx:
        k -= 1
    while 224.0 * 2.0 ** k < mx:
        k += 1
    return 2.0 ** max(k, -126)


def _quantize(x):
    s = _scale(x)
    v = (x.astype(np.float64) / s).astype(np.float32)
    dec = torch.from_numpy(v).to(torch.float8_e4m3fn).to(torch.float32).numpy()
    return s, dec


def _sums32(p):
    """fp32 sums of the products p: sequential and numpy's pairwise order."""
    p = p.astype(np.float32)
    return float(np.cumsum(p, dtype=np.float32)[-1]), float(np.sum(p, dtype=np.float32))


def _bound(d, x, q, s, dec):
    cr, cx, delta = _lib.filter_bounds_fp8(d)
    nx = float(np.linalg.norm(x.astype(np.float64)))
    nq = float(np.linalg.norm(q.astype(np.float64)))
    ne = float(np.linalg.norm(x.astype(np.float64) - s * dec.astype(np.float64)))
    return nq * (cr * ne + cx * nx) + delta * max(nq, 1.0) * max(s, 1.0), cr, ne, nq


def _check(x, q):
    d = x.shape[0]
    s, dec = _quantize(x)
    bound, _, _, _ = _bound(d, x, q, s, dec)
    for a0 in _sums32(dec.astype(np.float32) * q.astype(np.float32)):
        a = float(np.float32(a0) * np.float32(s))
        for sp in _sums32(x.astype(np.float32) * q.astype(np.float32)):
            assert abs(a - sp) <= bound, (a, sp, bound)


def test_scale_rule():
    rng = np.random.default_rng(3)
    for mag in (1e-30, 1e-3, 1.0, 224.0, 225.0, 1e20):
        x = (rng.standard_normal(64) * mag).astype(np.float32)
        s = _scale(x)
        r = float(np.max(np.abs(x))) / s
        assert 112.0 < r <= 224.0, (mag, r)
        assert np.log2(s) == int(np.log2(s))


def _worst_case():
    # 1.0625 is halfway between the e4m3 values 1 and 1.125 and rounds to 1
    # (ties to even); the row's maximum 224 sets s = 1 (224 itself is exact).
    x = np.full(64, 1.0625, np.float32)
    x[0] = 224.0
    q = np.ones(64, np.float32)
    q[0] = 0.0
    return x, q


def test_worst_case_is_covered_and_tight():
    x, q = _worst_case()
    s, dec = _quantize(x)
    assert s == 1.0 and dec[0] == 224.0 and np.all(dec[1:] == 1.0)
    exact_a = sum(Fraction(float(v)) * Fraction(float(w)) for v, w in zip(dec, q))
    exact_s = sum(Fraction(float(v)) * Fraction(float(w)) for v, w in zip(x, q))
    err = float(exact_s - exact_a)  # 63 elements x 2^-4
    bound, cr, ne, nq = _bound(64, x, q, s, dec)
    assert err <= bound
    # the shortfall equals |x - x~| |q| (q is 1 on every rounded element): half of cr fails
    assert abs(err - ne * nq) <= 1e-12 * err
    assert err > 0.5 * cr * ne * nq + (bound - cr * ne * nq)
    _check(x, q)


@pytest.mark.parametrize("d", [256, 1024, 2048])
def test_random_rows_within_bound(d):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([17, d])))
    for trial in range(30):
        kind = trial % 6
        x = rng.standard_normal(d).astype(np.float32)
        q = rng.standard_normal(d).astype(np.float32)
        if kind == 1:
            x *= np.exp(3.0 * rng.standard_normal(d)).astype(np.float32)
        elif kind == 2:      # values near and below 2^-126: the scale stops at 2^-126
            x *= np.float32(1e-38)
        elif kind == 3:      # large values and an unnormalised query
            x *= np.float32(1e30)
            q *= np.float32(1e3)
        elif kind == 4:      # a few huge entries: most others become e4m3 subnormals or zero
            x[rng.integers(0, d, 3)] *= np.float32(1e6)
        elif kind == 5:      # small integers: exact in e4m3 after scaling
            x = rng.integers(-3, 4, d).astype(np.float32)
        _check(x, q)


def test_gaussian_unit_rows_within_bound_and_error_size():
    x = workloads.gaussian_rows(64, 1024, config_id=903)
    q = workloads.gaussian_rows(1, 1024, config_id=903, stream=1)[0]
    ratios = []
    for row in x:
        _check(row, q)
        s, dec = _quantize(row)
        ratios.append(np.linalg.norm(row.astype(np.float64) - s * dec) / np.linalg.norm(row))
    # about 0.027 |x|: far wider than bf16's ~0.0017 |x|, hence the larger re-rank
    assert 0.015 < float(np.mean(ratios)) < 0.04


def test_constants_follow_the_derivation():
    for d in (1, 256, 1024, 2048, 100_000):
        cr, cx, delta = _lib.filter_bounds_fp8(d)
        u = Fraction(1, 2 ** 24)
        gamma = d * u / (1 - d * u)
        for c, base in ((cr, 1 + gamma), (cx, 2 * gamma)):
            assert Fraction(c) >= base * (1 + Fraction(1, 1024))
            assert Fraction(c) <= base * (1 + Fraction(1, 512))
        assert Fraction(delta) == Fraction(4 * d, 2 ** 126)


def test_rejects_bad_depth():
    with pytest.raises(_lib.ResidentTopKError):
        _lib.filter_bounds_fp8(0)
