"""The bound behind the batched first pass of search_resident_filtered, on the
host (no GPU).

For a row x and query q the batched pass computes a = sum_j bf16(x_j) hi_j +
bf16(x_j) lo_j on bf16 matrix cores, with the query split into two bf16 parts
hi = bf16(q), lo = bf16(q - hi); the single-query scan computes s = the fp32
dot product of x with q.  The library's constants (cr, cx, delta) =
rt_filter_bounds_batched(d) must give
    |a - s| <= |q| (cr |x - bf16(x)| + cx |x|) + delta max(|q|, 1) max(|x|, 1)
for any fp32 accumulation order and rounding direction of the 2 d exact
products.  bf16 rounding here is torch's float -> bfloat16 conversion (round to
nearest, ties to even), a library routine independent of the HIP code.  The
worst case is built by hand: every element of x sits halfway between two bf16
values and rounds down, so a falls short by 2^-8 of sum |x q|, the most that
rounding to 8 significant bits allows, and equals |x - bf16(x)| |q|: half of cr
fails it.  The query
split is checked on its own: q - (hi + lo) is at most 2^-16 |q|."""
from fractions import Fraction

import numpy as np
import pytest

import workloads
from top_search_resident_amd import _lib

torch = pytest.importorskip("torch")


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def _split(q):
    hi = _bf16(q)
    lo = _bf16((q.astype(np.float32) - hi).astype(np.float32))
    return hi, lo


def _round32(v, mode):
    """fp32 rounding of an exact rational: to nearest (numpy) or toward zero."""
    f = np.float32(float(v))
    if mode == "zero" and abs(Fraction(float(f))) > abs(v):
        f = np.nextafter(f, np.float32(0.0))
    return f


def _mfma_like_sums(xb, hi, lo):
    """The 2 d exact products summed in fp32 by several orders and roundings a
    matrix core could use: sequential (nearest, toward zero), and blocks of 16
    summed exactly and rounded once before joining the running sum (nearest,
    toward zero)."""
    prods = []
    for j in range(xb.shape[0]):
        prods.append(Fraction(float(xb[j])) * Fraction(float(hi[j])))
        prods.append(Fraction(float(xb[j])) * Fraction(float(lo[j])))
    out = []
    for mode in ("nearest", "zero"):
        acc = np.float32(0.0)
        for p in prods:
            acc = _round32(Fraction(float(acc)) + p, mode)
        out.append(float(acc))
        acc = np.float32(0.0)
        for b in range(0, len(prods), 16):
            acc = _round32(Fraction(float(acc)) + sum(prods[b:b + 16]), mode)
        out.append(float(acc))
    return out


def _plain_sums(x, q):
    """fp32 dot products of x and q: sequential and numpy's pairwise order."""
    p = (x.astype(np.float32) * q.astype(np.float32)).astype(np.float32)
    return float(np.cumsum(p, dtype=np.float32)[-1]), float(np.sum(p, dtype=np.float32))


def _bound(d, x, q):
    """The library's bound, with |x - bf16(x)| and the norms in fp64 (the
    library rounds them up to fp32)."""
    cr, cx, delta = _lib.filter_bounds_batched(d)
    nx = float(np.sqrt(np.sum(x.astype(np.float64) ** 2)))
    nq = float(np.sqrt(np.sum(q.astype(np.float64) ** 2)))
    ne = float(np.sqrt(np.sum((x.astype(np.float64) - _bf16(x).astype(np.float64)) ** 2)))
    return nq * (cr * ne + cx * nx) + delta * max(nq, 1.0) * max(nx, 1.0), cr, ne, nq


def _check(x, q):
    d = x.shape[0]
    xb = _bf16(x)
    hi, lo = _split(q)
    bound, _, _, _ = _bound(d, x, q)
    for a in _mfma_like_sums(xb, hi, lo):
        for s in _plain_sums(x, q):
            assert abs(a - s) <= bound, (a, s, bound)


def test_query_split_error():
    """q - (hi + lo) is at most 2^-16 |q| (and exactly 0 for values with at
    most 16 significant bits)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([11])))
    q = rng.standard_normal(4096).astype(np.float32) * np.exp(3 * rng.standard_normal(4096)).astype(np.float32)
    hi, lo = _split(q)
    for v, h, l in zip(q, hi, lo):
        r = Fraction(float(v)) - Fraction(float(h)) - Fraction(float(l))
        assert abs(r) <= abs(Fraction(float(v))) * Fraction(1, 2 ** 16)
    short = (q.view(np.uint32) & np.uint32(0xFFFF8000)).view(np.float32)
    hi, lo = _split(short)
    assert np.array_equal(hi.astype(np.float64) + lo.astype(np.float64), short.astype(np.float64))


def _worst_case():
    # 1 + 2^-8 is halfway between the bf16 values 1 and 1 + 2^-7 and rounds to
    # 1 (ties to even); the query 1 splits exactly (hi = 1, lo = 0).
    x = np.full(64, 1 + 2.0 ** -8, np.float32)
    q = np.ones(64, np.float32)
    return x, q


def test_worst_case_roundings():
    x, q = _worst_case()
    assert np.all(_bf16(x) == 1.0)
    hi, lo = _split(q)
    assert np.all(hi == 1.0) and np.all(lo == 0.0)


def test_worst_case_is_covered_and_tight():
    x, q = _worst_case()
    xb = _bf16(x)
    hi, lo = _split(q)
    exact_a = sum(Fraction(float(a)) * (Fraction(float(h)) + Fraction(float(l))) for a, h, l in zip(xb, hi, lo))
    exact_s = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x, q))
    err = float(exact_s - exact_a)
    bound, cr, ne, nq = _bound(64, x, q)
    assert err <= bound
    # the whole rounding error counts: the shortfall equals |x - bf16(x)| |q|,
    # so half of cr (or a bound that charged only part of it) fails
    assert abs(err - ne * nq) <= 1e-12 * err
    assert err > 0.5 * cr * ne * nq + (bound - cr * ne * nq)
    _check(x, q)


@pytest.mark.parametrize("d", [256, 768, 1024])
def test_random_rows_within_bound(d):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([13, d])))
    for trial in range(10):
        kind = trial % 5
        x = rng.standard_normal(d).astype(np.float32)
        q = rng.standard_normal(d).astype(np.float32)
        if kind == 1:
            x *= np.exp(2.0 * rng.standard_normal(d)).astype(np.float32)
            q *= np.exp(2.0 * rng.standard_normal(d)).astype(np.float32)
        elif kind == 2:      # values below 2^-126 in the row and the query
            x *= np.float32(1e-39)
            q *= np.float32(1e-30)
        elif kind == 3:      # large values and an unnormalised query
            x *= np.float32(1e30)
            q *= np.float32(1e3)
        elif kind == 4:      # every element halfway between two bf16 values
            x = ((x.view(np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
            q = ((q.view(np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
        _check(x, q)


def test_gaussian_unit_rows_within_bound():
    x = workloads.gaussian_rows(12, 768, config_id=901)
    q = workloads.gaussian_rows(1, 768, config_id=901, stream=1)[0]
    for row in x:
        _check(row, q)


def test_constants_follow_the_derivation():
    for d in (1, 256, 768, 1024, 100_000):
        cr, cx, delta = _lib.filter_bounds_batched(d)
        u = Fraction(1, 2 ** 24)
        gamma = d * u / (1 - d * u)
        g8 = 8 * d * u / (1 - 8 * d * u)
        base_r = 1 + Fraction(1, 2 ** 16)
        base_x = Fraction(1, 2 ** 16) + gamma + Fraction(102, 100) * g8
        for c, base in ((cr, base_r), (cx, base_x)):
            assert Fraction(c) >= base * (1 + Fraction(1, 1024))
            assert Fraction(c) <= base * (1 + Fraction(1, 512))
        assert Fraction(delta) == Fraction(16 * d, 2 ** 126)


def test_rounding_error_norm_is_smaller_than_the_elementwise_bound():
    """For Gaussian rows |x - bf16(x)| is well below 2^-8 |x| (what an
    elementwise bound would charge): the reason the bound uses it."""
    x = workloads.gaussian_rows(64, 768, config_id=902).astype(np.float64)
    ne = np.linalg.norm(x - _bf16(x.astype(np.float32)), axis=1)
    ratio = ne / np.linalg.norm(x, axis=1) / 2.0 ** -8
    assert np.all(ratio < 0.6) and np.all(ratio > 0.2)


def test_rejects_bad_depth():
    with pytest.raises(_lib.ResidentTopKError):
        _lib.filter_bounds_batched(0)
