"""The bound behind search_resident_filtered, checked on the host (no GPU).

For a row x and query q, a = the fp32 dot product of bf16(x) with q and s = the
fp32 dot product of x with q (any summation order) must satisfy
    |a - s| <= cb |q| |x| + delta max(|q|, 1)
with (cb, delta) = rt_filter_bounds(d).  bf16(x) is torch's float -> bfloat16
conversion (round to nearest, ties to even), a library routine independent of
the HIP code.  The worst case is built by hand: every element sits exactly
halfway between two bf16 values and the signs of q make every rounding lower
the product, so the bf16 dot product falls short by 2^-8 of sum |x q|, the most
that rounding to 8 significant bits allows; a factor below 2^-8 fails it."""
from fractions import Fraction

import numpy as np
import pytest

import workloads
from top_search_resident_amd import _lib

torch = pytest.importorskip("torch")


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def _sums32(x, q):
    """fp32 dot products of x and q in two orders: sequential and numpy's pairwise."""
    p = (x.astype(np.float32) * q.astype(np.float32)).astype(np.float32)
    return float(np.cumsum(p, dtype=np.float32)[-1]), float(np.sum(p, dtype=np.float32))


def _bound(d, x, q):
    cb, delta = _lib.filter_bounds(d)
    nx = float(np.sqrt(np.sum(x.astype(np.float64) ** 2)))
    nq = float(np.sqrt(np.sum(q.astype(np.float64) ** 2)))
    return cb * nq * nx + delta * max(nq, 1.0), cb, nx, nq


def _check(x, q):
    d = x.shape[0]
    xb = _bf16(x)
    bound, _, _, _ = _bound(d, x, q)
    a_orders, s_orders = _sums32(xb, q), _sums32(x, q)
    for a in a_orders:
        for s in s_orders:
            assert abs(a - s) <= bound, (a, s, bound)


def _worst_case_row():
    # 1 + 2^-8 is halfway between the bf16 values 1 and 1 + 2^-7 and rounds to 1;
    # 1 + 3 2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6 and rounds to 1 + 2^-6.
    x = np.empty(64, np.float32)
    x[:40] = 1 + 2.0 ** -8
    x[40:] = -(1 + 3 * 2.0 ** -8)
    return x, np.ones(64, np.float32)


def test_bf16_rounding_used_by_the_worst_case():
    x, _ = _worst_case_row()
    xb = _bf16(x)
    assert np.all(xb[:40] == 1.0) and np.all(xb[40:] == -(1 + 2.0 ** -6))


def test_worst_case_rounding_is_covered_and_tight():
    x, q = _worst_case_row()
    xb = _bf16(x)
    exact_a = sum(Fraction(float(v)) for v in xb)
    exact_s = sum(Fraction(float(v)) for v in x)
    assert exact_s == Fraction(127, 8) and exact_a == Fraction(125, 8)
    err = float(exact_s - exact_a)                     # 0.25 = 64 elements x 2^-8
    bound, cb, nx, nq = _bound(64, x, q)
    assert err <= bound
    # the case needs the full 2^-8: half of it (or any factor < 0.99 2^-8) fails
    assert err / (nx * nq) > 0.99 * 2.0 ** -8
    assert err > 0.5 * cb * nx * nq
    _check(x, q)


def test_worst_case_decides_a_search():
    """The competitor row b (exact in bf16) scores 15.8125 < 15.875: a lower
    bound for b above the upper bound for the worst-case row would drop the
    true winner.  With the library's constants it does not."""
    x, q = _worst_case_row()
    b = np.full(64, 253 / 1024, np.float32)
    assert np.array_equal(_bf16(b), b)
    s_x, s_b = 127 / 8, float(np.sum(b, dtype=np.float64))
    assert s_b < s_x
    a_x = float(np.sum(_bf16(x), dtype=np.float64))
    ex, _, _, _ = _bound(64, x, q)
    eb, _, _, _ = _bound(64, b, q)
    assert a_x + ex >= s_b - eb  # upper bound of the winner reaches the competitor's lower bound
    # the same construction with half the factor excludes the winner
    cb, delta = _lib.filter_bounds(64)
    nx, nb, nq = np.linalg.norm(x.astype(np.float64)), np.linalg.norm(b.astype(np.float64)), 8.0
    assert a_x + cb / 2 * nx * nq < s_b - cb / 2 * nb * nq


@pytest.mark.parametrize("d", [8, 64, 384, 1024, 2048])
def test_random_rows_within_bound(d):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([7, d])))
    for trial in range(40):
        kind = trial % 5
        x = rng.standard_normal(d).astype(np.float32)
        q = rng.standard_normal(d).astype(np.float32)
        if kind == 1:
            x *= np.exp(2.0 * rng.standard_normal(d)).astype(np.float32)
        elif kind == 2:      # values below 2^-126 (bf16 and fp32 subnormals)
            x *= np.float32(1e-39)
        elif kind == 3:      # large values and an unnormalised query
            x *= np.float32(1e30)
            q *= np.float32(1e3)
        elif kind == 4:      # every element halfway between two bf16 values
            bits = (x.view(np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
            x = bits.view(np.float32)
        _check(x, q)


def test_gaussian_unit_rows_within_bound():
    x = workloads.gaussian_rows(300, 1024, config_id=900)
    q = workloads.gaussian_rows(1, 1024, config_id=900, stream=1)[0]
    for row in x:
        _check(row, q)


def test_constants_follow_the_derivation():
    for d in (1, 8, 64, 1024, 2048, 100_000):
        cb, delta = _lib.filter_bounds(d)
        u = Fraction(1, 2 ** 24)
        gamma = d * u / (1 - d * u)
        base = Fraction(1, 256) + gamma * (2 + Fraction(1, 256))
        assert Fraction(cb) >= base * (1 + Fraction(1, 1024))
        assert Fraction(cb) <= base * (1 + Fraction(1, 512))
        assert Fraction(delta) == Fraction(4 * d, 2 ** 126)


def test_rejects_bad_depth():
    with pytest.raises(_lib.ResidentTopKError):
        _lib.filter_bounds(0)
