"""Pins of the oracle's fp32 building blocks against exact rational arithmetic."""
from fractions import Fraction
import numpy as np
import pytest

from oracle.fp import fma32, pairwise_sum, f16_round, f16_of_exact, F32


def _rn32(q: Fraction) -> np.float32:
    """Correctly rounded float32 of an exact rational (ties to even), by bracketing."""
    x = np.float32(float(q))            # float() of a Fraction is correctly rounded to float64
    # walk to the float32 neighbours and pick the nearest exactly
    cands = [np.nextafter(x, np.float32(-np.inf)), x, np.nextafter(x, np.float32(np.inf))]
    best = None
    for c in cands:
        d = abs(Fraction(float(c)) - q)
        if best is None or d < best[0] or (d == best[0] and (int(np.float32(c).view(np.uint32)) & 1) == 0):
            best = (d, c)
    return np.float32(best[1])


def test_fma32_matches_exact_rounding_random():
    rng = np.random.default_rng(7)
    a = (rng.standard_normal(3000) * np.exp2(rng.integers(-20, 20, 3000))).astype(np.float32)
    b = (rng.standard_normal(3000) * np.exp2(rng.integers(-20, 20, 3000))).astype(np.float32)
    c = (rng.standard_normal(3000) * np.exp2(rng.integers(-40, 40, 3000))).astype(np.float32)
    got = fma32(a, b, c)
    for i in range(len(a)):
        exact = Fraction(float(a[i])) * Fraction(float(b[i])) + Fraction(float(c[i]))
        assert got[i] == _rn32(exact), (a[i], b[i], c[i])


def test_fma32_double_rounding_midpoints():
    # a*b + c lands exactly on a float32 midpoint plus a tiny tail: the float64 sum
    # rounds onto the midpoint, and only the exact error decides the direction.
    one = np.float32(1.0)
    cases = []
    for k in range(1, 200):
        a = np.float32(1.0 + k * 2.0 ** -23)
        b = np.float32(1.0 + 2.0 ** -23)
        # a*b = 1 + (k+1) 2^-23 + k 2^-46 ; choose c to move the sum near a midpoint
        for c in (np.float32(2.0 ** -24), np.float32(-(2.0 ** -24)), np.float32(3 * 2.0 ** -24)):
            cases.append((a, b, c))
    cases.append((np.float32(1 + 2 ** -12), np.float32(1 + 2 ** -12), np.float32(-1.0)))
    cases.append((np.float32(1.0), np.float32(2 ** -24), one))
    cases.append((np.float32(1.0), np.float32(3 * 2 ** -24), one))
    a, b, c = map(np.array, zip(*cases))
    got = fma32(a.astype(np.float32), b.astype(np.float32), c.astype(np.float32))
    for i in range(len(cases)):
        exact = Fraction(float(a[i])) * Fraction(float(b[i])) + Fraction(float(c[i]))
        assert got[i] == _rn32(exact)


def test_fma32_single_rounding_differs_from_two():
    # 1 + 2^-24 is a tie: fl(fl(a*b) + c) and fma differ here.
    a = np.float32(1 + 2 ** -12)
    b = np.float32(1 + 2 ** -12)
    c = np.float32(-1.0)
    assert fma32(a, b, c) == np.float32(2 ** -11 + 2 ** -24)
    assert np.float32(a * b) + c != np.float32(2 ** -11 + 2 ** -24)


def test_pairwise_sum_tree_shape():
    # values chosen so that the association order shows in the float32 result
    x = np.array([1.0, 2 ** -24, 2 ** -24, 2 ** -24, -1.0, 2 ** -24, 2 ** -24, 2 ** -24], np.float32)
    tree = ((x[0] + x[1]) + (x[2] + x[3])) + ((x[4] + x[5]) + (x[6] + x[7]))
    assert pairwise_sum(x, 0, F32.add) == np.float32(tree)
    seq = np.float32(0)
    for v in x:
        seq = np.float32(seq + v)
    assert np.float32(tree) != seq   # the order matters for this input, and the tree is what is computed


def test_pairwise_sum_is_close_to_exact():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((50, 128)).astype(np.float32)
    got = pairwise_sum(x, 1, F32.add).astype(np.float64)
    exact = np.array([float(sum(Fraction(float(v)) for v in row)) for row in x])
    bound = 8 * 2.0 ** -24 * np.sum(np.abs(x), axis=1)    # log2(128) levels, one rounding each
    assert np.all(np.abs(got - exact) <= bound)


def test_pairwise_sum_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        pairwise_sum(np.ones(6, np.float32), 0, F32.add)


def test_f16_round_ties_and_subnormals():
    vals = np.array([1 + 2 ** -11, 1 + 3 * 2 ** -11, 2 ** -24, 2 ** -25, 3 * 2 ** -25, 65504.0, 65520.0],
                    np.float32)
    exp = np.array([1.0, 1 + 2 ** -9, 2 ** -24, 0.0, 2 ** -23, 65504.0, np.inf], np.float32)
    assert np.array_equal(f16_round(vals), exp)


def _rn16(q: Fraction) -> float:
    """Correctly rounded binary16 of an exact rational (ties to even), by bracketing."""
    if q == 0:
        return 0.0
    h = np.float16(float(q))
    cands = [np.nextafter(h, np.float16(-np.inf)), h, np.nextafter(h, np.float16(np.inf))]
    best = None
    for c in cands:
        if not np.isfinite(c):
            continue
        d = abs(Fraction(float(c)) - q)
        if best is None or d < best[0] or (d == best[0] and (int(np.float16(c).view(np.uint16)) & 1) == 0):
            best = (d, c)
    return float(best[1])


def test_f16_of_exact_rounds_products_once():
    rng = np.random.default_rng(21)
    a = rng.uniform(0.5, 1.0, 4000).astype(np.float32)
    u = (rng.standard_normal(4000) * np.exp2(rng.integers(-26, 4, 4000))).astype(np.float16)
    got = f16_of_exact(a.astype(np.float64) * u.astype(np.float64))
    for i in range(len(a)):
        exact = Fraction(float(a[i])) * Fraction(float(u[i]))
        assert float(got[i]) == _rn16(exact), (a[i], u[i])
    # the single rounding differs from rounding to float32 first on some inputs
    a = rng.uniform(0.5, 1.0, 2_000_000).astype(np.float32)
    u = rng.standard_normal(2_000_000).astype(np.float16)
    once = f16_of_exact(a.astype(np.float64) * u.astype(np.float64))
    twice = f16_round((a * u.astype(np.float32)).astype(np.float32))
    i = np.flatnonzero(once != twice)
    assert len(i) > 0
    exact = Fraction(float(a[i[0]])) * Fraction(float(u[i[0]]))
    assert float(once[i[0]]) == _rn16(exact)
