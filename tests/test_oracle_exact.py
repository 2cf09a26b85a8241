"""Pins for oracle.exact: every result is checked against exact rational arithmetic.

The reference rounding here is a brute-force search over the fp32 neighbours of
a value, compared with Python Fractions, so it shares nothing with the
round-to-odd construction it checks.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import exact

F32 = np.float32


def _neighbours(x):
    x = F32(x)
    return [np.nextafter(x, F32(-np.inf)), x, np.nextafter(x, F32(np.inf))]


def rn32(q: Fraction) -> F32:
    """Round an exact rational to the nearest fp32 (ties to even) by search."""
    approx = F32(float(q))
    best = None
    for c in _neighbours(approx) + _neighbours(np.nextafter(approx, F32(np.inf))) + \
            _neighbours(np.nextafter(approx, F32(-np.inf))):
        if not np.isfinite(c):
            continue
        d = abs(Fraction(float(c)) - q)
        key = (d, int(np.asarray(c, F32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return F32(best[1])


def rd32(q: Fraction) -> F32:
    """Largest fp32 not above q, by search."""
    approx = F32(float(q))
    cands = set()
    for c in _neighbours(approx) + _neighbours(np.nextafter(approx, F32(-np.inf))):
        if np.isfinite(c) and Fraction(float(c)) <= q:
            cands.add(float(c))
    return F32(max(cands))


def _rand_f32(rng, n, lo=-30, hi=30):
    mant = rng.uniform(1.0, 2.0, n)
    sign = rng.choice([-1.0, 1.0], n)
    return (sign * mant * np.exp2(rng.integers(lo, hi, n))).astype(F32)


def test_fma32_random_against_fractions():
    rng = np.random.default_rng(1)
    a = _rand_f32(rng, 4000)
    b = _rand_f32(rng, 4000)
    c = _rand_f32(rng, 4000)
    # make a quarter of the cases cancel heavily: c ~ -a*b
    k = slice(0, 1000)
    c[k] = -(a[k].astype(np.float64) * b[k].astype(np.float64)).astype(F32)
    got = exact.fma32(a, b, c)
    for i in range(a.size):
        want = rn32(Fraction(float(a[i])) * Fraction(float(b[i])) + Fraction(float(c[i])))
        assert got[i] == want, (a[i], b[i], c[i], got[i], want)


def test_fma32_double_rounding_cases():
    # a*b = 1 + 2^-11 + 2^-24 is an exact fp32 tie; a tiny c decides the direction.
    a = F32(1 + 2.0 ** -12)
    tiny = F32(2.0 ** -80)
    up = exact.fma32(a, a, tiny)
    down = exact.fma32(a, a, -tiny)
    assert up == F32(1 + 2.0 ** -11 + 2.0 ** -23)
    assert down == F32(1 + 2.0 ** -11)
    # the tie itself rounds to the even neighbour
    assert exact.fma32(a, a, F32(0)) == F32(1 + 2.0 ** -11)


def test_fma32_matches_separate_ops_when_exact():
    # when a*b is exactly representable, fma equals fl(fl(a*b) + c)
    rng = np.random.default_rng(2)
    a = rng.integers(-2048, 2048, 1000).astype(F32)
    b = rng.integers(-2048, 2048, 1000).astype(F32)
    c = _rand_f32(rng, 1000, -5, 20)
    assert np.array_equal(exact.fma32(a, b, c), ((a * b).astype(F32) + c).astype(F32))


@pytest.mark.parametrize("num", [127.0, 7.0])
def test_rd_div32_against_fractions(num):
    rng = np.random.default_rng(3)
    m = np.abs(_rand_f32(rng, 3000, -60, 60))
    m = np.concatenate([m, np.array([1.0, 2.0, 127.0, 7.0, 0.5, 3.0, 1e-38, 1.5e-45,
                                     3.4e38], F32)])
    got = exact.rd_div32(F32(num), m)
    for i in range(m.size):
        q = Fraction(num) / Fraction(float(m[i]))
        if q > Fraction(float(np.finfo(F32).max)):
            want = np.finfo(F32).max
        else:
            want = rd32(q)
        assert got[i] == want, (m[i], got[i], want)
        # and it is the largest such value
        assert Fraction(float(got[i])) <= q


def test_rd_div32_zero_is_zero():
    assert exact.rd_div32(F32(127), F32(0)) == 0


def test_rn_div32_against_fractions():
    rng = np.random.default_rng(4)
    m = np.abs(_rand_f32(rng, 2000, -40, 40))
    for r in (127.0, 7.0):
        got = exact.rn_div32(m, F32(r))
        for i in range(m.size):
            assert got[i] == rn32(Fraction(float(m[i])) / Fraction(r))


def test_dot_rn32_is_correctly_rounded_on_small_cases():
    rng = np.random.default_rng(5)
    A = _rand_f32(rng, 8 * 16, -4, 4).reshape(8, 16)
    x = _rand_f32(rng, 16, -4, 4)
    got = exact.dot_rn32(A, x)
    for i in range(8):
        want = rn32(sum(Fraction(float(A[i, j])) * Fraction(float(x[j])) for j in range(16)))
        assert got[i] == want


def test_bf16_to_f32_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x4049, 0x7F7F], np.uint16)
    vals = exact.bf16_to_f32(bits)
    assert list(vals[:4]) == [1.0, -1.0, 0.0, -0.0]
    assert vals[4] == F32(3.140625)
