"""Pins of the atomic variant's reference (oracle.sum_abs), independent of
it: exact rational sums (oracle/exact.py), closed forms, and the summation
bound it is used with, checked against arrival-order binary32 folds taken
in exact arithmetic over every permutation of small rank sets."""
import itertools
from fractions import Fraction

import numpy as np

import oracle
from oracle import exact

U = Fraction(1, 2 ** 24)


def _val(bits):
    cls, _, v = exact.decode(int(bits), exact.BF16)
    assert cls == exact.FIN
    return v


def _rand(rng, shape, lo=-20, hi=20):
    sign = rng.integers(0, 2, size=shape, dtype=np.uint16) << 15
    expo = (rng.integers(127 + lo, 127 + hi, size=shape, dtype=np.uint16) & 0xFF) << 7
    mant = rng.integers(0, 128, size=shape, dtype=np.uint16)
    return (sign | expo | mant).astype(np.uint16)


def test_sum_is_the_exact_rational_sum():
    rng = np.random.default_rng(31)
    for N in (1, 2, 5, 8, 16):
        x = _rand(rng, (N, 200))                    # 40 binades: binary64 holds them exactly
        s, a = oracle.sum_abs(list(x))
        for i in range(200):
            vals = [_val(x[r, i]) for r in range(N)]
            assert Fraction(s[i]) == sum(vals), (N, i)
            assert Fraction(a[i]) == sum(abs(v) for v in vals), (N, i)


def test_closed_forms():
    rng = np.random.default_rng(32)
    x = _rand(rng, 300)
    s, a = oracle.sum_abs([x, x ^ np.uint16(0x8000)])          # x + (-x)
    assert np.all(s == 0.0)
    v = np.array([float(_val(b)) for b in x])
    assert np.array_equal(a, 2 * np.abs(v))
    s, a = oracle.sum_abs([x] * 7)                             # identical copies
    assert np.array_equal(s, 7 * v) and np.array_equal(a, 7 * np.abs(v))
    z = np.zeros(10, np.uint16)
    s, a = oracle.sum_abs([z, z ^ np.uint16(0x8000), z])
    assert np.all(s == 0.0) and np.all(a == 0.0)


def test_arrival_order_folds_stay_within_the_bound():
    """Every order of binary32 additions (start 0, then each rank's value,
    as the shared accumulator sees them) lands within gamma_{N-1} * abs of
    the reference sum; and orders do disagree, so the bound is not vacuous."""
    rng = np.random.default_rng(33)
    differs = 0
    for N in (3, 4, 5):
        x = _rand(rng, (N, 40), -12, 12)
        s, a = oracle.sum_abs(list(x))
        g = (N - 1) * U / (1 - (N - 1) * U)
        for i in range(40):
            results = set()
            for perm in itertools.permutations(range(N)):
                acc = (exact.FIN, 0, Fraction(0))
                for r in perm:
                    acc = exact.round_to(exact.add_exact(acc, exact.decode(int(x[r, i]), exact.BF16)),
                                         exact.F32)
                got = acc[2]
                assert abs(got - Fraction(s[i])) <= g * Fraction(a[i]), (N, i, perm)
                results.add(got)
            differs += len(results) > 1
    assert differs > 0
