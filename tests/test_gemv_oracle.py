"""Pins of the decode-projection oracle (oracle.gemv), independent of it:
exact rational dot products, closed forms and exact linearity."""
from fractions import Fraction

import numpy as np

import oracle
from oracle import exact


def _bf16_value(h):
    cls, _, value = exact.decode(int(h), exact.BF16)
    assert cls == exact.FIN
    return value


def _random_bf16(rng, shape, lo=-40, hi=40):
    """bf16 patterns with mixed exponents (finite, no subnormal extremes)."""
    sign = rng.integers(0, 2, size=shape, dtype=np.uint16) << 15
    expo = (rng.integers(127 + lo, 127 + hi, size=shape, dtype=np.uint16) & 0xFF) << 7
    mant = rng.integers(0, 128, size=shape, dtype=np.uint16)
    return (sign | expo | mant).astype(np.uint16)


def test_matches_exact_rational_dot_products():
    """Against sums of exact rational products: the binary64 result is within
    K * 2^-53 * sum|w x| of the exact value (products are exact in binary64)."""
    rng = np.random.default_rng(11)
    for M, K in ((3, 40), (5, 17), (2, 200)):
        W = _random_bf16(rng, (M, K))
        x = _random_bf16(rng, (K,))
        y = oracle.gemv(W, x)
        for m in range(M):
            terms = [_bf16_value(W[m, k]) * _bf16_value(x[k]) for k in range(K)]
            ex = sum(terms, Fraction(0))
            bound = Fraction(K) * Fraction(1, 2 ** 53) * sum(abs(t) for t in terms)
            assert abs(Fraction(y[m]) - ex) <= bound, (M, K, m)


def test_integer_dot_products_are_exact():
    rng = np.random.default_rng(5)
    M, K = 7, 64
    Wi = rng.integers(-8, 9, size=(M, K))
    xi = rng.integers(-8, 9, size=K)
    to_bf16 = lambda a: (np.asarray(a, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y = oracle.gemv(to_bf16(Wi), to_bf16(xi))
    assert np.array_equal(y, (Wi @ xi).astype(np.float64))


def test_closed_forms():
    K = 96
    one = np.uint16(0x3F80)
    assert np.all(oracle.gemv(np.full((4, K), one), np.full(K, one)) == K)
    # identity rows pick out x exactly
    rng = np.random.default_rng(3)
    x = _random_bf16(rng, (K,))
    eye = np.where(np.eye(K, dtype=bool), one, np.uint16(0)).astype(np.uint16)
    want = np.array([float(_bf16_value(h)) for h in x])
    assert np.array_equal(oracle.gemv(eye, x), want)
    # a row [a, -a, b] gives b
    a, b = np.uint16(0x4321), np.uint16(0x3E55)
    W = np.array([[a, a | 0x8000, b]], dtype=np.uint16)
    assert oracle.gemv(W, np.array([one, one, one], dtype=np.uint16))[0] == float(_bf16_value(b))


def test_scaling_by_two_is_exact():
    rng = np.random.default_rng(9)
    W = _random_bf16(rng, (6, 50), -20, 20)
    x = _random_bf16(rng, (50,), -20, 20)
    x2 = (x + np.uint16(1 << 7)).astype(np.uint16)        # exponent + 1: each x doubled
    assert np.array_equal(oracle.gemv(W, x2), 2.0 * oracle.gemv(W, x))
