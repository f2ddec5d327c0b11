"""Pins of the residual-add + RMS-norm oracle (oracle.add_rmsnorm),
independent of it: exact binary32 addition and rounding (oracle/exact.py),
closed forms, invariances, and a 60-digit decimal computation of y."""
from decimal import Decimal, getcontext

import numpy as np

import oracle
from oracle import exact


def _val(h):
    cls, _, v = exact.decode(int(h), exact.BF16)
    assert cls == exact.FIN
    return v


def _rand(rng, n, lo=-30, hi=30):
    sign = rng.integers(0, 2, size=n, dtype=np.uint16) << 15
    expo = (rng.integers(127 + lo, 127 + hi, size=n, dtype=np.uint16) & 0xFF) << 7
    mant = rng.integers(0, 128, size=n, dtype=np.uint16)
    return (sign | expo | mant).astype(np.uint16)


def test_residual_add_is_binary32_add_rounded_once():
    rng = np.random.default_rng(21)
    n = 500
    a, res, g = _rand(rng, n), _rand(rng, n), _rand(rng, n, -4, 4)
    h, _ = oracle.add_rmsnorm(a, res, g, 1e-5)
    for i in range(n):
        s32 = exact.f32_add(int(a[i]) << 16, int(res[i]) << 16)
        assert h[i] == exact.f32_to_bf16(s32), i


def test_y_matches_decimal_computation():
    getcontext().prec = 60
    rng = np.random.default_rng(8)
    for n in (1, 7, 64, 300):
        a, res, g = _rand(rng, n, -6, 6), _rand(rng, n, -6, 6), _rand(rng, n, -2, 2)
        eps = np.float32(1e-6)
        h, y = oracle.add_rmsnorm(a, res, g, eps)
        hv = [Decimal(_val(x).numerator) / Decimal(_val(x).denominator) for x in h]
        ms = sum(v * v for v in hv) / Decimal(n) + Decimal(float(eps))
        inv = 1 / ms.sqrt()
        for i in range(n):
            gv = Decimal(_val(g[i]).numerator) / Decimal(_val(g[i]).denominator)
            want = hv[i] * gv * inv
            assert abs(Decimal(y[i]) - want) <= abs(want) * Decimal(2) ** -48 + Decimal(2) ** -1000


def test_closed_forms():
    n = 128
    one = np.uint16(0x3F80)
    zero = np.zeros(n, dtype=np.uint16)
    c = np.full(n, np.uint16(0x4040), dtype=np.uint16)           # 3.0
    # constant row, eps = 0: every y is gamma (sign of c)
    h, y = oracle.add_rmsnorm(c, zero, np.full(n, one), 0.0)
    assert np.all(h == 0x4040) and np.allclose(y, 1.0, rtol=0, atol=1e-15)
    # a = -res: h is +0 everywhere, y = 0
    rng = np.random.default_rng(2)
    r = _rand(rng, n)
    h, y = oracle.add_rmsnorm(r ^ np.uint16(0x8000), r, np.full(n, one), 1e-5)
    assert np.all(h == 0) and np.all(y == 0)
    # gamma = 0 gives 0
    _, y = oracle.add_rmsnorm(_rand(rng, n), zero, zero, 1e-5)
    assert np.all(y == 0)


def test_scale_invariance_without_eps():
    rng = np.random.default_rng(4)
    n = 256
    a, g = _rand(rng, n, -10, 10), _rand(rng, n, -2, 2)
    zero = np.zeros(n, dtype=np.uint16)
    _, y1 = oracle.add_rmsnorm(a, zero, g, 0.0)
    _, y2 = oracle.add_rmsnorm((a + np.uint16(1 << 7)).astype(np.uint16), zero, g, 0.0)  # 2a
    assert np.allclose(y1, y2, rtol=1e-14, atol=0)
