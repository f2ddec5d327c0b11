"""The norm tests' comparison helper (tests/norm_util.py) against brute
force: bf16_rne picks the nearest bf16 value (ties to the even pattern) by
exact rational distance, and y_violations accepts exactly the interval."""
from fractions import Fraction

import numpy as np

from norm_util import bf16_rne, bf16_value, y_violations


def _nearest_bf16(y):
    """Brute force: the bf16 value nearest to y, ties to even mantissa."""
    f = Fraction(y)
    bits = int(np.array([y], dtype=np.float32).view(np.uint32)[0] >> 16)
    best = None
    for b in range(max(bits - 3, 0), bits + 4):
        for s in (b, b | 0x8000):
            v = bf16_value(np.array([s], dtype=np.uint16))[0]
            if not np.isfinite(v):
                continue
            d = abs(Fraction(float(v)) - f)
            key = (d, s & 1)                       # ties: even pattern first
            if best is None or key < best[0]:
                best = (key, float(v))
    return best[1]


def test_bf16_rne_matches_brute_force():
    rng = np.random.default_rng(5)
    ys = np.concatenate([rng.normal(0, 1, 300), rng.normal(0, 1e-3, 100),
                         np.ldexp(rng.uniform(1, 2, 50), rng.integers(-130, -120, 50)),
                         np.ldexp(rng.uniform(1, 2, 50), rng.integers(60, 120, 50))])
    for y in ys:
        assert bf16_rne(np.array([y]))[0] == _nearest_bf16(float(y)), y


def test_bf16_rne_ties_go_to_even():
    # 1 + 2^-8 lies halfway between 1 (even) and 1 + 2^-7 (odd)
    assert bf16_rne(np.array([1 + 2.0 ** -8]))[0] == 1.0
    # 1 + 3 * 2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert bf16_rne(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    assert bf16_rne(np.array([-(1 + 2.0 ** -8)]))[0] == -1.0
    assert bf16_rne(np.array([0.0]))[0] == 0.0


def test_y_violations_interval():
    y = np.array([1.0 + 2.0 ** -8])                   # a tie: both neighbours allowed
    one = np.array([0x3F80], dtype=np.uint16)         # 1.0
    up = np.array([0x3F81], dtype=np.uint16)          # 1 + 2^-7
    assert y_violations(one, y).size == 0
    assert y_violations(up, y).size == 0
    y = np.array([1.0 + 2.0 ** -10])                  # well inside: only 1.0
    assert y_violations(one, y).size == 0
    assert y_violations(up, y).size == 1
    assert y_violations(np.array([0x3F7F], dtype=np.uint16), y).size == 1


def test_atomic_interval():
    """The atomic variant's acceptance interval: for an exactly representable
    sum only that value passes; where the slack straddles a rounding
    boundary both neighbours pass, and nothing further out."""
    from atomic_util import bf16_violations, slack
    s = np.array([3.0])
    a = np.array([3.0])
    assert bf16_violations(np.array([0x4040], np.uint16), s, a, 2).size == 0      # 3.0
    assert bf16_violations(np.array([0x4041], np.uint16), s, a, 2).size == 1
    # a sum sitting on the midpoint between 1 and 1 + 2^-7, with a large sum|x|
    s = np.array([1.0 + 2.0 ** -8])
    a = np.array([2.0 ** 10])
    assert slack(8, a)[0] > 2.0 ** -14
    for bits, bad in ((0x3F80, 0), (0x3F81, 0), (0x3F82, 1), (0x3F7F, 1)):
        assert bf16_violations(np.array([bits], np.uint16), s, a, 8).size == bad, hex(bits)
