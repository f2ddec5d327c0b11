"""IEEE-754 binary32 / bfloat16 arithmetic from the definitions, in exact
rationals -- TEST INFRASTRUCTURE ONLY (pins the C oracle; never used by the
product path).

Nothing here uses floating-point hardware.  A value is decoded from its bit
pattern into (class, sign, Fraction); a sum is formed exactly; rounding to a
format picks the nearest representable value, ties to the one with an even
significand, and gives infinity when the rounded magnitude reaches 2**(emax+1)
(IEEE 754-2019 clause 4.3.1 and 7.4).  Zero signs follow clause 6.3: an exact
zero sum of operands of opposite sign is +0 under round-to-nearest; -0 + -0 is
-0.

The fold it checks is the reading of the "Every Microsecond Counts" write-up
("微秒必争…"), sections "张量并行与AllReduce" and "统一原语与API设计": sum the N
ranks' values; here in fixed rank order 0..N-1 with a binary32 accumulator
started from rank 0, then round the sum to bfloat16.
"""
from fractions import Fraction

# (exponent bits, stored mantissa bits)
BF16 = (8, 7)
F32 = (8, 23)

FIN, INF, NAN = "fin", "inf", "nan"


def _params(fmt):
    ebits, mbits = fmt
    bias = (1 << (ebits - 1)) - 1
    emin = 1 - bias
    emax = bias
    return ebits, mbits, bias, emin, emax


def decode(bits, fmt):
    """Bit pattern -> (class, sign, value); value is a Fraction for FIN."""
    ebits, mbits, bias, emin, _ = _params(fmt)
    width = 1 + ebits + mbits
    sign = (bits >> (width - 1)) & 1
    e = (bits >> mbits) & ((1 << ebits) - 1)
    m = bits & ((1 << mbits) - 1)
    if e == (1 << ebits) - 1:
        return (NAN, sign, None) if m else (INF, sign, None)
    if e == 0:
        mag = Fraction(m, 1) * Fraction(2) ** (emin - mbits)
    else:
        mag = Fraction((1 << mbits) + m, 1) * Fraction(2) ** (e - bias - mbits)
    return (FIN, sign, -mag if sign else mag)


def _floor_log2(q):
    """Largest e with 2**e <= q, for a positive Fraction q."""
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    elif Fraction(2) ** (e + 1) <= q:
        e += 1
    return e


def _rne_integer(q):
    """Round a non-negative Fraction to an integer, ties to even."""
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def encode(value, fmt):
    """(class, sign, Fraction) -> bit pattern, rounding FIN values RNE."""
    ebits, mbits, bias, emin, emax = _params(fmt)
    width = 1 + ebits + mbits
    cls, sign, q = value
    sbit = sign << (width - 1)
    exp_all = ((1 << ebits) - 1) << mbits
    if cls == NAN:
        return sbit | exp_all | (1 << (mbits - 1))
    if cls == INF:
        return sbit | exp_all
    a = abs(q)
    if a == 0:
        return sbit
    e = max(_floor_log2(a), emin)
    quantum = Fraction(2) ** (e - mbits)
    sig = _rne_integer(a / quantum)          # integer significand, may carry
    mag = sig * quantum
    if mag >= Fraction(2) ** (emax + 1):
        return sbit | exp_all                # overflow -> infinity
    if mag == 0:
        return sbit                          # rounded to a signed zero
    e2 = _floor_log2(mag)
    if e2 < emin:                            # subnormal
        field = int(mag / Fraction(2) ** (emin - mbits))
        return sbit | field
    frac = int(mag / Fraction(2) ** (e2 - mbits)) - (1 << mbits)
    return sbit | ((e2 + bias) << mbits) | frac


def round_to(value, fmt):
    """Round an exact value to fmt and decode it back (the value the format holds)."""
    return decode(encode(value, fmt), fmt)


def add_exact(a, b):
    """Exact sum of two decoded values, with IEEE class and zero-sign rules."""
    ca, sa, qa = a
    cb, sb, qb = b
    if ca == NAN or cb == NAN:
        return (NAN, 0, None)
    if ca == INF and cb == INF:
        return (INF, sa, None) if sa == sb else (NAN, 0, None)
    if ca == INF:
        return a
    if cb == INF:
        return b
    s = qa + qb
    if s == 0:
        # exact zero: -0 only when both operands are -0 (round-to-nearest)
        return (FIN, 1 if (sa == 1 and sb == 1 and qa == 0 and qb == 0) else 0, Fraction(0))
    return (FIN, 1 if s < 0 else 0, s)


def f32_add(a_bits, b_bits):
    """binary32 + binary32 -> binary32 bits, round to nearest even."""
    return encode(add_exact(decode(a_bits, F32), decode(b_bits, F32)), F32)


def f32_to_bf16(bits):
    """binary32 bits -> bfloat16 bits, round to nearest even (NaN -> quiet NaN)."""
    return encode(decode(bits, F32), BF16)


def fold_bf16(values):
    """Left fold of bfloat16 patterns in a binary32 accumulator, then to bfloat16.

    Returns the bfloat16 pattern of the result (NaN results as the quiet NaN
    pattern with the sign cleared; compare NaN results by class only).
    """
    acc = round_to(decode(values[0], BF16), F32)     # widening is exact
    for v in values[1:]:
        acc = round_to(add_exact(acc, decode(v, BF16)), F32)
    return encode(acc, BF16)


def fold_f32(values):
    """The binary32 accumulator (bits) of the same fold, before the bf16 rounding."""
    acc = round_to(decode(values[0], BF16), F32)
    for v in values[1:]:
        acc = round_to(add_exact(acc, decode(v, BF16)), F32)
    return encode(acc, F32)


def is_nan_bf16(bits):
    return (bits & 0x7F80) == 0x7F80 and (bits & 0x007F) != 0
