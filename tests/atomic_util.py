"""Comparison of the arrival-order atomic variant with the oracle's exact
sum.  Any order of the N-1 binary32 additions lies within
gamma_{N-1} * sum|x| (gamma_k = k u / (1 - k u), u = 2^-24) of the exact sum
(pinned in tests/test_atomic_oracle.py); the reference sum from
oracle.sum_abs is itself within (N-1) 2^-53 sum|x| of it.  A bf16 output is
acceptable when it is the round-to-nearest-even of some binary32 value in
that interval, i.e. lies between the roundings of its two ends."""
import numpy as np

from norm_util import bf16_rne, bf16_value


def slack(N, abs_sum):
    u = 2.0 ** -24
    g = (N - 1) * u / (1 - (N - 1) * u)
    return (g + N * 2.0 ** -50) * np.asarray(abs_sum, dtype=np.float64)


def bf16_violations(got_bits, ref_sum, abs_sum, N):
    got = bf16_value(got_bits)
    d = slack(N, abs_sum)
    lo = bf16_rne(ref_sum - d)
    hi = bf16_rne(ref_sum + d)
    return np.nonzero(~((got >= lo) & (got <= hi)))[0]


def f32_violations(got_f32, ref_sum, abs_sum, N):
    got = np.asarray(got_f32, dtype=np.float32).astype(np.float64)
    return np.nonzero(np.abs(got - ref_sum) > slack(N, abs_sum))[0]


def ulp_distance(got_bits, want_bits):
    """|got - want| in bf16 units in the last place of want (finite values)."""
    g = bf16_value(got_bits)
    w = bf16_value(want_bits)
    ulp = np.ldexp(1.0, np.maximum(np.frexp(np.abs(w))[1], -125) - 8)
    return np.abs(g - w) / ulp
