"""Comparison helpers for the residual add + RMS norm tests.

The oracle returns y unrounded in binary64.  A kernel computes
z = (h * r) * gamma in binary32, with r = 1 / sqrt(S / hidden + eps) and S
a binary32 sum of the squares of bf16 values (exact products, at most 18
roundings deep for rows of up to 65536 elements: 3 per lane, 6 per wave,
3 + 6 across the row's blocks), then rounds z once to bf16.  For sums of
non-negative terms the relative error of S is at most (1+u)^18 - 1 with
u = 2^-24; division by hidden, the eps add, the square root, the reciprocal
and the two products add about 4.5 u after the square root halves the rest,
so |z - y| <= 14 u |y| < 2^-20 |y|.  The test allows twice that:
got must equal bf16_rne(z) for some z within Y_REL = 2^-19 of y relatively,
i.e. lie between bf16_rne(y - Y_REL |y|) and bf16_rne(y + Y_REL |y|)
(rounding is monotonic).  That is far inside one bf16 unit in the last
place (2^-8 relative), so a dropped term, wrong eps, wrong row or wrong
gamma index fails.
"""
import numpy as np

Y_REL = 2.0 ** -19


def bf16_rne(y):
    """binary64 values -> nearest bfloat16 values (ties to even), as binary64.

    Exact: for |y| in [2^(e-1), 2^e) the bf16 spacing is 2^(e-8) (e clamped
    to -125 below the smallest normal), y * 2^(8-e) is exact in binary64 and
    numpy's rint rounds half to even."""
    y = np.asarray(y, dtype=np.float64)
    ay = np.abs(y)
    _, e = np.frexp(ay)
    e = np.maximum(e, -125)
    q = np.rint(np.ldexp(ay, 8 - e))
    return np.copysign(np.ldexp(q, e - 8), y)


def bf16_value(bits):
    """uint16 bf16 patterns -> binary64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def y_violations(got_bits, y_exact, rel=Y_REL):
    """Indices where a kernel's bf16 y is outside the allowed rounding interval."""
    got = bf16_value(got_bits)
    y = np.asarray(y_exact, dtype=np.float64)
    lo = bf16_rne(y - rel * np.abs(y))
    hi = bf16_rne(y + rel * np.abs(y))
    ok = (got >= lo) & (got <= hi)
    ok |= np.isnan(got) & np.isnan(y)
    return np.nonzero(~ok)[0]


def expected(a_bits, residuals, gamma, eps, rows, hidden, oracle):
    """Oracle h [N, n] (uint16) and y [N, n] (binary64) for the AllReduce
    result a [n] shared by all ranks and per-rank residuals [N, n]."""
    N, n = residuals.shape
    h = np.empty((N, n), dtype=np.uint16)
    y = np.empty((N, n), dtype=np.float64)
    for r in range(N):
        for i in range(rows):
            sl = slice(i * hidden, (i + 1) * hidden)
            h[r, sl], y[r, sl] = oracle.add_rmsnorm(a_bits[sl], residuals[r, sl], gamma, eps)
    return h, y
