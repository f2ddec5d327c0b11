"""Pins of the CPU oracle against things other than itself.

The oracle (oracle/ar_oracle.c) computes the fixed-order AllReduce of the
"Every Microsecond Counts" write-up ("微秒必争…", sections "张量并行与AllReduce"
and "统一原语与API设计") under the reading: binary32 left fold over ranks
0..N-1 from rank 0's value, then binary32 -> bfloat16 round-to-nearest-even.

Its two arithmetic parts are pinned separately against IEEE 754 written out
in exact rational arithmetic (oracle/exact.py, which uses no float hardware):
  * the bf16 rounding: exhaustive over every upper half with the interesting
    lower halves (all rounding classes), plus every NaN/Inf class;
  * the binary32 fold: brute force over a 48-value set, N = 2 (all pairs) and
    N = 3 (all triples), plus random patterns at N up to 16.
And the whole reduction against hand-worked cases (tests/golden/), the order
witness, closed forms and invariants.
"""
import itertools
import os

import numpy as np
import pytest

import oracle
from oracle import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.txt")

# 48 bfloat16 values that exercise signed zeros, subnormals, the normal
# boundary, rounding ties around 1, large magnitudes near overflow and
# small integers.
V_POS = [0x0000, 0x0001, 0x007F, 0x0080, 0x3F80, 0x3F81, 0x3B80, 0x3B81,
         0x3C00, 0x4000, 0x4040, 0x4380, 0x3580, 0x4B80, 0x477F, 0x7F7F,
         0x7B00, 0x7A80, 0x3F00, 0x3FC0, 0x3DCD, 0x4049, 0x0040, 0x4B00]
V = V_POS + [v | 0x8000 for v in V_POS]


def _bf16_to_f32_bits(h):
    return (h & 0xFFFF) << 16


def _load_golden():
    cases = []
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            lhs, rhs = line.split("->")
            toks = lhs.split()
            n = int(toks[0])
            ins = [int(t, 16) for t in toks[1:]]
            assert len(ins) == n, line
            cases.append((ins, int(rhs.strip(), 16)))
    return cases


def test_exact_decoder_closed_forms():
    # spot values of the definitions themselves
    assert exact.decode(0x3F80, exact.BF16)[2] == 1
    assert exact.decode(0x0001, exact.BF16)[2] == exact.Fraction(1, 2 ** 133)
    assert exact.decode(0x7F7F, exact.BF16)[2] == 2 ** 128 - 2 ** 120
    assert exact.decode(0x00000001, exact.F32)[2] == exact.Fraction(1, 2 ** 149)
    assert exact.encode(exact.decode(0x7F7FFFFF, exact.F32), exact.F32) == 0x7F7FFFFF
    # every finite bf16 pattern survives a decode/encode round trip
    for h in range(0x10000):
        if exact.is_nan_bf16(h):
            continue
        assert exact.encode(exact.decode(h, exact.BF16), exact.BF16) == h


def test_bf16_rounding_sweep_against_exact():
    """Every upper half x lower halves {0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF}."""
    lows = [0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF]
    his = np.arange(0x10000, dtype=np.uint32)
    bits = (his[:, None] << 16 | np.array(lows, dtype=np.uint32)[None, :]).ravel()
    got = oracle.f32_to_bf16_array(bits)
    for b, g in zip(bits.tolist(), got.tolist()):
        want = exact.f32_to_bf16(b)
        if (b >> 23) & 0xFF == 0xFF and b & 0x7FFFFF:
            # NaN: stays NaN with its sign
            assert exact.is_nan_bf16(g) and (g >> 15) == (b >> 31), hex(b)
        else:
            assert g == want, (hex(b), hex(g), hex(want))


def test_f32_add_brute_force_pairs_against_exact():
    f = [_bf16_to_f32_bits(v) for v in V]
    for a in f:
        for b in f:
            assert oracle.f32_add_bits(a, b) == exact.f32_add(a, b), (hex(a), hex(b))


def _run_oracle_cases(cases_by_n):
    out = {}
    for n_ranks, tuples in cases_by_n.items():
        cols = np.array(tuples, dtype=np.uint16).T          # [N, cases]
        out[n_ranks] = oracle.allreduce(list(cols))
    return out


def test_fold_brute_force_n2_n3():
    pairs = list(itertools.product(V, repeat=2))
    triples = list(itertools.product(V, repeat=3))
    res = _run_oracle_cases({2: pairs, 3: triples})
    for n_ranks, tuples in ((2, pairs), (3, triples)):
        got = res[n_ranks]
        assert (got == got[0]).all(), "copies differ"
        for t, g in zip(tuples, got[0].tolist()):
            want = exact.fold_bf16(list(t))
            if exact.is_nan_bf16(want):
                assert exact.is_nan_bf16(g), t
            else:
                assert g == want, ([hex(x) for x in t], hex(g), hex(want))


@pytest.mark.parametrize("n_ranks", [2, 4, 5, 8, 16])
def test_fold_random_patterns(n_ranks):
    rng = np.random.Generator(np.random.PCG64(1234 + n_ranks))
    count = 400
    # random finite bf16 patterns over the whole exponent range
    pats = rng.integers(0, 0x10000, size=(n_ranks, count), dtype=np.uint32)
    pats = np.where((pats & 0x7F80) == 0x7F80, pats & 0xBFFF, pats).astype(np.uint16)
    # and patterns concentrated near one exponent so that sums cancel and round
    near = (0x3F00 + rng.integers(0, 0x100, size=(n_ranks, count))) | \
        (rng.integers(0, 2, size=(n_ranks, count)) << 15)
    for data in (pats, near.astype(np.uint16)):
        got = oracle.allreduce(list(data))
        acc = oracle.allreduce_f32(list(data))
        for i in range(count):
            col = [int(x) for x in data[:, i]]
            want = exact.fold_bf16(col)
            if exact.is_nan_bf16(want):
                assert exact.is_nan_bf16(int(got[0, i]))
            else:
                assert int(got[0, i]) == want, [hex(c) for c in col]
            assert int(acc.view(np.uint32)[i]) == exact.fold_f32(col) or \
                np.isnan(acc[i])


def test_golden_hand_cases():
    for ins, want in _load_golden():
        got = oracle.allreduce([np.array([x], dtype=np.uint16) for x in ins])
        assert all(int(g) == want for g in got[:, 0]), ([hex(x) for x in ins], hex(int(got[0, 0])), hex(want))
        assert exact.fold_bf16(ins) == want, [hex(x) for x in ins]


def test_order_witness():
    """A left fold, a right fold and a rank-permuted fold give different bits."""
    a = [0x4380, 0xC380, 0x3580]              # 256, -256, 2^-20
    assert oracle.allreduce([np.array([x], np.uint16) for x in a])[0, 0] == 0x3580
    perm = [0x3580, 0x4380, 0xC380]
    assert oracle.allreduce([np.array([x], np.uint16) for x in perm])[0, 0] == 0x0000
    # the right fold x0 + (x1 + x2) of the first order would be +0: not what the oracle does
    right = exact.encode(exact.round_to(exact.add_exact(
        exact.decode(0x4380, exact.BF16),
        exact.round_to(exact.add_exact(exact.decode(0xC380, exact.BF16),
                                       exact.decode(0x3580, exact.BF16)), exact.F32)),
        exact.F32), exact.BF16)
    assert right == 0x0000


def test_identity_single_rank_all_patterns():
    pats = np.arange(0x10000, dtype=np.uint16)
    got = oracle.allreduce([pats])[0]
    nan = ((pats & 0x7F80) == 0x7F80) & ((pats & 0x7F) != 0)
    assert (got[~nan] == pats[~nan]).all()
    assert (((got[nan] & 0x7F80) == 0x7F80) & ((got[nan] & 0x7F) != 0)).all()


def test_zero_and_sign_invariants():
    n = 257
    for n_ranks in (2, 3, 8, 16):
        pz = [np.zeros(n, np.uint16)] * n_ranks
        nz = [np.full(n, 0x8000, np.uint16)] * n_ranks
        assert (oracle.allreduce(pz) == 0x0000).all()
        assert (oracle.allreduce(nz) == 0x8000).all()


def test_one_nonzero_rank_gives_that_value():
    rng = np.random.Generator(np.random.PCG64(7))
    n = 1000
    x = rng.integers(0, 0x10000, size=n, dtype=np.uint32).astype(np.uint16)
    x = np.where((x & 0x7F80) == 0x7F80, x & 0xBFFF, x).astype(np.uint16)
    x = np.where(x == 0x8000, 0x0000, x).astype(np.uint16)   # -0 + +0 = +0, excluded
    for n_ranks in (2, 5, 16):
        for pos in (0, n_ranks // 2, n_ranks - 1):
            ranks = [np.zeros(n, np.uint16) for _ in range(n_ranks)]
            ranks[pos] = x
            assert (oracle.allreduce(ranks) == x).all()


def test_small_integers_exact_and_permutation_invariant():
    rng = np.random.Generator(np.random.PCG64(11))
    n_ranks, n = 8, 2000
    ints = rng.integers(-32, 33, size=(n_ranks, n))
    f32 = ints.astype(np.float32)
    bits = (f32.view(np.uint32) >> 16).astype(np.uint16)   # small integers are exact in bf16
    assert ((bits.astype(np.uint32) << 16).view(np.float32) == f32).all()
    want = ints.sum(axis=0).astype(np.float32)             # |sum| <= 256: exact in bf16
    base = oracle.allreduce(list(bits))
    assert ((base[0].astype(np.uint32) << 16).view(np.float32) == want).all()
    for perm in ([7, 6, 5, 4, 3, 2, 1, 0], [3, 0, 7, 1, 6, 2, 5, 4]):
        assert (oracle.allreduce(list(bits[perm])) == base).all()


def test_pairs_cancel_to_plus_zero():
    rng = np.random.Generator(np.random.PCG64(5))
    x = rng.integers(0, 0x7F80, size=500, dtype=np.uint32).astype(np.uint16)
    got = oracle.allreduce([x, x ^ 0x8000])
    assert (got == 0).all()


def test_copies_identical_and_threads_agree():
    rng = np.random.Generator(np.random.PCG64(3))
    data = rng.integers(0, 0x7F00, size=(8, 4099), dtype=np.uint32).astype(np.uint16)
    a = oracle.allreduce(list(data), threads=1)
    b = oracle.allreduce(list(data), threads=4)
    assert (a == a[0]).all()
    assert (a == b).all()
