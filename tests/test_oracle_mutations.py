"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of the C oracle (on the CPU, in a
temporary directory), builds it, and checks that the hand-worked golden cases
plus the exact-arithmetic rounding pins reject it.  The real oracle must pass
the same checks.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

from oracle import exact

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "ar_oracle.c")
GOLDEN = os.path.join(HERE, "golden", "hand_cases.txt")

MUTANTS = {
    "ties_away_from_zero": ("if (rest > 0x8000u || (rest == 0x8000u && (hi & 1u)))",
                            "if (rest >= 0x8000u)"),
    "truncating_conversion": ("hi += 1u;", "hi += 0u;"),
    "fold_starts_at_plus_zero": ("float acc = widen_bf16(in[0][i]);\n    for (int r = 1;",
                                 "float acc = 0.0f;\n    for (int r = 0;"),
    "reversed_rank_order": ("for (int r = 1; r < n_ranks; ++r)\n        acc = acc + widen_bf16(in[r][i]);",
                            "for (int r = n_ranks - 1; r >= 1; --r)\n        acc = acc + widen_bf16(in[r][i]);"),
    "dropped_last_rank": ("for (int r = 1; r < n_ranks; ++r)\n        acc = acc + widen_bf16(in[r][i]);",
                          "for (int r = 1; r < n_ranks - 1; ++r)\n        acc = acc + widen_bf16(in[r][i]);"),
    "nan_not_quieted": ("| 0x0040u", "| 0x0000u"),
    "sign_lost": ("return (uint16_t)hi;", "return (uint16_t)(hi & 0x7FFFu);"),
}


def _build(tmp_path, name, src_text):
    c = tmp_path / (name + ".c")
    so = tmp_path / (name + ".so")
    c.write_text(src_text)
    subprocess.run(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c11", "-fPIC",
                    "-shared", "-fopenmp", str(c), "-o", str(so)], check=True)
    L = ctypes.CDLL(str(so))
    L.oracle_allreduce_bf16.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                                        ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int]
    L.oracle_f32_to_bf16.argtypes = [ctypes.c_uint32]
    L.oracle_f32_to_bf16.restype = ctypes.c_uint16
    return L


def _golden_cases():
    cases = []
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if line:
            lhs, rhs = line.split("->")
            toks = lhs.split()
            cases.append(([int(t, 16) for t in toks[1:]], int(rhs, 16)))
    return cases


def _pins_pass(L):
    """True when library L passes the golden cases and a rounding sample."""
    for ins, want in _golden_cases():
        arrs = [np.array([x], dtype=np.uint16) for x in ins]
        ptrs = (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])
        out = np.empty(len(arrs), dtype=np.uint16)
        L.oracle_allreduce_bf16(ptrs, len(arrs), 1, out.ctypes.data, 1)
        if any(int(o) != want for o in out):
            return False
    rng = np.random.Generator(np.random.PCG64(99))
    sample = rng.integers(0, 2 ** 32, size=3000, dtype=np.uint64).tolist()
    sample += [0x3F808000, 0x3F818000, 0xBF808000, 0x7FC00001, 0xFF800001, 0x7F7F8000]
    for b in sample:
        g = int(L.oracle_f32_to_bf16(b))
        if (b >> 23) & 0xFF == 0xFF and b & 0x7FFFFF:
            if not exact.is_nan_bf16(g) or (g >> 15) != (b >> 31):
                return False
        elif g != exact.f32_to_bf16(b):
            return False
    return True


def test_real_oracle_passes(tmp_path):
    assert _pins_pass(_build(tmp_path, "real", open(SRC).read()))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert old in text, "mutation anchor missing: %s" % name
    assert not _pins_pass(_build(tmp_path, name, text.replace(old, new, 1)))
