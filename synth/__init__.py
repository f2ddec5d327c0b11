"""Seeded synthetic inputs for the AllReduce workloads.

This module is shared by the oracle side and the GPU side of every test and
of the benchmark, and by nothing else.  It holds none of the reduction's
arithmetic: it draws binary32 values with numpy's PCG64 and keeps the upper
16 bits of each draw as the bfloat16 pattern (truncation toward zero -- a
property of the synthetic recipe, deliberately not the reduction's
round-to-nearest-even), so that the two sides of a parity test share no
rounding code.

Workloads stand in for tensor-parallel decode activations: the hidden size
8192 with 80 layers and two AllReduces per layer ("vLLM 分布式推理核心：NCCL 集合
通信与 CUDA Stream 异步掩盖实战", section 一) and batch-1 decode messages of tens
to hundreds of KB ("微秒必争…", section "张量并行与AllReduce").  No dataset is
involved.
"""
from dataclasses import dataclass

import numpy as np

SEED_BASE = 20261202


@dataclass(frozen=True)
class Workload:
    cid: int                 # 1..5
    name: str
    n_ranks: int
    rows: int
    hidden: int
    dist: str                # "normal" | "normal_outliers" | "uniform"
    scale: float             # sigma for normal, half-width for uniform
    sets: int                # rotating input sets
    calls: int               # calls in the workload's run
    outlier_frac: float = 0.0
    outlier_mult: float = 1.0
    delay_max_ns: int = 0

    @property
    def n(self) -> int:
        """Elements per rank."""
        return self.rows * self.hidden

    @property
    def bytes_per_rank(self) -> int:
        return 2 * self.n


WORKLOADS = {
    1: Workload(1, "4 ranks x [1x4096] bf16, N(0,1), 1000 calls", 4, 1, 4096,
                "normal", 1.0, sets=4, calls=1000),
    2: Workload(2, "8 ranks x [1x8192] bf16 (16 KiB/rank), N(0,0.5), 160 calls/step", 8, 1, 8192,
                "normal", 0.5, sets=4, calls=160),
    3: Workload(3, "8 ranks x [32x8192] bf16 (512 KiB/rank), N(0,1) + 1% x100 outliers, 160 calls/step",
                8, 32, 8192, "normal_outliers", 1.0, sets=4, calls=160,
                outlier_frac=0.01, outlier_mult=100.0),
    4: Workload(4, "8 ranks x [256x8192] bf16 (4 MiB/rank), U(-1,1)", 8, 256, 8192,
                "uniform", 1.0, sets=8, calls=200),
    5: Workload(5, "16 ranks x [8x7168] bf16, N(0,1), 0-5 us start delays, 10000 calls", 16, 8, 7168,
                "normal", 1.0, sets=8, calls=10000, delay_max_ns=5000),
}


def seed_for(cid: int, set_idx: int, rank: int) -> int:
    return SEED_BASE + 1000 * cid + 100 * set_idx + rank


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """binary32 draw -> bfloat16 pattern by keeping the upper half (truncation)."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def draw(rng: np.random.Generator, n: int, dist: str, scale: float = 1.0,
         outlier_frac: float = 0.0, outlier_mult: float = 1.0) -> np.ndarray:
    """n bfloat16 patterns from one distribution."""
    if dist in ("normal", "normal_outliers"):
        x = rng.normal(0.0, scale, size=n).astype(np.float32)
        if dist == "normal_outliers" and n:
            k = int(round(outlier_frac * n))
            idx = rng.permutation(n)[:k]
            x[idx] = x[idx] * np.float32(outlier_mult)
    elif dist == "uniform":
        x = rng.uniform(-scale, scale, size=n).astype(np.float32)
    else:
        raise ValueError("unknown distribution %r" % dist)
    return _to_bf16_bits(x)


def rank_input(cid: int, set_idx: int, rank: int, n: int = None) -> np.ndarray:
    """Rank `rank`'s input of rotating set `set_idx` of workload `cid` (uint16 [n])."""
    w = WORKLOADS[cid]
    n = w.n if n is None else n
    rng = np.random.Generator(np.random.PCG64(seed_for(cid, set_idx, rank)))
    return draw(rng, n, w.dist, w.scale, w.outlier_frac, w.outlier_mult)


def input_set(cid: int, set_idx: int, n: int = None, n_ranks: int = None) -> np.ndarray:
    """All ranks' inputs of one set: uint16 [N, n]."""
    w = WORKLOADS[cid]
    N = w.n_ranks if n_ranks is None else n_ranks
    return np.stack([rank_input(cid, set_idx, r, n) for r in range(N)])


def delays_ns(cid: int, calls: int = None, n_ranks: int = None) -> np.ndarray:
    """Per (call, rank) start delays, uint32 [calls, N], uniform on [0, delay_max_ns]."""
    w = WORKLOADS[cid]
    calls = w.calls if calls is None else calls
    N = w.n_ranks if n_ranks is None else n_ranks
    rng = np.random.Generator(np.random.PCG64(SEED_BASE + 1000 * cid + 999))
    return rng.integers(0, w.delay_max_ns + 1, size=(calls, N), dtype=np.uint32)


def random_bits(seed: int, shape, finite_only: bool = True, avoid: int = None) -> np.ndarray:
    """Uniformly random bfloat16 patterns (edge-case tests); optionally finite only
    and never equal to `avoid`."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.integers(0, 0x10000, size=shape, dtype=np.uint32)
    if finite_only:
        x = np.where((x & 0x7F80) == 0x7F80, x & 0xBFFF, x)
    x = x.astype(np.uint16)
    if avoid is not None:
        x = np.where(x == avoid, np.uint16(0), x).astype(np.uint16)
    return x


NORM_EPS = 1e-5


def norm_operands(cid: int, set_idx: int, n_ranks: int = None, replicated: bool = False):
    """Operands of the residual add + RMS norm after workload `cid`'s AllReduce:
    residuals uint16 [N, n] drawn N(0, 2) (the residual stream), gamma uint16
    [hidden] drawn N(1, 0.2) (a trained norm weight's typical spread).  With
    replicated=True every rank holds the same residual, as in tensor-parallel
    decode; otherwise each rank's is drawn separately, so that a kernel which
    mixes up ranks' residuals cannot pass."""
    w = WORKLOADS[cid]
    N = w.n_ranks if n_ranks is None else n_ranks
    base = SEED_BASE + 100000 + 1000 * cid + 20 * set_idx     # apart from the input seeds
    res = []
    for r in range(N):
        rng = np.random.Generator(np.random.PCG64(base + (0 if replicated else r)))
        res.append(draw(rng, w.n, "normal", 2.0))
    rng = np.random.Generator(np.random.PCG64(base + 19))
    gamma = _to_bf16_bits(rng.normal(1.0, 0.2, size=w.hidden).astype(np.float32))
    return np.stack(res), gamma


def bounded_bits(seed: int, shape, exp_lo: int = -30, exp_hi: int = 30) -> np.ndarray:
    """Random finite bfloat16 patterns with unbiased exponents in [exp_lo,
    exp_hi) and random sign and mantissa: wide dynamic range, no overflow
    when up to 16 of them are summed (edge cases of the arrival-order
    variant, whose bound assumes no overflow)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    sign = rng.integers(0, 2, size=shape, dtype=np.uint32) << 15
    expo = rng.integers(127 + exp_lo, 127 + exp_hi, size=shape, dtype=np.uint32) << 7
    mant = rng.integers(0, 128, size=shape, dtype=np.uint32)
    return (sign | expo | mant).astype(np.uint16)
