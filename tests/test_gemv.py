"""The decode projection of the overlap harness on the GPU (include/ar_gemv.h)
against the oracle, and the projection feeding the AllReduce.

Bound.  The kernel sums each row in binary32: lane l adds its K/64 products
in order (fused multiply-adds), then 6 butterfly levels combine the lanes,
then one bf16 rounding.  So |y_gpu - y| <= 2^-8 |y| + 1.01 d 2^-24 sum|w x|
with d = ceil(K/512)*8 + 6 additions on the longest path, plus a tiny
absolute term for subnormal results; y is the oracle's binary64 sum."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import ar_context, assert_bits_equal, host_bits, log, torch_mod

pytestmark = pytest.mark.gpu


def _bf16(a):
    """float array -> bf16 patterns (truncation, as the input recipe does)."""
    return (np.asarray(a, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _value(h):
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _problem(seed, N, M, K):
    rng = np.random.default_rng(seed)
    W = [_bf16(rng.normal(0.0, 1.0 / np.sqrt(K), size=(M, K))) for _ in range(N)]
    x = [_bf16(rng.normal(0.0, 1.0, size=K)) for _ in range(N)]
    return W, x


def _run(W, x, M, K, stream=None, cap=0):
    import tp_decode_comms_amd as ar
    torch = torch_mod()
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16).copy()).to("cuda:0")
    Wd = [dev(w) for w in W]
    xd = [dev(v) for v in x]
    yd = [torch.empty(M, dtype=torch.int16, device="cuda:0") for _ in W]
    ar.gemv(Wd, xd, yd, M, K, stream=stream, max_workgroups=cap)
    return Wd, xd, yd


def _check(W, x, y_bits, K):
    d = -(-K // 512) * 8 + 6
    for r in range(len(W)):
        ref = oracle.gemv(W[r], x[r], threads=0)
        mag = np.abs(_value(W[r])) @ np.abs(_value(x[r]))
        got = _value(y_bits[r])
        tol = 2.0 ** -8 * np.abs(ref) + 1.01 * d * 2.0 ** -24 * mag + 2.0 ** -130
        bad = np.nonzero(np.abs(got - ref) > tol)[0]
        assert bad.size == 0, "rank %d row %d: got %r want %r tol %r" % (
            r, bad[0], got[bad[0]], ref[bad[0]], tol[bad[0]])


@pytest.mark.parametrize("N,M,K,cap", [(8, 8192, 1024, 0), (3, 37, 200, 0), (1, 1, 8, 0),
                                       (16, 515, 64 * 8 + 8, 0), (8, 8192, 1024, 96)])
def test_gemv_within_binary32_bound(N, M, K, cap):
    log("gemv N=%d M=%d K=%d cap=%d" % (N, M, K, cap))
    torch = torch_mod()
    W, x = _problem(100 + N + M, N, M, K)
    _, _, yd = _run(W, x, M, K, cap=cap)
    torch.cuda.synchronize()
    _check(W, x, [host_bits(y) for y in yd], K)


def test_projection_feeds_allreduce_bit_exact():
    """GEMV -> AllReduce on one stream (the dependent decode step): the
    AllReduce of the GPU's projections equals the oracle's fold of them."""
    log("gemv -> allreduce")
    torch = torch_mod()
    N, M, K = 8, 8192, 1024
    W, x = _problem(7, N, M, K)
    stream = torch.cuda.Stream()
    import tp_decode_comms_amd as ar
    with ar_context(N, M) as a:
        with torch.cuda.stream(stream):
            Wd, xd, yd = _run(W, x, M, K, stream=stream)
            out = torch.empty((N, M), dtype=torch.int16, device="cuda:0")
            a.allreduce(yd, out, M, 1, stream=stream)
        torch.cuda.synchronize()
        ys = [host_bits(y) for y in yd]
        _check(W, x, ys, K)
        assert_bits_equal(host_bits(out), oracle.allreduce(ys))


@pytest.mark.parametrize("cap", [0, 1024], ids=["full-projection", "budgeted-projection"])
def test_concurrent_overlap_graph(cap):
    """The overlap harness's concurrent form (the compute stream behind one
    event, the communication stream behind another, "vLLM 分布式推理核心"
    page, sections 二 and 三): one hipGraph holds `layers` projections on one
    stream and `layers` independent AllReduces (16 KiB per rank, one-shot LL)
    on a second, forked from and joined back to the first with events.  The
    graph is replayed three times, with the outputs poisoned before each
    replay; every AllReduce output must be bit-exact against the oracle and
    every projection within its binary32 bound, after every replay."""
    import tp_decode_comms_amd as ar
    log("concurrent overlap graph, projection cap %d" % cap)
    torch = torch_mod()
    N, M, K, layers = 8, 8192, 1024, 6
    W, x = _problem(11, N, M, K)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16).copy()).to("cuda:0")
    Wd = [dev(w) for w in W]
    xd = [dev(v) for v in x]
    yd = [torch.empty(M, dtype=torch.int16, device="cuda:0") for _ in range(N)]
    sets = [synth.input_set(2, s) for s in range(3)]
    ins = [[dev(d[r]) for r in range(N)] for d in sets]
    want = [oracle.allreduce(list(d)) for d in sets]
    outs = [torch.empty((N, M), dtype=torch.int16, device="cuda:0") for _ in range(layers)]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    with ar_context(N, M, 1, 1) as a:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s1):
            with torch.cuda.graph(g, stream=s1):
                fork = torch.cuda.Event()
                fork.record(s1)
                s2.wait_event(fork)
                for _ in range(layers):
                    ar.gemv(Wd, xd, yd, M, K, stream=s1, max_workgroups=cap)
                for k in range(layers):
                    a.allreduce(ins[k % 3], outs[k], M, k + 1, stream=s2)
                a.step_end(stream=s2)
                join = torch.cuda.Event()
                join.record(s2)
                s1.wait_event(join)
        torch.cuda.synchronize()
        for rep in range(3):
            with torch.cuda.stream(s1):
                for o in outs:
                    o.fill_(-1)
                for y in yd:
                    y.fill_(-1)
                g.replay()
            torch.cuda.synchronize()
            for k in range(layers):
                assert_bits_equal(host_bits(outs[k]), want[k % 3], "replay %d call %d" % (rep, k))
            _check(W, x, [host_bits(y) for y in yd], K)
        del g
        st = a.get_status()
    assert st[0] == 0, st
