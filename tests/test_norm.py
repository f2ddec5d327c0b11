"""The AllReduce with the residual add and RMS norm fused behind it
(ar_allreduce_add_rmsnorm), and the same norm as a kernel of its own
(ar_add_rmsnorm), against the oracle: h bit for bit, y within the rounding
interval derived in norm_util.py, and fused == unfused bit for bit.

Shapes: the workloads' rows x hidden (1x4096, 1x8192, 32x8192, 8x7168 with
16 ranks) plus the edges of the norm's blocking -- one 256-element block per
row, 65536-element rows (256 blocks, more than one per lane in the fold),
row counts that leave surplus workgroups, and forced launch geometries in
which one workgroup walks many rounds across several rows."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import (ar_context, assert_bits_equal, check_status_clean, dev_bits, host_bits,
                      log, rank_tensors, torch_mod)
from norm_util import expected, y_violations

pytestmark = pytest.mark.gpu

EPS = synth.NORM_EPS
LL, DIRECT = 1, 4
PROTOS = [(LL, "ll"), (DIRECT, "direct")]


def _operands(data, res, gamma):
    return rank_tensors(data), rank_tensors(res), dev_bits(gamma)


def _outs(N, n):
    torch = torch_mod()
    mk = lambda: torch.full((N, n), -1, dtype=torch.int16, device="cuda:0")
    return mk(), mk()


def _check(h_dev, y_dev, h_want, y_want, what):
    assert_bits_equal(host_bits(h_dev), h_want, what + " h")
    y = host_bits(y_dev)
    bad = y_violations(y.ravel(), y_want.ravel())
    if bad.size:
        i = bad[0]
        raise AssertionError("%s y: %d elements outside the interval, first flat index %d: "
                             "got bits %#06x, exact %r" % (what, bad.size, i, int(y.ravel()[i]),
                                                           float(y_want.ravel()[i])))


def _run_case(data, res, gamma, rows, hidden, eps=EPS, calls=2, wgs=0, scope=0, proto=0):
    """`calls` fused calls with the same operands (on the one-shot LL or the
    in-place one-shot as `proto` fixes it, else by size); checks the last
    one, and that the stand-alone kernel on the AllReduce result gives the
    same bits."""
    N, n = data.shape
    a = oracle.allreduce(list(data))[0]
    h_want, y_want = expected(a, res, gamma, eps, rows, hidden, oracle)
    ins, rs, g = _operands(data, res, gamma)
    with ar_context(N, n, proto=proto, wgs=wgs, scope=scope) as ar:
        oh, oy = _outs(N, n)
        for k in range(calls):
            ar.allreduce_add_rmsnorm(ins, rs, g, eps, oh, oy, rows, hidden, k + 1)
        torch_mod().cuda.synchronize()
        check_status_clean()
        _check(oh, oy, h_want, y_want, "fused")
        # unfused: AllReduce, then the stand-alone kernel
        torch = torch_mod()
        out = torch.empty((N, n), dtype=torch.int16, device="cuda:0")
        ar.set_options(0, 0)
        ar.allreduce(ins, out, n, calls + 1)
        uh, uy = _outs(N, n)
        ar.add_rmsnorm(out, rs, g, eps, uh, uy, rows, hidden)
        torch.cuda.synchronize()
        check_status_clean()
        assert_bits_equal(host_bits(uh), host_bits(oh), "unfused vs fused h")
        assert_bits_equal(host_bits(uy), host_bits(oy), "unfused vs fused y")


@pytest.mark.parametrize("proto", [0, LL, DIRECT], ids=["auto", "ll", "direct"])
@pytest.mark.parametrize("cid", [1, 2, 3, 5], ids=["c1", "c2", "c3", "c5"])
def test_workload_shapes(cid, proto):
    w = synth.WORKLOADS[cid]
    log("norm workload %d proto %d" % (cid, proto))
    data = synth.input_set(cid, 0)
    res, gamma = synth.norm_operands(cid, 0)
    _run_case(data, res, gamma, w.rows, w.hidden, proto=proto)


@pytest.mark.parametrize("proto,pname", PROTOS, ids=[p[1] for p in PROTOS])
@pytest.mark.parametrize("scope", [0, 1], ids=["auto", "device"])
def test_replicated_residual_scopes(scope, proto, pname):
    log("norm replicated residual, scope %d, %s" % (scope, pname))
    data = synth.input_set(2, 1)
    res, gamma = synth.norm_operands(2, 1, replicated=True)
    _run_case(data, res, gamma, 1, 8192, scope=scope, proto=proto)


@pytest.mark.parametrize("N,rows,hidden,wgs", [
    (8, 1, 256, 0),        # one block per row; 1 part rounded up to 8: surplus workgroups
    (8, 3, 256, 0),        # rows share no workgroup
    (4, 2, 65536, 0),      # 256 blocks per row: the fold holds 4 per lane
    (8, 4, 8192, 8),       # 8 workgroups per rank: 16 rounds each across 4 rows
    (8, 6, 1280, 3),       # 3 workgroups per rank (not a multiple of 8): ragged rounds
    (2, 5, 512, 1),        # 1 workgroup per rank walks every row
    (16, 2, 7168, 0),      # 16 ranks
    (1, 2, 4096, 0),       # one rank: h = a + res
    # row-wise in-place kernel (8 or more rows of at most 8192 elements)
    (8, 8, 256, 0),        # one block per row: 15 of 16 waves idle
    (4, 9, 8192, 0),       # 32 blocks per row (2 per wave); 9 rows: device scope
    (8, 16, 7168, 0),      # 28 blocks: some waves hold 2, some 1
    (16, 8, 1280, 0),      # 16 ranks, 5 blocks per row
    (1, 8, 4096, 0),       # one rank
    (8, 40, 8192, 0),      # more rows than fit at once: the cross-workgroup kernel
    (2, 8, 16384, 0),      # rows too long for it: the cross-workgroup kernel
], ids=lambda v: str(v))
@pytest.mark.parametrize("proto,pname", PROTOS, ids=[p[1] for p in PROTOS])
def test_blocking_edges(N, rows, hidden, wgs, proto, pname):
    log("norm edge N=%d rows=%d hidden=%d wgs=%d %s" % (N, rows, hidden, wgs, pname))
    rng = np.random.Generator(np.random.PCG64(7100 + N * 131 + rows * 17 + hidden))
    n = rows * hidden
    data = synth.draw(rng, N * n, "normal", 1.0).reshape(N, n)
    res = synth.draw(rng, N * n, "normal", 2.0).reshape(N, n)
    gamma = synth.draw(rng, hidden, "uniform", 1.5)
    _run_case(data, res, gamma, rows, hidden, wgs=wgs, proto=proto)


@pytest.mark.parametrize("proto,pname", PROTOS, ids=[p[1] for p in PROTOS])
def test_cancelled_row_and_zero_eps(proto, pname):
    """A row whose residual cancels the AllReduce result exactly (h = 0, so
    y = 0 with eps > 0), and eps = 0 on rows that are not all zero."""
    log("norm cancelled row")
    N, rows, hidden = 4, 3, 1024
    n = rows * hidden
    data = synth.input_set(1, 2, n=n, n_ranks=N)
    a = oracle.allreduce(list(data))[0]
    rng = np.random.Generator(np.random.PCG64(7300))
    res = synth.draw(rng, N * n, "normal", 2.0).reshape(N, n)
    res[:, hidden:2 * hidden] = a[hidden:2 * hidden] ^ np.uint16(0x8000)   # -a: exact zero
    gamma = synth.draw(rng, hidden, "normal", 1.0)
    _run_case(data, res, gamma, rows, hidden, eps=1e-5, proto=proto)
    res2 = synth.draw(rng, N * n, "normal", 2.0).reshape(N, n)
    _run_case(data, res2, gamma, rows, hidden, eps=0.0, proto=proto)


@pytest.mark.parametrize("proto,pname", PROTOS, ids=[p[1] for p in PROTOS])
def test_graph_decode_step_mixed_with_plain_allreduce(proto, pname):
    """A decode step as a hipGraph: per layer an AllReduce and a fused
    AllReduce + norm (80 layers, 160 calls of one epoch sequence), replayed
    with the step end; every call's outputs checked after every replay."""
    torch = torch_mod()
    log("norm graph %s" % pname)
    w = synth.WORKLOADS[2]
    N, n = w.n_ranks, w.n
    sets = [synth.input_set(2, s) for s in range(4)]
    res, gamma = synth.norm_operands(2, 2)
    want_a = [oracle.allreduce(list(d))[0] for d in sets]
    want = [expected(a, res, gamma, EPS, 1, n, oracle) for a in want_a]
    ins = [rank_tensors(d) for d in sets]
    rs, g = rank_tensors(res), dev_bits(gamma)
    layers = 80
    with ar_context(N, n, proto=proto) as ar:
        outs = [torch.empty((N, n), dtype=torch.int16, device="cuda:0") for _ in range(layers)]
        hs = [torch.empty((N, n), dtype=torch.int16, device="cuda:0") for _ in range(layers)]
        ys = [torch.empty((N, n), dtype=torch.int16, device="cuda:0") for _ in range(layers)]
        stream = torch.cuda.Stream()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(graph, stream=stream):
                for l in range(layers):
                    ar.allreduce(ins[(2 * l) % 4], outs[l], n, 2 * l + 1, stream=stream)
                    ar.allreduce_add_rmsnorm(ins[(2 * l + 1) % 4], rs, g, EPS, hs[l], ys[l], 1, n,
                                             2 * l + 2, stream=stream)
                ar.step_end(stream=stream)
        torch.cuda.synchronize()
        for rep in range(3):
            with torch.cuda.stream(stream):
                for t in outs + hs + ys:
                    t.fill_(-1)
                graph.replay()
            torch.cuda.synchronize()
            for l in range(layers):
                assert_bits_equal(host_bits(outs[l]), np.broadcast_to(want_a[(2 * l) % 4], (N, n)),
                                  "replay %d layer %d allreduce" % (rep, l))
                h_want, y_want = want[(2 * l + 1) % 4]
                _check(hs[l], ys[l], h_want, y_want, "replay %d layer %d" % (rep, l))
        check_status_clean()
        del graph


def test_norm_argument_validation():
    import tp_decode_comms_amd as arm
    torch = torch_mod()
    N, rows, hidden = 4, 2, 1024
    n = rows * hidden
    mk = lambda *s: torch.zeros(s, dtype=torch.int16, device="cuda:0")
    ins = [mk(n) for _ in range(N)]
    rs = [mk(n) for _ in range(N)]
    g = mk(hidden)
    oh, oy = mk(N, n), mk(N, n)
    with ar_context(N, n) as ar:
        call = lambda **kw: ar.allreduce_add_rmsnorm(
            kw.get("ins", ins), kw.get("rs", rs), kw.get("g", g), kw.get("eps", EPS),
            kw.get("oh", oh), kw.get("oy", oy), kw.get("rows", rows), kw.get("hidden", hidden),
            kw.get("epoch", 1), check=False)
        bad = arm.ar.AR_ERR_INVALID
        assert call(hidden=1000, rows=2) == bad            # not a multiple of 256
        assert call(hidden=128, rows=16) == bad            # below one block
        assert call(rows=3) == bad                         # beyond max_elems
        assert call(rows=0) == bad
        assert call(eps=-1.0) == bad
        assert call(eps=float("nan")) == bad
        assert call(oy=oh) == bad                          # outputs overlap
        assert call(rs=[oh[0]] + rs[1:]) == bad           # residual inside out_h
        assert call(g=oy[1, :hidden]) == bad               # gamma inside out_y
        assert call(ins=[oy[2]] + ins[1:]) == bad          # input inside out_y
        assert call(g=g[1:]) == bad                        # misaligned gamma
        assert call(epoch=2) == bad                        # epoch sequence
        ar.set_options(0, 3)
        assert call() == bad                               # sentinel: no fused form
        ar.set_options(2, 4)
        assert call() == bad                               # two-shot: no fused form
        ar.set_options(0, 0)
        assert call() == arm.ar.AR_OK
        torch.cuda.synchronize()
        check_status_clean()
        # the stand-alone kernel checks its operands the same way
        a = mk(N, n)
        assert ar.add_rmsnorm(a, rs, g, EPS, oh, oy, rows, 1000, check=False) == bad
        assert ar.add_rmsnorm(oh, rs, g, EPS, oh, oy, rows, hidden, check=False) == bad
        assert ar.add_rmsnorm(a, rs, g, EPS, oh, oy, rows, hidden, check=False) == arm.ar.AR_OK
        torch.cuda.synchronize()
