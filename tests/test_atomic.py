"""The arrival-order atomic variant (AR_PROTO_ATOMIC, two-shot only) on the
GPU.  Its sums follow the order in which the ranks' atomic adds arrive, so it
is held to the order-independent bound against the oracle's exact sum
(tests/atomic_util.py) instead of bit equality; all N output copies must
agree bit for bit, the fp32 debug accumulators must sit inside the same
bound, and the lines must clean themselves between calls (rotating input
sets, both parities, other protocols in between, graph replays)."""
import numpy as np
import pytest

import oracle
import synth
from atomic_util import bf16_violations, f32_violations, ulp_distance
from gpu_util import (ar_context, check_status_clean, empty_out, host_bits, log, rank_tensors,
                      torch_mod)

pytestmark = pytest.mark.gpu

TWO = 2
ATOMIC = 6


def _check_bf16(out_bits, data, what):
    N = data.shape[0]
    s, a = oracle.sum_abs(list(data))
    for r in range(1, N):
        assert np.array_equal(out_bits[r], out_bits[0]), "%s: copy %d differs from copy 0" % (what, r)
    bad = bf16_violations(out_bits[0], s, a, N)
    if bad.size:
        i = bad[0]
        raise AssertionError("%s: %d elements outside the bound, first %d: got %#06x, exact sum %r, "
                             "sum|x| %r" % (what, bad.size, i, int(out_bits[0][i]), s[i], a[i]))
    return float(np.max(ulp_distance(out_bits[0], oracle.allreduce(list(data))[0]), initial=0.0))


def _calls(ar, datas, n, calls, f32=False):
    torch = torch_mod()
    ins = [rank_tensors(d) for d in datas]
    outs = []
    for k in range(calls):
        out = empty_out(datas[0].shape[0], n, f32)
        if f32:
            ar.allreduce_f32_debug(ins[k % len(ins)], out, n, k + 1)
        else:
            ar.allreduce(ins[k % len(ins)], out, n, k + 1)
        outs.append(out)
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("scope", [0, 1], ids=["auto", "device"])
@pytest.mark.parametrize("N,n", [(8, 8192), (8, 4096 + 8), (4, 20008), (2, 968), (16, 3592),
                                 (8, 263600), (3, 8), (1, 248)])
def test_within_bound(N, n, scope):
    log("atomic N=%d n=%d scope=%d" % (N, n, scope))
    datas = [synth.bounded_bits(4000 + 10 * s + N, (N, n)) for s in range(3)]
    with ar_context(N, n + 64, TWO, ATOMIC, scope=scope) as ar:
        outs = _calls(ar, datas, n, 6)
        check_status_clean()
    worst = 0.0
    for k, out in enumerate(outs):
        worst = max(worst, _check_bf16(host_bits(out), datas[k % 3], "call %d" % (k + 1)))
    log("  max distance from the fixed-order result: %.3f ulp" % worst)


def test_f32_accumulators_within_bound():
    N, n = 8, 20008
    log("atomic f32 debug")
    datas = [synth.bounded_bits(4100 + s, (N, n)) for s in range(2)]
    with ar_context(N, n, TWO, ATOMIC) as ar:
        outs = _calls(ar, datas, n, 4, f32=True)
        check_status_clean()
    for k, out in enumerate(outs):
        got = out.cpu().numpy()
        for r in range(1, N):
            assert np.array_equal(got[r].view(np.uint32), got[0].view(np.uint32))
        s, a = oracle.sum_abs(list(datas[k % 2]))
        bad = f32_violations(got[0], s, a, N)
        assert bad.size == 0, (k, bad[:5])


@pytest.mark.parametrize("cid", [2, 3, 4], ids=["c2", "c3", "c4"])
def test_workloads(cid):
    """The decode workloads: a 160-call hipGraph replayed (c2, c3) or 24
    stream calls over 8 rotating sets (c4, 4 MiB per rank)."""
    torch = torch_mod()
    w = synth.WORKLOADS[cid]
    log("atomic workload %d" % cid)
    nsets = 4 if cid != 4 else 8
    datas = [synth.input_set(cid, s) for s in range(nsets)]
    N, n = w.n_ranks, w.n
    with ar_context(N, n, TWO, ATOMIC) as ar:
        ins = [rank_tensors(d) for d in datas]
        if cid == 4:
            outs = [torch.empty((N, n), dtype=torch.int16, device="cuda:0") for _ in range(2)]
            for k in range(24):
                ar.allreduce(ins[k % nsets], outs[k % 2], n, k + 1)
                if k >= 22:
                    torch.cuda.synchronize()
                    _check_bf16(host_bits(outs[k % 2]), datas[k % nsets], "c4 call %d" % (k + 1))
        else:
            calls = 160
            outs = [torch.empty((N, n), dtype=torch.int16, device="cuda:0") for _ in range(nsets)]
            stream = torch.cuda.Stream()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(stream):
                with torch.cuda.graph(g, stream=stream):
                    for k in range(calls):
                        ar.allreduce(ins[k % nsets], outs[k % nsets], n, k + 1, stream=stream)
                    ar.step_end(stream=stream)
            torch.cuda.synchronize()
            for rep in range(3):
                with torch.cuda.stream(stream):
                    for o in outs:
                        o.fill_(-1)
                    g.replay()
                torch.cuda.synchronize()
                for s in range(nsets):
                    _check_bf16(host_bits(outs[s]), datas[s], "replay %d set %d" % (rep, s))
            del g
        check_status_clean()


def test_mixed_with_other_protocols():
    """Atomic calls between calls of every other protocol, both parities:
    the accumulator lines must be zero whenever an atomic call starts."""
    torch = torch_mod()
    log("atomic mixed")
    N, n = 8, 8192
    datas = [synth.bounded_bits(4200 + s, (N, n)) for s in range(4)]
    combos = [(TWO, ATOMIC), (1, 1), (TWO, ATOMIC), (TWO, ATOMIC), (1, 2), (TWO, 4), (TWO, ATOMIC),
              (1, 3), (TWO, 2), (TWO, ATOMIC), (TWO, 5)]
    with ar_context(N, n) as ar:
        ins = [rank_tensors(d) for d in datas]
        out = torch.empty((N, n), dtype=torch.int16, device="cuda:0")
        for k in range(44):
            algo, proto = combos[k % len(combos)]
            ar.set_options(algo, proto)
            ar.allreduce(ins[k % 4], out, n, k + 1)
            torch.cuda.synchronize()
            got = host_bits(out)
            if proto == ATOMIC:
                _check_bf16(got, datas[k % 4], "call %d" % (k + 1))
            else:
                assert np.array_equal(got, oracle.allreduce(list(datas[k % 4]))), k
        check_status_clean()


def test_watchdog_then_reset_cleans_lines():
    """A rank held back from the host (10 ms start delay against a 1 ms
    watchdog) leaves half-summed lines behind; the peers' polls give up and
    record the failure, every kernel exits, and ar_reset zeroes the lines so
    that later calls are within the bound again."""
    import tp_decode_comms_amd as arm
    torch = torch_mod()
    log("atomic watchdog")
    N, n = 8, 8192
    datas = [synth.bounded_bits(4300 + s, (N, n)) for s in range(2)]
    with ar_context(N, n, TWO, ATOMIC, watchdog_us=1000) as ar:
        ins = [rank_tensors(d) for d in datas]
        table = np.zeros((2, N), dtype=np.uint32)
        table[1, 5] = 10_000_000            # flag 2: rank 5 starts 10 ms late
        dtab = torch.from_numpy(table.view(np.int32).copy()).to("cuda:0")   # kept alive
        ar.set_delays(dtab, 2)
        out = torch.empty((N, n), dtype=torch.int16, device="cuda:0")
        for k in range(2):
            ar.allreduce(ins[k], out, n, k + 1)
        torch.cuda.synchronize()
        ar.set_delays(None, 0)
        code, rank, src, flag = ar.get_status()
        assert code == 6 and flag == 2 and rank != 5, (code, rank, src, flag)
        assert arm.lib().ar_get_status((arm.ar.ctypes.c_uint32 * 4)()) == arm.ar.AR_ERR_TIMEOUT
        ar.reset()
        torch.cuda.synchronize()
        for k in range(4):
            ar.allreduce(ins[k % 2], out, n, k + 1)
            torch.cuda.synchronize()
            _check_bf16(host_bits(out), datas[k % 2], "after reset call %d" % (k + 1))
        check_status_clean()


def test_options():
    import tp_decode_comms_amd as arm
    with ar_context(4, 1024) as ar:
        assert arm.lib().ar_set_options(1, ATOMIC) == arm.ar.AR_ERR_INVALID     # one-shot: no
        ar.set_options(0, ATOMIC)                                             # auto -> two-shot
        assert ar.query(2, 1024) == TWO and ar.query(3, 1024) == ATOMIC
