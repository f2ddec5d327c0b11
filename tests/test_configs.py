"""The five workloads end to end on the GPU, every call checked bit for bit.

  1: 4 ranks x [1x4096], N(0,1), 1000 back-to-back calls, epochs 1..1000,
     4 rotating input sets -- sentinel and LL one-shot.
  2: 8 ranks x [1x8192] (16 KiB), N(0,0.5), LL one-shot, 160 calls per step
     captured in one hipGraph, replayed; also plain stream calls.
  3: 8 ranks x [32x8192] (512 KiB), N(0,1) + 1% x100 outliers, LL128 one-shot
     and two-shot, 160 calls in one hipGraph, replayed.
  4: 8 ranks x [256x8192] (4 MiB), U(-1,1), 8 rotating buffer sets, one-shot
     vs two-shot.
  5: 16 ranks x [8x7168], N(0,1), seeded 0-5 us start delays per (call,
     rank), 10000 calls, sentinel two-shot and one-shot.

Inputs of consecutive calls differ, and so do those of calls k and k-2, so
consuming a stale mailbox or an unarmed inbox cannot go unseen.  Outputs are
compared on the device against the oracle's result uploaded once per input
set; the watchdog must never fire.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import ar_context, check_status_clean, log, torch_mod

pytestmark = pytest.mark.gpu

ONE, TWO = 1, 2
LL, LL128, SENT, DIRECT, BARRIER = 1, 2, 3, 4, 5


def _dev(arr):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16).copy()).to("cuda:0")


class Sets:
    """Rotating input sets of a workload, their expected outputs on the device."""

    def __init__(self, cid, nsets, n=None, n_ranks=None):
        self.data = [synth.input_set(cid, s, n=n, n_ranks=n_ranks) for s in range(nsets)]
        self.N, self.n = self.data[0].shape
        self.ins = [[_dev(d[r]) for r in range(self.N)] for d in self.data]
        self.want = [_dev(oracle.allreduce(list(d))[0]) for d in self.data]   # [n] each

    def __len__(self):
        return len(self.data)


def _count_bad(out, want):
    """Mismatching elements of out [N, n] against want [n] (device scalar)."""
    return (out != want.unsqueeze(0)).sum()


def _stream_calls(ar, sets, calls, nbuf=4, delays=None):
    torch = torch_mod()
    outs = [torch.empty((sets.N, sets.n), dtype=torch.int16, device="cuda:0") for _ in range(nbuf)]
    bad = torch.zeros((), dtype=torch.int64, device="cuda:0")
    for k in range(calls):
        s = k % len(sets)
        out = outs[k % nbuf]
        ar.allreduce(sets.ins[s], out, sets.n, k + 1)
        bad += _count_bad(out, sets.want[s])
    torch.cuda.synchronize()
    return int(bad.item())


@pytest.mark.parametrize("proto", [SENT, LL], ids=["sentinel", "ll"])
def test_config1_1000_calls(proto):
    log("config 1, proto %d" % proto)
    sets = Sets(1, 4)
    with ar_context(4, sets.n, ONE, proto) as ar:
        bad = _stream_calls(ar, sets, 1000)
        check_status_clean()
    assert bad == 0


def _graph_steps(ar, sets, replays, calls=160):
    """Captures `calls` calls plus the step end in one graph, replays it and
    checks every call's output after every replay."""
    torch = torch_mod()
    outs = [torch.empty((sets.N, sets.n), dtype=torch.int16, device="cuda:0") for _ in range(calls)]
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for k in range(calls):
                ar.allreduce(sets.ins[k % len(sets)], outs[k], sets.n, k + 1, stream=stream)
            ar.step_end(stream=stream)
    torch.cuda.synchronize()
    bad = torch.zeros((), dtype=torch.int64, device="cuda:0")
    # poison, replay and compare all on one stream, so that no comparison of
    # replay r overlaps the writes of replay r + 1
    with torch.cuda.stream(stream):
        for r in range(replays):
            for o in outs:              # a call that wrote nothing is seen
                o.fill_(-1)
            g.replay()
            for k in range(calls):
                bad += _count_bad(outs[k], sets.want[k % len(sets)])
    torch.cuda.synchronize()
    del g
    return int(bad.item())


def test_config2_graph_160_calls():
    log("config 2, graph")
    sets = Sets(2, 4)
    with ar_context(8, sets.n, ONE, LL) as ar:
        bad = _graph_steps(ar, sets, replays=20)
        check_status_clean()
    assert bad == 0


def test_config2_stream_160_calls_per_step():
    log("config 2, stream")
    torch = torch_mod()
    sets = Sets(2, 4)
    with ar_context(8, sets.n, ONE, LL) as ar:
        outs = [torch.empty((8, sets.n), dtype=torch.int16, device="cuda:0") for _ in range(4)]
        bad = torch.zeros((), dtype=torch.int64, device="cuda:0")
        for step in range(5):
            for k in range(160):
                s = k % 4
                ar.allreduce(sets.ins[s], outs[k % 4], sets.n, k + 1)
                bad += _count_bad(outs[k % 4], sets.want[s])
            ar.step_end()
        torch.cuda.synchronize()
        check_status_clean()
    assert int(bad.item()) == 0


@pytest.mark.parametrize("algo", [ONE, TWO], ids=["oneshot", "twoshot"])
def test_config3_ll128_graph(algo):
    log("config 3, LL128, algo %d" % algo)
    sets = Sets(3, 4)
    with ar_context(8, sets.n, algo, LL128) as ar:
        bad = _graph_steps(ar, sets, replays=3)
        check_status_clean()
    assert bad == 0


@pytest.mark.parametrize("algo,proto", [(TWO, DIRECT), (ONE, DIRECT), (TWO, LL128), (TWO, SENT),
                                        (TWO, BARRIER)],
                         ids=["twoshot-direct", "oneshot-direct", "twoshot-ll128",
                              "twoshot-sentinel", "twoshot-barrier"])
def test_config4_rotating_sets(algo, proto):
    log("config 4, algo %d proto %d" % (algo, proto))
    sets = Sets(4, 8)
    with ar_context(8, sets.n, algo, proto) as ar:
        bad = _stream_calls(ar, sets, 40, nbuf=2)
        check_status_clean()
    assert bad == 0


@pytest.mark.parametrize("cid,algo,proto,calls", [
    (4, TWO, DIRECT, 400), (4, ONE, DIRECT, 200), (4, TWO, LL128, 200),
    (3, TWO, LL128, 1000), (3, ONE, LL128, 1000), (2, ONE, LL, 2000), (2, ONE, DIRECT, 2000)],
    ids=["4mib-twoshot-direct", "4mib-oneshot-direct", "4mib-twoshot-ll128",
         "512kib-twoshot-ll128", "512kib-oneshot-ll128", "16kib-ll", "16kib-oneshot-direct"])
def test_start_delays_other_kinds(cid, algo, proto, calls):
    """Config 5's seeded 0-5 us start delays per (call, rank) on the other
    kinds and workloads: ranks that arrive late (the in-place kernels'
    arrival flags, their first poll taken before the delay) or publish late
    (LL units, LL128 lines) still give every call bit-exactly, with no
    watchdog record."""
    log("delays: workload %d, algo %d, proto %d, %d calls" % (cid, algo, proto, calls))
    torch = torch_mod()
    sets = Sets(cid, 8 if cid == 4 else 4)
    delays = torch.from_numpy(synth.delays_ns(5, calls, n_ranks=sets.N).view(np.int32).copy()
                              ).to("cuda:0")
    with ar_context(sets.N, sets.n, algo, proto) as ar:
        ar.set_delays(delays, calls)
        bad = _stream_calls(ar, sets, calls, nbuf=len(sets))
        ar.set_delays(None, 0)
        check_status_clean()
    assert bad == 0


@pytest.mark.parametrize("algo", [TWO, ONE], ids=["twoshot", "oneshot"])
def test_config5_delays_10000_calls(algo):
    log("config 5, sentinel, algo %d" % algo)
    torch = torch_mod()
    sets = Sets(5, 8)
    calls = 10000
    delays = torch.from_numpy(synth.delays_ns(5, calls).view(np.int32).copy()).to("cuda:0")
    with ar_context(16, sets.n, algo, SENT) as ar:
        ar.set_delays(delays, calls)
        bad = _stream_calls(ar, sets, calls, nbuf=8)
        ar.set_delays(None, 0)
        check_status_clean()
    assert bad == 0


def test_watchdog_records_and_reset_recovers():
    """A rank held back (from the host: a 10 ms start delay in one call)
    beyond a 1 ms watchdog makes its peers' polls give up and record the
    failure; every kernel still exits.  ar_reset re-arms everything and later
    calls are exact again."""
    import tp_decode_comms_amd as arm
    torch = torch_mod()
    log("watchdog")
    sets = Sets(2, 4)
    with ar_context(8, sets.n, ONE, LL, watchdog_us=1000) as ar:
        table = np.zeros((4, 8), dtype=np.uint32)
        table[2, 3] = 10_000_000            # call with flag 3: rank 3 starts 10 ms late
        dtab = torch.from_numpy(table.view(np.int32).copy()).to("cuda:0")
        ar.set_delays(dtab, 4)
        out = torch.empty((8, sets.n), dtype=torch.int16, device="cuda:0")
        for k in range(4):
            ar.allreduce(sets.ins[k % 4], out, sets.n, k + 1)
        torch.cuda.synchronize()
        ar.set_delays(None, 0)
        code, rank, src, flag = ar.get_status()
        assert code == 6 and flag == 3 and src == 3 and rank != 3, (code, rank, src, flag)
        assert arm.lib().ar_get_status((arm.ar.ctypes.c_uint32 * 4)()) == arm.ar.AR_ERR_TIMEOUT
        ar.reset()
        torch.cuda.synchronize()
        assert ar.get_status()[0] == 0
        bad = _stream_calls(ar, sets, 40)
        check_status_clean()
    assert bad == 0


def test_protocol_switch_between_calls():
    """Calls may change algorithm and protocol between calls of one step."""
    log("protocol switch")
    torch = torch_mod()
    sets = Sets(2, 4)
    combos = [(ONE, LL), (ONE, SENT), (TWO, DIRECT), (ONE, LL128), (TWO, LL128), (TWO, SENT),
              (ONE, DIRECT), (ONE, BARRIER), (TWO, BARRIER)]
    with ar_context(8, sets.n) as ar:
        out = torch.empty((8, sets.n), dtype=torch.int16, device="cuda:0")
        bad = torch.zeros((), dtype=torch.int64, device="cuda:0")
        for k in range(90):
            algo, proto = combos[k % len(combos)]
            ar.set_options(algo, proto)
            s = k % 4
            ar.allreduce(sets.ins[s], out, sets.n, k + 1)
            bad += _count_bad(out, sets.want[s])
        torch.cuda.synchronize()
        check_status_clean()
    assert int(bad.item()) == 0


# ---- fixed-size staging: the workloads with windows far smaller than their
# messages, so every call walks many rounds through the two buffers and each
# buffer is overwritten within a call (the double buffer's permit at work)

def _rounds(ar, n):
    return ar.query(12, n)


def test_config2_graph_small_window_rounds():
    """16 KiB LL messages through a 4 KiB window: 8 rounds per call, 160
    calls per graph, every call of every replay checked."""
    log("config 2, LL, 4 KiB window")
    sets = Sets(2, 4)
    with ar_context(8, sets.n, ONE, LL) as ar:
        ar.set_staging(4096)
        assert ar.query(15, sets.n) == 4096 and _rounds(ar, sets.n) == 8
        bad = _graph_steps(ar, sets, replays=5)
        check_status_clean()
    assert bad == 0


@pytest.mark.parametrize("algo", [ONE, TWO], ids=["oneshot", "twoshot"])
def test_config3_ll128_small_window(algo):
    """512 KiB LL128 messages through a 16 KiB window (the one-shot's lines
    are 546 KiB per rank, the two-shot's 68 KiB per slice)."""
    log("config 3, LL128, 16 KiB window, algo %d" % algo)
    sets = Sets(3, 4)
    with ar_context(8, sets.n, algo, LL128) as ar:
        ar.set_staging(16384)
        assert _rounds(ar, sets.n) >= 3
        bad = _graph_steps(ar, sets, replays=2)
        check_status_clean()
    assert bad == 0


@pytest.mark.parametrize("algo,proto", [(TWO, LL128), (TWO, SENT), (ONE, LL128)],
                         ids=["twoshot-ll128", "twoshot-sentinel", "oneshot-ll128"])
def test_config4_small_window(algo, proto):
    """4 MiB messages through a 64 KiB window (64 times smaller than the
    message), 8 rotating buffer sets."""
    log("config 4, 64 KiB window, algo %d proto %d" % (algo, proto))
    sets = Sets(4, 8)
    with ar_context(8, sets.n, algo, proto) as ar:
        ar.set_staging(65536)
        assert ar.query(15, sets.n) == 65536 and _rounds(ar, sets.n) >= 8
        bad = _stream_calls(ar, sets, 24, nbuf=2)
        check_status_clean()
    assert bad == 0


@pytest.mark.parametrize("algo", [TWO, ONE], ids=["twoshot", "oneshot"])
def test_config5_delays_small_window_10000_calls(algo):
    """16 ranks with seeded 0-5 us start delays, 10,000 calls, sentinel
    inboxes of 4 KiB per pair and buffer (the one-shot's 112 KiB messages take
    28 rounds per call, the two-shot's 7 KiB slices 2)."""
    log("config 5, sentinel, 4 KiB window, algo %d" % algo)
    torch = torch_mod()
    sets = Sets(5, 8)
    calls = 10000
    delays = torch.from_numpy(synth.delays_ns(5, calls).view(np.int32).copy()).to("cuda:0")
    with ar_context(16, sets.n, algo, SENT) as ar:
        ar.set_staging(4096)
        assert _rounds(ar, sets.n) >= 2
        ar.set_delays(delays, calls)
        bad = _stream_calls(ar, sets, calls, nbuf=8)
        ar.set_delays(None, 0)
        check_status_clean()
    assert bad == 0


@pytest.mark.parametrize("algo,proto,n", [(ONE, LL, 8200), (ONE, LL, 8192), (ONE, LL128, 65536),
                                           (ONE, LL128, 131072), (TWO, LL128, 262144)])
def test_default_window_takes_one_round(algo, proto, n):
    """With the default windows a message that fits them runs in one round
    even when its part count is rounded up to a multiple of 8 (the window
    holds whole 8-part rounds)."""
    log("default window, algo %d proto %d n %d" % (algo, proto, n))
    sets = Sets(2, 2, n=n, n_ranks=8)
    with ar_context(8, n, algo, proto) as ar:
        assert _rounds(ar, n) == 1, (ar.query(15, n), ar.query(4, n))
        bad = _stream_calls(ar, sets, 6)
        check_status_clean()
    assert bad == 0


@pytest.mark.parametrize("N,n", [(8, 524288 + 8), (4, 1048576 + 24)])
def test_oneshot_ll128_four_groups_per_batch(N, n):
    """One-shot LL128 above 512 KiB per rank takes batches of four line
    groups (two above 8 ranks), several rounds through the default window."""
    log("one-shot LL128, N=%d n=%d" % (N, n))
    sets = Sets(2, 2, n=n, n_ranks=N)
    with ar_context(N, n, ONE, LL128) as ar:
        assert _rounds(ar, n) >= 1
        bad = _stream_calls(ar, sets, 6)
        check_status_clean()
    assert bad == 0


def test_staging_window_validation():
    import tp_decode_comms_amd as arm
    with ar_context(8, 1 << 20) as ar:
        lib = arm.lib()
        assert lib.ar_set_staging(1024) == arm.ar.AR_ERR_INVALID       # below 4 KiB
        assert lib.ar_set_staging(5000) == arm.ar.AR_ERR_INVALID       # not a multiple of 1 KiB
        assert lib.ar_set_staging(8192) == 0
        ar.set_options(ONE, LL)
        assert ar.query(15, 8192) == 8192
        ar.set_staging(0)
        assert ar.query(15, 8192) == 1 << 20                         # LL: 1 MiB per rank, buffer
        ar.set_options(TWO, DIRECT)
        assert ar.query(15, 8192) == 0                                # no staging


@pytest.mark.parametrize("algo,proto,window", [(ONE, LL, 0), (ONE, LL, 4096), (TWO, LL128, 0),
                                               (ONE, LL128, 16384), (TWO, DIRECT, 0),
                                               (TWO, SENT, 4096)],
                         ids=["oneshot-ll", "oneshot-ll-rounds", "twoshot-ll128",
                              "oneshot-ll128-rounds", "twoshot-direct", "twoshot-sentinel-rounds"])
def test_sequence_restart_across_steps(algo, proto, window):
    """The step-end kernel restarts the round sequence (clearing every flag
    word) once it passes 0xF0000000.  Started just below that with the test
    hook, steps of 160 calls run across the restart; every call of every
    step must stay bit-exact, the device sequence must be small afterwards
    and the call count must have kept counting."""
    import tp_decode_comms_amd as arm
    torch = torch_mod()
    log("sequence restart %d/%d window %d" % (algo, proto, window))
    sets = Sets(2, 4)
    with ar_context(8, sets.n, algo, proto) as ar:
        ar.set_staging(window)
        rounds = ar.query(12, sets.n)
        per_step = 160 * rounds
        start = 0xF0000000 - per_step - per_step // 2      # the second step crosses the limit
        ar.set_sequence(start)
        assert arm.lib().ar_set_sequence(0xF0000001, None) == arm.ar.AR_ERR_INVALID
        outs = [torch.empty((8, sets.n), dtype=torch.int16, device="cuda:0") for _ in range(4)]
        bad = torch.zeros((), dtype=torch.int64, device="cuda:0")
        seqs = []
        for step in range(4):
            for k in range(160):
                s = k % 4
                ar.allreduce(sets.ins[s], outs[k % 4], sets.n, k + 1)
                bad += _count_bad(outs[k % 4], sets.want[s])
            ar.step_end()
            seqs.append(ar.query(14, 0))
        assert ar.query(14, 1) == 4 * 160                     # calls keep counting
        check_status_clean()
    assert int(bad.item()) == 0
    assert seqs[0] == start + per_step
    assert seqs[1] == 0 and seqs[2] == per_step and seqs[3] == 2 * per_step, seqs
