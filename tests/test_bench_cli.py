"""bench.py's command-line contract, without a GPU: it measures one GPU and
refuses other GPU counts (and multi-rank launches) with exit status 2 and
a message, before touching the device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                          capture_output=True, text=True, timeout=120, env=e, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "1 GPU" in r.stderr or "one MI355X" in r.stderr


def test_multi_rank_launch_is_refused():
    r = _run([], env={"WORLD_SIZE": "2"})
    assert r.returncode == 2
    assert "single-process" in r.stderr


# ---- bench.py's host-side bookkeeping (no GPU): the epoch tracker, the leg
# guard and the per-call statistics of the timestamp table

def _bench():
    import importlib
    sys.path.insert(0, ROOT)
    return importlib.import_module("bench")


class _FakeLib:
    """Keeps the library's epoch contract (include/ar.h): epoch = previous + 1,
    at most 65535, and 1 again after a step end."""

    def __init__(self):
        self.last, self.steps, self.calls = 0, 0, 0

    def allreduce(self, epoch):
        assert epoch == self.last + 1 and 1 <= epoch <= 65535, (epoch, self.last)
        self.last = epoch
        self.calls += 1

    def step_end(self, stream=None):
        self.last = 0
        self.steps += 1


def test_epoch_tracker_odd_warmups_and_long_runs():
    b = _bench()
    for warmup in (0, 1, 5, 7, 160, 161):
        for calls in (1, 3, 200, 401):
            lib = _FakeLib()
            ep = b.Epochs(lib)
            for _ in range(warmup + 2 * calls):
                lib.allreduce(ep.next())
            ep.close()
            assert lib.last == 0 and lib.calls == warmup + 2 * calls
            # a graph captured afterwards starts at epoch 1
            lib.allreduce(1)
            # steps close every 160 calls, as a decode step would
            assert lib.steps == -(-(warmup + 2 * calls) // b.CALLS_PER_STEP)


def test_leg_guard_records_failures_and_stops_after_device_errors():
    b = _bench()
    legs = b.Legs()
    assert legs.run("ok", lambda: {"mismatches": 0, "status": [0, 0, 0, 0]}) is not None

    def boom():
        raise ValueError("host-side problem")

    assert legs.run("bad", boom) is None
    assert "host-side problem" in legs.results["bad"]["error"] and not legs.stopped
    assert legs.run("after", lambda: {"mismatches": 0}) == {"mismatches": 0}

    def device():
        raise RuntimeError("HIP error: an illegal memory access was encountered")

    legs.run("dev", device)
    assert legs.stopped
    legs.run("later", lambda: {"mismatches": 0})
    assert "skipped" in legs.results["later"]
    assert b.parity_ok({"a": {"mismatches": 0, "status": [0] * 4}})
    assert not b.parity_ok(legs.results)
    assert not b.parity_ok({"a": {"mismatches": 0, "status": [6, 1, 2, 3]}})


def test_timestamp_stats_per_call_figures():
    """Two replays of three calls, two waves each, with known times (ticks of
    10 ns): intervals, spans, gaps and phases come out as constructed."""
    import numpy as np
    b = _bench()
    calls, replays = 3, 2
    recs = []
    t = 1000
    for r in range(replays):
        for k in range(calls):
            start = t
            # wave 0 starts at `start`, wave 1 20 ticks later; sync at +50/+60,
            # data at +100/+130, end at +150/+200 (call span 200 ticks = 2 us)
            recs.append([[start, start + 50, start + 100, start + 150],
                         [start + 20, start + 60, start + 130, start + 200]])
            t = start + 200 + 40                 # 40-tick launch gap
        t += 5000                                # replay boundary
    tab = np.zeros((calls * (replays + 1), 2, 4), dtype=np.uint64)
    tab[calls:] = np.array(recs, dtype=np.uint64)   # the untimed replay's slots stay empty
    intervals, spans, gaps, phases = b.timestamp_stats(tab, calls)
    assert intervals.size == replays * (calls - 1)
    assert np.allclose(intervals, 2.4) and np.allclose(gaps, 0.4)
    assert np.allclose(spans, 2.0)
    assert np.allclose(phases["last_sync_us"], 0.6)
    assert np.allclose(phases["last_data_us"], 1.3)
    assert np.allclose(phases["end_us"], 2.0)
    # per wave: waits 50/40, data 50/70, tails 50/70 ticks; medians of two
    assert np.allclose(phases["median_wave_sync_wait_us"], 0.45)
    assert np.allclose(phases["median_wave_data_us"], 0.6)
    assert np.allclose(phases["p90_wave_data_us"], 0.68)
    assert np.allclose(phases["median_wave_tail_us"], 0.6)
    assert np.allclose(phases["median_wave_end_us"], 1.75)
    lat = {"instrumented": {"agreement": 0.03, "interval_us": {"p50": 2.4, "p99": 2.5}},
           "event_us_per_call": {"p50": 2.5, "p99": 2.6}}
    assert b.headline_latency(lat)[:2] == (2.4, 2.5)
    lat["instrumented"]["agreement"] = 0.08
    assert b.headline_latency(lat)[:2] == (2.5, 2.6)


def test_start_stats_periods():
    """Starts only (no phases): periods are start(k+1) - start(k) within a
    replay, and the dispatch spread is first to last workgroup start."""
    import numpy as np
    b = _bench()
    calls, replays = 4, 2
    tab = np.zeros((calls * (replays + 1), 3, 4), dtype=np.uint64)
    t = 5000
    for r in range(replays):
        for k in range(calls):
            slot = calls + r * calls + k
            tab[slot, :, 0] = [t + 10, t, t + 30]      # workgroups start 0.1-0.3 us apart
            t += 250                                   # 2.5 us per call
        t += 10000
    intervals, dispatch = b.start_stats(tab, calls)
    assert intervals.size == replays * (calls - 1)
    assert np.allclose(intervals, 2.5) and np.allclose(dispatch, 0.3)
