"""Helpers shared by the GPU tests: torch tensors for the seeded inputs, the
library context, and bit-level comparison against the oracle."""
import contextlib
import sys

import numpy as np

import oracle
import synth


def torch_mod():
    import torch
    return torch


def log(msg):
    print("[gpu-test] " + msg, flush=True)
    sys.stdout.flush()


def dev_bits(arr):
    """uint16 numpy array -> int16 tensor on cuda:0 holding the same bits."""
    torch = torch_mod()
    a = np.ascontiguousarray(arr, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16).copy()).to("cuda:0")


def host_bits(t):
    return t.cpu().numpy().view(np.uint16)


def rank_tensors(data):
    """[N, n] uint16 -> list of N separate device buffers (distinct allocations)."""
    return [dev_bits(data[r]) for r in range(data.shape[0])]


def empty_out(N, n, f32=False):
    torch = torch_mod()
    dt = torch.float32 if f32 else torch.int16
    return torch.empty((N, n), dtype=dt, device="cuda:0")


@contextlib.contextmanager
def ar_context(N, max_elems, algo=0, proto=0, wgs=0, threads=0, watchdog_us=0, scope=0):
    import tp_decode_comms_amd as ar
    ar.init(N, max_elems)
    try:
        ar.set_options(algo, proto)
        ar.set_launch(wgs, threads)
        ar.set_scope(scope)
        ar.set_watchdog(watchdog_us)
        yield ar
    finally:
        torch_mod().cuda.synchronize()
        ar.destroy()


def expect(data):
    """Oracle output [N, n] for inputs [N, n] (uint16)."""
    return oracle.allreduce(list(data))


def assert_bits_equal(got, want, what=""):
    got = np.asarray(got, dtype=np.uint16)
    want = np.asarray(want, dtype=np.uint16)
    assert got.shape == want.shape, (got.shape, want.shape)
    bad = np.nonzero(got != want)
    if bad[0].size:
        idx = tuple(b[0] for b in bad)
        raise AssertionError("%s: %d mismatching elements, first at %s: got %#06x want %#06x"
                             % (what, bad[0].size, idx, int(got[idx]), int(want[idx])))


def check_status_clean():
    import tp_decode_comms_amd as ar
    st = ar.get_status()
    assert st[0] == 0, "watchdog fired: %r" % (st,)


__all__ = ["synth", "oracle"]
