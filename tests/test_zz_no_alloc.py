"""The allocation-free entry point (ar_allreduce_noalloc) through the C ABI:
its outputs equal the existing entry point's (ar_allreduce) bit for bit --
and the oracle's -- on two calls in a row, the second with a smaller input,
without ar_init having been called in between and with no allocation by
the library; also across the window's rounds (16 ranks), from a captured
graph, after a re-arm, and for every refused argument."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from gpu_util import ar_context, assert_bits_equal, host_bits, log, rank_tensors, torch_mod

pytestmark = pytest.mark.gpu


def _noalloc(ins, out, n, stream=None):
    import tp_decode_comms_amd as ar
    arr = (ctypes.c_void_p * len(ins))(*[t.data_ptr() for t in ins])
    s = 0 if stream is None else stream.cuda_stream
    return ar.lib().ar_allreduce_noalloc(arr, out.data_ptr() if out is not None else None, n,
                                         len(ins), s)


def _existing(N, n_max, datas):
    """The existing entry point's outputs for the same inputs."""
    torch = torch_mod()
    outs = []
    with ar_context(N, n_max) as a:
        for k, d in enumerate(datas):
            out = torch.empty(d.shape, dtype=torch.int16, device="cuda:0")
            a.allreduce(rank_tensors(d), out, d.shape[1], k + 1)
            outs.append(out)
        torch.cuda.synchronize()
    return [host_bits(o) for o in outs]


@pytest.mark.parametrize("N,n1,n2", [(8, 8192 * 4 + 8, 8192), (16, 57344, 7168), (4, 4096, 8),
                                     (1, 1024, 16)])
def test_noalloc_matches_existing_entry_point(N, n1, n2):
    """Two calls in a row, the second smaller; 16 ranks walk several rounds
    through their 8 KiB windows."""
    torch = torch_mod()
    log("noalloc N=%d n=%d then %d" % (N, n1, n2))
    datas = [synth.random_bits(7000 + N, (N, n1), finite_only=True, avoid=0xFFFF),
             synth.random_bits(7100 + N, (N, n2), finite_only=True, avoid=0xFFFF)]
    want = _existing(N, n1, datas)
    got = []
    for d in datas:
        out = torch.empty(d.shape, dtype=torch.int16, device="cuda:0")
        out.fill_(-1)
        assert _noalloc(rank_tensors(d), out, d.shape[1]) == 0
        torch.cuda.synchronize()
        got.append(host_bits(out))
    for k in range(2):
        assert_bits_equal(got[k], want[k], "call %d vs the existing entry point" % (k + 1))
        assert_bits_equal(got[k], oracle.allreduce(list(datas[k])), "call %d vs the oracle" % (k + 1))


def test_noalloc_many_calls_graph_and_rearm():
    """200 back-to-back calls over rotating sets (a stale inbox would show),
    a captured graph of 20 calls replayed 3 times, a re-arm (n == 0), and
    the refused arguments."""
    import tp_decode_comms_amd as ar
    torch = torch_mod()
    N, n = 8, 8192
    sets = [synth.input_set(2, s) for s in range(4)]
    ins = [rank_tensors(d) for d in sets]
    want = [torch.from_numpy(oracle.allreduce(list(d)).view(np.int16).copy()).to("cuda:0")
            for d in sets]
    outs = [torch.empty((N, n), dtype=torch.int16, device="cuda:0") for _ in range(4)]
    bad = torch.zeros((), dtype=torch.int64, device="cuda:0")
    for k in range(200):
        assert _noalloc(ins[k % 4], outs[k % 4], n) == 0
        bad += (outs[k % 4] != want[k % 4]).sum()
    torch.cuda.synchronize()
    assert int(bad.item()) == 0
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    gouts = [torch.empty((N, n), dtype=torch.int16, device="cuda:0") for _ in range(20)]
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for k in range(20):
                assert _noalloc(ins[k % 4], gouts[k], n, stream) == 0
    torch.cuda.synchronize()
    for rep in range(3):
        with torch.cuda.stream(stream):
            for o in gouts:
                o.fill_(-1)
            g.replay()
            for k in range(20):
                bad += (gouts[k] != want[k % 4]).sum()
        torch.cuda.synchronize()
    del g
    assert int(bad.item()) == 0
    assert _noalloc(ins[0], None, 0) == 0                     # re-arm
    assert _noalloc(ins[1], outs[1], n) == 0
    torch.cuda.synchronize()
    assert_bits_equal(host_bits(outs[1]), host_bits(want[1]))
    E = ar.ar.AR_ERR_INVALID
    assert _noalloc(ins[0], outs[0], 12) == E                   # n % 8
    assert _noalloc(ins[0], ins[0][0], 8) == E                  # output aliases an input
    assert _noalloc([ins[0][0]] * 17, outs[0], 8) == E          # 17 ranks
    huge = torch.empty(8, dtype=torch.int16, device="cuda:0")
    assert _noalloc(ins[0][:8], huge, (1 << 31) // 16 + 8) == E  # outputs beyond 2^31 bytes
