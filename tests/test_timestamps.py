"""The measurement twins (kernels built with the timestamp hooks) against the
oracle: every staged and in-place kind, with a start-record table and with a
phase-record table, bit-exact outputs and sane records (a start in every
workgroup's slot; with phases start <= sync <= data <= end where marked)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import ar_context, assert_bits_equal, check_status_clean, host_bits, log, torch_mod

pytestmark = pytest.mark.gpu

ONE, TWO = 1, 2
LL, LL128, SENT, DIRECT = 1, 2, 3, 4
KINDS = [(ONE, LL), (ONE, LL128), (TWO, LL128), (ONE, SENT), (TWO, SENT), (ONE, DIRECT),
         (TWO, DIRECT)]


@pytest.mark.parametrize("phases", [False, True], ids=["starts", "phases"])
@pytest.mark.parametrize("algo,proto", KINDS, ids=["%d-%d" % k for k in KINDS])
def test_twin_matches_oracle_and_records(algo, proto, phases):
    torch = torch_mod()
    import tp_decode_comms_amd as ar
    N, n, calls = 8, 8192 * 4 + 8, 6
    log("timestamps algo %d proto %d phases %d" % (algo, proto, phases))
    data = [synth.input_set(2, s, n=n, n_ranks=N) for s in range(2)]
    want = [oracle.allreduce(list(d))[0] for d in data]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16).copy()).to("cuda:0")
    ins = [[dev(d[r]) for r in range(N)] for d in data]
    with ar_context(N, n, algo, proto) as a:
        grid, threads = a.query(4, n), a.query(5, n)
        records = grid * (threads // 64 if phases else 1)
        ts = torch.zeros((calls, records, 4), dtype=torch.int64, device="cuda:0")
        a.set_timestamps(ts, calls, records, phases)
        try:
            for k in range(calls):
                out = torch.empty((N, n), dtype=torch.int16, device="cuda:0")
                a.allreduce(ins[k % 2], out, n, k + 1)
                torch.cuda.synchronize()
                got = host_bits(out)
                for r in range(N):
                    assert_bits_equal(got[r], want[k % 2], "call %d rank %d" % (k, r))
        finally:
            a.set_timestamps(None, 0, 0)
        check_status_clean()
        tab = ts.cpu().numpy().view(np.uint64)
    starts = tab[:, :, 0]
    assert (starts != 0).all(), "a workgroup (or wave) wrote no start record"
    if phases:
        t = tab.astype(np.float64)
        end = t[:, :, 3]
        assert (end >= t[:, :, 0]).all()
        for f in (1, 2):
            m = tab[:, :, f] != 0
            assert (t[:, :, f][m] >= t[:, :, 0][m]).all() and (t[:, :, f][m] <= end[m]).all()
    else:
        assert (tab[:, :, 1:] == 0).all(), "start records wrote beyond their field"
