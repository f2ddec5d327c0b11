"""The flag hop between two workgroups (include/ar_ping.h) on the GPU: both
placements land where they are meant to, every wait ends within its budget,
and the one-way hop is positive and far below a microsecond-scale bound,
also over consecutive calls whose flag values continue from the last."""
import pytest

from gpu_util import log, torch_mod

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cross", [0, 1])
def test_flag_ping_placement_and_hop(cross):
    import tp_decode_comms_amd as ar
    torch = torch_mod()
    log("flag ping cross_xcd=%d" % cross)
    out = torch.full((5,), -1, dtype=torch.int64, device="cuda:0")
    hops = []
    for rounds in (1, 100, 1000, 7):
        out.fill_(-1)
        ar.flag_ping(rounds, cross, out)
        torch.cuda.synchronize()
        ticks, st_a, xa, xb, st_b = out.tolist()
        assert st_a == 0 and st_b == 0
        assert 0 <= xa < 8 and 0 <= xb < 8
        assert (xa != xb) if cross else (xa == xb)
        assert ticks > 0
        hops.append(ticks * 0.01 / (2 * rounds))
    # one way: a store seen by a poll, through an L2 or between two; 1000
    # round trips well inside 10 us each
    assert 0.0 < hops[2] < 10.0
