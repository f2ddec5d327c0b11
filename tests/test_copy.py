"""The bandwidth reference copy (include/ar_copy.h) on the GPU: the exact
bytes at sizes from one vector to a whole grid round and ragged last rounds,
nothing written past the end, and the back-to-back graph form the bench
times."""
import numpy as np
import pytest

from gpu_util import log, torch_mod

pytestmark = pytest.mark.gpu

ROUND = 512 * 256 * 2 * 16          # bytes one round of the largest grid moves


@pytest.mark.parametrize("nbytes", [16, 48, 4096 + 16, ROUND, 3 * ROUND + 16 * 77, 32 << 20])
def test_copy_exact_and_bounded(nbytes):
    import tp_decode_comms_amd as ar
    torch = torch_mod()
    log("copy %d bytes" % nbytes)
    guard = 4096
    src_h = np.random.default_rng(nbytes).integers(0, 256, size=nbytes, dtype=np.uint8)
    src = torch.from_numpy(src_h).to("cuda:0")
    dst = torch.full((nbytes + guard,), 0xA5, dtype=torch.uint8, device="cuda:0")
    ar.copy(src, dst, nbytes)
    torch.cuda.synchronize()
    out = dst.cpu().numpy()
    assert np.array_equal(out[:nbytes], src_h)
    assert (out[nbytes:] == 0xA5).all()


def test_copy_graph_replays():
    """Copies captured in one graph and replayed several times, with eager
    work between the replays: every replay leaves every pair equal."""
    import tp_decode_comms_amd as ar
    torch = torch_mod()
    log("copy graph")
    pairs, nbytes = 3, 1 << 20
    srcs = [torch.randint(-32768, 32767, (nbytes // 2,), dtype=torch.int16, device="cuda:0")
            for _ in range(pairs)]
    dsts = [torch.zeros_like(x) for x in srcs]
    gs = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(gs):
        with torch.cuda.graph(g, stream=gs):
            for k in range(2 * pairs):
                ar.copy(srcs[k % pairs], dsts[k % pairs], nbytes, stream=gs)
    for rep in range(3):
        for d in dsts:
            d.zero_()
        for s in srcs:
            s.add_(1)
        torch.cuda.synchronize()
        with torch.cuda.stream(gs):
            g.replay()
        torch.cuda.synchronize()
        for k in range(pairs):
            assert torch.equal(srcs[k], dsts[k]), "replay %d pair %d" % (rep, k)
