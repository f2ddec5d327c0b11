"""Largest contexts the library accepts, checked on sampled outputs.

Staging is bounded (fixed windows walked in rounds), so the binding limit is
the output: all N copies in binary32 (the debug path) must span at most 2^31
bytes, the offset past every descriptor at which the kernels park skipped
accesses.  For 8 ranks max_elems = 2^26 (128 MiB of bf16 per rank) is the
largest accepted and 2^26 + 8 is refused; for 16 ranks the limit is 2^25.
At that size the kernels' output offsets run up to 2^30 bytes, and the
one-shot LL walks about a thousand rounds through its 1 MiB windows.  Outputs are compared with the
oracle at sampled element indices (the fold is element-wise, so the oracle on
the gathered columns is exact): the first and last 4096 elements, the
elements around every slice boundary of the two-shot split, and 65536 random
indices, on every rank's copy.  Inputs are random bf16 patterns with
exponents in [-30, 30)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_status_clean, log, torch_mod

pytestmark = pytest.mark.gpu


def _sample_idx(n, N, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    L = ((n + N - 1) // N + 7) // 8 * 8                 # two-shot slice length
    edges = [np.arange(0, 4096), np.arange(n - 4096, n)]
    for q in range(1, N):
        b = q * L
        if b < n:
            edges.append(np.arange(max(b - 64, 0), min(b + 64, n)))
    edges.append(rng.integers(0, n, size=65536))
    return np.unique(np.concatenate(edges))


@pytest.mark.parametrize("N,n,algo,proto", [(8, 1 << 26, 0, 0), (8, 1 << 26, 1, 1),
                                            (16, 1 << 25, 0, 0)],
                         ids=["n8-auto", "n8-oneshot-ll", "n16-auto"])
def test_largest_context(N, n, algo, proto):
    import tp_decode_comms_amd as ar
    torch = torch_mod()
    log("max size N=%d n=%d algo=%d proto=%d" % (N, n, algo, proto))
    # the next size up (a multiple of 8) is refused by ar_init
    assert ar.lib().ar_init(N, n + 8) == ar.ar.AR_ERR_INVALID
    # exponents within +-30: no overflow, so no NaN whose sign bit would
    # depend on the hardware that created it (special values are covered at
    # smaller sizes)
    x = np.stack([synth.bounded_bits(9100 + 37 * N + r, n) for r in range(N)])
    ins = [torch.from_numpy(x[r].view(np.int16)).to("cuda:0") for r in range(N)]
    out = torch.empty((N, n), dtype=torch.int16, device="cuda:0")
    idx = _sample_idx(n, N, 9200 + N)
    idx_dev = torch.from_numpy(idx.astype(np.int64)).to("cuda:0")
    want = oracle.allreduce(list(x[:, idx]))            # [N, k]
    ar.init(N, n)
    try:
        ar.set_options(algo, proto)
        for epoch in (1, 2):
            out.fill_(-1)
            ar.allreduce(ins, out, n, epoch)
            torch.cuda.synchronize()
            got = out.index_select(1, idx_dev).cpu().numpy().view(np.uint16)
            bad = np.nonzero(got != want)
            assert bad[0].size == 0, ("epoch %d: %d mismatches, first rank %d element %d"
                                      % (epoch, bad[0].size, bad[0][0], idx[bad[1][0]]))
        check_status_clean()
    finally:
        torch.cuda.synchronize()
        ar.destroy()
