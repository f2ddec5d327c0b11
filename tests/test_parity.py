"""GPU parity: the HIP path against the CPU oracle, bit for bit.

Every case calls the C ABI through the thin binding and compares all N
output copies with the oracle on the same seeded inputs.  Sizes span several
workgroup tiles and LL128 line groups and end in ragged tails.  The bf16
bar is 0 ULP; the fp32 debug path is held to 1e-6 relative (and is exact in
practice, since both sides perform the same binary32 additions).
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import (ar_context, assert_bits_equal, check_status_clean, dev_bits, empty_out,
                      expect, host_bits, log, rank_tensors, torch_mod)

pytestmark = pytest.mark.gpu

ONE, TWO = 1, 2
LL, LL128, SENT, DIRECT, BARRIER = 1, 2, 3, 4, 5
VARIANTS = [
    ("oneshot-ll", ONE, LL),
    ("oneshot-sentinel", ONE, SENT),
    ("oneshot-ll128", ONE, LL128),
    ("oneshot-direct", ONE, DIRECT),
    ("twoshot-ll128", TWO, LL128),
    ("twoshot-sentinel", TWO, SENT),
    ("twoshot-direct", TWO, DIRECT),
    ("oneshot-barrier", ONE, BARRIER),     # the barrier-ful baseline
    ("twoshot-barrier", TWO, BARRIER),
]


def _run_calls(ar, datas, n, calls, out_list=None, f32=False):
    """Runs `calls` back-to-back calls cycling through input sets `datas`."""
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


SCOPES = [("auto", 0), ("device", 1), ("cross-xcd", 2)]
WINDOWS = [("window-all", 0), ("window-4k", 4096)]


@pytest.mark.parametrize("win_name,window", WINDOWS, ids=[w[0] for w in WINDOWS])
@pytest.mark.parametrize("scope_name,scope", SCOPES, ids=[s[0] for s in SCOPES])
@pytest.mark.parametrize("name,algo,proto", VARIANTS, ids=[v[0] for v in VARIANTS])
@pytest.mark.parametrize("N,n", [(8, 8192), (8, 4096 + 8), (4, 20008), (2, 968), (16, 3592),
                                 (8, 262144 + 480 * 3 + 16)])
def test_variant_matches_oracle(name, algo, proto, N, n, scope_name, scope, win_name, window):
    """Every variant in every placement and coherence scope: XCD-local (auto,
    where the placement allows it), device scope, and ranks spread over the
    XCDs (rank r on XCD r mod 8, device scope); the staged protocols with their
    whole staging window and with a 4 KiB window, which walks the larger
    messages in many rounds through the two buffers (the window does not
    apply to the protocols without staging)."""
    log("variant %s N=%d n=%d scope=%s %s" % (name, N, n, scope_name, win_name))
    datas = [synth.random_bits(1000 + 10 * s + N, (N, n), finite_only=True, avoid=0xFFFF)
             for s in range(3)]
    with ar_context(N, n + 64, algo, proto, scope=scope) as ar:
        ar.set_staging(window)
        outs = _run_calls(ar, datas, n, 6)
        check_status_clean()
    for k, out in enumerate(outs):
        assert_bits_equal(host_bits(out), expect(datas[k % 3]), "%s call %d" % (name, k + 1))


@pytest.mark.parametrize("name,algo,proto", [("oneshot-direct", ONE, DIRECT), ("oneshot-barrier", ONE, BARRIER)],
                         ids=["oneshot-direct", "oneshot-barrier"])
@pytest.mark.parametrize("N,n", [(8, 32768), (8, 32768 + 8), (3, 32768), (3, 32768 + 8), (16, 8), (5, 4096 + 8)])
def test_oneshot_lane_unit_boundary(name, algo, proto, N, n):
    """The in-place one-shot gives each lane 4 elements up to 64 KiB per rank
    and 8 above: both sides of the switch, and the smallest call, bit-exact."""
    log("lane units %s N=%d n=%d" % (name, N, n))
    datas = [synth.random_bits(5000 + 10 * s + N, (N, n), finite_only=True, avoid=0xFFFF)
             for s in range(3)]
    with ar_context(N, n, algo, proto) as ar:
        outs = _run_calls(ar, datas, n, 6)
        check_status_clean()
    for k, out in enumerate(outs):
        assert_bits_equal(host_bits(out), expect(datas[k % 3]), "%s call %d" % (name, k + 1))


@pytest.mark.parametrize("name,algo,proto", VARIANTS, ids=[v[0] for v in VARIANTS])
def test_single_rank_identity(name, algo, proto):
    n = 2048 + 8
    data = synth.random_bits(7, (1, n), avoid=0xFFFF)
    log("identity %s" % name)
    with ar_context(1, n, algo, proto) as ar:
        outs = _run_calls(ar, [data, data], n, 2)
        check_status_clean()
    for out in outs:
        assert_bits_equal(host_bits(out), data, name)


@pytest.mark.parametrize("name,algo,proto", VARIANTS, ids=[v[0] for v in VARIANTS])
def test_f32_debug_accumulators(name, algo, proto):
    N, n = 8, 8192 + 480
    datas = [synth.random_bits(77 + s, (N, n), avoid=0xFFFF) for s in range(2)]
    log("f32 debug %s" % name)
    with ar_context(N, n, algo, proto) as ar:
        outs = _run_calls(ar, datas, n, 4, f32=True)
        check_status_clean()
    for k, out in enumerate(outs):
        want = oracle.allreduce_f32(list(datas[k % 2]))
        got = out.cpu().numpy()
        for r in range(N):
            finite = np.isfinite(want)
            assert np.array_equal(np.isfinite(got[r]), finite)
            rel = np.abs(got[r][finite].astype(np.float64) - want[finite]) / \
                np.maximum(np.abs(want[finite].astype(np.float64)), 1e-30)
            assert rel.max(initial=0.0) <= 1e-6
            # the same binary32 additions in the same order: bitwise equal
            assert np.array_equal(got[r].view(np.uint32)[finite], want.view(np.uint32)[finite])


def _golden_cases():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.txt")
    cases = []
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if line:
            lhs, rhs = line.split("->")
            toks = lhs.split()
            cases.append(([int(t, 16) for t in toks[1:]], int(rhs, 16)))
    return cases


@pytest.mark.parametrize("name,algo,proto", VARIANTS, ids=[v[0] for v in VARIANTS])
def test_golden_cases_on_gpu(name, algo, proto):
    """Hand-worked cases (rounding ties, signed zeros, subnormals, overflow,
    order witness), each replicated across a vector of 1000 elements."""
    log("golden %s" % name)
    n = 1000
    by_n = {}
    for ins, want in _golden_cases():
        by_n.setdefault(len(ins), []).append((ins, want))
    for N, cases in sorted(by_n.items()):
        data = np.zeros((N, n), dtype=np.uint16)
        wants = np.zeros(n, dtype=np.uint16)
        for i in range(n):
            ins, want = cases[i % len(cases)]
            data[:, i] = ins
            wants[i] = want
        with ar_context(N, n, algo, proto) as ar:
            outs = _run_calls(ar, [data, data], n, 2)
            check_status_clean()
        for out in outs:
            got = host_bits(out)
            for r in range(N):
                assert_bits_equal(got[r], wants, "%s N=%d" % (name, N))


def test_all_variants_agree_bitwise():
    """One-shot and two-shot with every protocol produce identical bits."""
    N, n = 8, 65536 + 4096 + 8
    data = synth.input_set(3, 0, n=n)
    results = []
    for name, algo, proto in VARIANTS:
        log("agree %s" % name)
        with ar_context(N, n, algo, proto) as ar:
            outs = _run_calls(ar, [data, data], n, 2)
        results.append(host_bits(outs[1]))
    want = expect(data)
    for (name, _, _), got in zip(VARIANTS, results):
        assert_bits_equal(got, want, name)


def test_rejects_bad_calls():
    import tp_decode_comms_amd as ar
    torch = torch_mod()
    N, n = 4, 1024
    data = synth.random_bits(3, (N, n))
    ins = rank_tensors(data)
    out = empty_out(N, n)
    with ar_context(N, n) as a:
        assert a.allreduce(ins, out, n, 2, check=False) == ar.ar.AR_ERR_INVALID   # epoch must be 1
        assert a.allreduce(ins, out, 12, 1, check=False) == ar.ar.AR_ERR_INVALID  # n % 8
        assert a.allreduce(ins, out, n + 8, 1, check=False) == ar.ar.AR_ERR_INVALID
        assert a.allreduce(ins, ins[0], n // 8, 1, check=False) == ar.ar.AR_ERR_INVALID  # aliasing
        assert a.allreduce(ins, out, n, 1) == 0
        assert a.allreduce(ins, out, n, 1, check=False) == ar.ar.AR_ERR_INVALID   # repeat
        assert a.allreduce(ins, out, n, 2) == 0
        assert a.allreduce(ins, out, n, 3) == 0
        assert a.query(7) == 3 and a.query(13) >= 3
        assert a.lib().ar_step_end(None) == 0           # any number of calls closes a step
        assert a.query(7) == 0 and a.query(13) == 0
        assert a.allreduce(ins, out, n, 1) == 0
        torch.cuda.synchronize()
    assert_bits_equal(host_bits(out), expect(data))


def test_cross_xcd_placement_is_selected():
    """AR_SCOPE_CROSS_XCD launches every call on the rank-per-XCD grid with
    device-scope accesses; the default keeps part p of every rank on XCD p."""
    import tp_decode_comms_amd as ar
    with ar_context(8, 1 << 21) as a:
        for n in (8192, 32 * 8192, 256 * 8192):
            assert a.query(16, n) == 0 and a.query(8, n) == 1, n
        a.set_scope(ar.AR_SCOPE_CROSS_XCD)
        for n in (8192, 32 * 8192, 256 * 8192):
            assert a.query(16, n) == 1 and a.query(8, n) == 0, n
        assert ar.lib().ar_set_scope(3) == ar.ar.AR_ERR_INVALID


def test_xcd_local_scope_is_used():
    """On MI355X the round-robin placement verifies, and the small-message
    and bandwidth shapes launch with the XCD-local scope; AR_SCOPE_DEVICE
    turns it off."""
    import tp_decode_comms_amd as ar
    with ar_context(8, 1 << 21) as a:
        assert a.query(9, 0) == 1
        for n in (8192, 32 * 8192, 256 * 8192):
            assert a.query(8, n) == 1, n
        a.set_scope(ar.AR_SCOPE_DEVICE)
        assert a.query(8, 8192) == 0


def test_device_clock_and_units():
    """ar_init accepted the device only because its constant clock runs at
    the 100 MHz the kernels' timers count; the compute-unit count it plans
    grids with is the device's."""
    torch = torch_mod()
    with ar_context(2, 1024) as a:
        assert a.query(10, 0) == 100000
        assert a.query(11, 0) == torch.cuda.get_device_properties(0).multi_processor_count


def test_auto_selection():
    """AUTO follows the crossovers measured on MI355X (include/ar.h)."""
    with ar_context(8, 1 << 20) as a:
        for kib, algo, proto in ((4, ONE, DIRECT), (16, ONE, DIRECT), (32, ONE, DIRECT), (512, ONE, DIRECT),
                                 (1024 - 16, ONE, DIRECT), (1024, TWO, DIRECT)):
            n = kib * 512
            assert (a.query(2, n), a.query(3, n)) == (algo, proto), kib
        for p, last_one in ((SENT, 64), (LL128, 128), (DIRECT, 1024 - 16)):
            a.set_options(0, p)
            assert a.query(2, last_one * 512) == ONE, (p, last_one)
            nxt = 1024 if p == DIRECT else 2 * last_one
            assert a.query(2, nxt * 512) == TWO, (p, nxt)
