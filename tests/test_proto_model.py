"""The staged protocols' double buffering, modelled with host threads
(tests/proto_model/proto_model.cpp) and run under ThreadSanitizer on the CPU.

Each thread plays one (rank, part) of the GPU kernels, or one wave of a
workgroup that splits its peers over waves and meets at a barrier each
round.  Messages several times larger than the staging window are walked in
rounds through two alternating buffers, every round with its own flag; a
round may be published only once the previous round has been received from
every peer (the double-buffer permit of the "Every Microsecond Counts"
write-up, page "微秒必争…", section "四大核心机制", item 3).  The clean
protocols must give exact sums with no race reported; each planted mistake
-- one buffer, one flag per call, publishing before the permit, re-arming
after the next round's pushes, waves not meeting -- must be caught (wrong
sum, a poll that never completes, or a data race)."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "proto_model", "proto_model.cpp")


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("proto") / "proto_model")
    subprocess.run(["g++", "-std=c++20", "-O1", "-g", "-fsanitize=thread", "-pthread", SRC,
                    "-o", exe], check=True, capture_output=True, text=True)
    return exe


def _run(exe, proto, ranks, parts, units, elems, calls, seed, waves, mutant="none"):
    env = dict(os.environ, TSAN_OPTIONS="exitcode=66")
    r = subprocess.run([exe, proto, str(ranks), str(parts), str(units), str(elems), str(calls),
                        str(seed), str(waves), mutant], capture_output=True, text=True,
                       timeout=300, env=env)
    return r.returncode, r.stdout + r.stderr


@pytest.mark.parametrize("proto", ["ll", "ll128", "sentinel"])
@pytest.mark.parametrize("waves", [1, 2])
def test_double_buffer_rounds_are_exact_and_race_free(model, proto, waves):
    # 8 ranks would only slow TSan down; 4 ranks x 2 parts x 8 units: a window
    # of 16 elements per rank and buffer against messages of 2000 (125 rounds)
    for seed in (1, 2):
        rc, out = _run(model, proto, 4, 2, 8, 2000, 4, seed, waves)
        assert rc == 0, out[-3000:]
        assert "ThreadSanitizer" not in out, out[-3000:]
    # ragged: the last round is partial, a single part, 3 ranks
    rc, out = _run(model, proto, 3, 1, 16, 1000 + 5, 3, 9, 1)
    assert rc == 0, out[-3000:]


MUTANTS = [("ll", "single_buffer", 1), ("ll", "call_flag", 1), ("ll", "eager_publish", 1),
           ("ll", "no_barrier", 2),
           ("ll128", "single_buffer", 1), ("ll128", "call_flag", 1),
           ("ll128", "eager_publish", 1), ("ll128", "no_barrier", 2),
           ("sentinel", "single_buffer", 1), ("sentinel", "eager_publish", 1),
           ("sentinel", "late_rearm", 1), ("sentinel", "no_barrier", 2)]


@pytest.mark.parametrize("proto,mutant,waves", MUTANTS,
                         ids=["%s-%s" % (p, m) for p, m, _ in MUTANTS])
def test_planted_protocol_mistakes_are_caught(model, proto, mutant, waves):
    # a race needs an unlucky interleaving: up to four seeded runs of 250
    # rounds, and at least one must fail (none has needed more than one)
    codes = []
    for seed in (1, 2, 3, 4):
        rc, out = _run(model, proto, 4, 2, 8, 2000, 4, seed, waves, mutant)
        codes.append(rc)
        if rc != 0:
            assert rc in (2, 3, 66), out[-2000:]
            return
    pytest.fail("%s/%s was never caught: exit codes %r" % (proto, mutant, codes))
