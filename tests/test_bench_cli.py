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
