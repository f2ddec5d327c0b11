"""bench.py end to end on the GPU with a short, odd warm-up: it must finish
with exit status 0 and print one JSON line that carries the headline, the
4 MiB roofline and the parity result (a bench leg that failed would be
listed under failed_legs)."""
import json
import os
import subprocess
import sys

import pytest

from gpu_util import log

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_runs_to_its_json_line():
    log("bench.py --steps 3 --warmup 5 --bw-calls 3 --no-cpu")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3",
                        "--warmup", "5", "--bw-calls", "3", "--no-cpu"],
                       capture_output=True, text=True, timeout=900, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-4000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    line = json.loads(lines[0])
    assert line["failed_legs"] == [], line["failed_legs"]
    assert line["parity_ok"] is True
    assert line["value"] is not None and line["value"] > 0
    assert line["config"]["workload"]
    assert line["roofline"]["bound"] == "hbm" and 0 < line["roofline"]["frac"] < 1
    fl = line["latency_floor"]
    # the floor is a graph node plus one flag hop inside an XCD's L2; the
    # device-scope hop between XCDs is the longer one
    assert fl["floor_us"] == pytest.approx(fl["graph_node_us"] + fl["flag_hop_us"], abs=1e-3)
    assert 0 < fl["flag_hop_us"] < fl["flag_hop_cross_xcd_us"]
    assert 0 < fl["frac"] < 1.5
    hops = line["results"]["floor"]["flag_hop"]
    assert hops["xcd_local"]["placement_ok"] and hops["cross_xcd"]["placement_ok"]
