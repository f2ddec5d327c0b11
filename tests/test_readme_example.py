"""The usage example in README.md runs as written on the GPU (a graph of 160
calls and the step end, a clean status), and its result is the oracle's."""
import os
import re

import numpy as np
import pytest

from gpu_util import log

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_python_example_runs():
    import oracle
    text = open(os.path.join(ROOT, "README.md"), encoding="utf-8").read()
    blocks = re.findall(r"```python\n(.*?)```", text, re.S)
    assert len(blocks) == 1
    code = blocks[0].replace("ar.destroy()", "")      # keep the outputs to compare
    log("README example")
    env = {}
    exec(compile(code, "README.md", "exec"), env)
    torch, ar = env["torch"], env["ar"]
    try:
        ins = [t.view(torch.int16).cpu().numpy().view(np.uint16) for t in env["ins"]]
        got = env["out"].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, oracle.allreduce(ins))
    finally:
        ar.destroy()
