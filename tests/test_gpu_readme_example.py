"""The Python example in README.md runs as written and returns what it says."""
import os
import re

import pytest
import torch

from gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu

README = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "README.md")


def test_readme_python_example_runs():
    need_gpu()
    text = open(README).read()
    blocks = re.findall(r"```python\n(.*?)```", text, flags=re.S)
    assert blocks, "README.md has no python example"
    say("README example,", len(blocks[0].splitlines()), "lines")
    ns = {}
    exec(compile(blocks[0], "README.md example", "exec"), ns)
    torch.cuda.synchronize()
    B, Hq, Hkv, d, T, N = (ns[k] for k in ("B", "Hq", "Hkv", "d", "T", "N"))
    assert ns["out"].shape == (B, Hq, d) and ns["out"].dtype == torch.float32
    assert ns["o"].shape == (B, Hq, N, d) and ns["lse"].shape == (B, Hq, N)
    assert ns["dq"].shape == (B, Hq, N, d) and ns["dk"].shape == (B, Hkv, N, d) and ns["dv"].shape == (B, Hkv, N, d)
    for name in ("out", "o", "lse", "dq", "dk", "dv"):
        assert torch.isfinite(ns[name]).all(), name
