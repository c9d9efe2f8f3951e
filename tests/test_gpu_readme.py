"""The README's Python example runs as written and gives the shapes and
dtypes its comments state."""
import os
import re

import pytest
import torch

from gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_example_runs():
    need_gpu()
    say("case README example")
    text = open(os.path.join(ROOT, "README.md")).read()
    blocks = re.findall(r"```python\n(.*?)```", text, re.S)
    assert len(blocks) == 1
    env = {}
    exec(compile(blocks[0], "README.md", "exec"), env)
    torch.cuda.synchronize()
    B, Hq, Hkv, N, d = env["B"], env["Hq"], env["Hkv"], env["N"], env["d"]
    assert env["o"].shape == (B, Hq, N, d) and env["o"].dtype == torch.bfloat16
    assert env["S"].shape == (B, Hkv, d, d) and env["S"].dtype == torch.float32
    assert env["ot"].shape == (B, Hq, d) and env["ot"].dtype == torch.float32
    assert env["dq"].shape == env["q"].shape and env["dk"].shape == env["k"].shape
    assert env["on"].shape == env["nc"].shape == env["o"].shape
    for name in ("o", "o2", "S2", "ot", "dq", "dk", "dv", "on", "nc"):
        assert bool(torch.isfinite(env[name].float()).all()), name
