"""The README's Python example runs as written on the GPU."""

import os
import re

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_python_example_runs():
    text = open(os.path.join(ROOT, "README.md")).read()
    blocks = re.findall(r"```python\n(.*?)```", text, re.S)
    assert len(blocks) == 1
    env = {}
    exec(compile(blocks[0], "README.md", "exec"), env)
    torch.cuda.synchronize()
    out, cache = env["out"], env["cache"]
    assert out.shape == (4, 16, 128) and out.dtype == torch.float32
    assert torch.isfinite(out).all()
    assert cache.seq_lens[0].tolist() == [101] * 4  # 100 appended, one stored by the step
