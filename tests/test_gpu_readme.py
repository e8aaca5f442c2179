"""The Python usage example of the README runs as written (full QKV sizes:
quantise a bf16 weight on the GPU, package and load it, run the layer, and
the AWQ weights through the GEMV), and its outputs have the stated shapes."""
import os
import re

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_example_runs(tmp_path, monkeypatch):
    text = open(os.path.join(ROOT, "README.md")).read()
    blocks = re.findall(r"```python\n(.*?)```", text, re.S)
    assert len(blocks) == 1
    monkeypatch.chdir(tmp_path)
    ns = {}
    exec(compile(blocks[0], "README.md", "exec"), ns)
    torch.cuda.synchronize()
    y, y_awq = ns["y"], ns["y_awq"]
    assert y.dtype == torch.bfloat16 and tuple(y.shape) == (4096, 9216)
    assert y_awq.dtype == torch.bfloat16 and tuple(y_awq.shape) == (4, 9216)
    assert torch.isfinite(y.float()).all() and torch.isfinite(y_awq.float()).all()
    assert (tmp_path / "qkv.safetensors").exists()
