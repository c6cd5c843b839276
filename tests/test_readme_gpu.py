"""The Python examples in README.md run as written on the GPU (seeded),
so the documented calls stay in step with the binding."""
import os
import re

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_python_examples_run(twn):
    import torch
    text = open(os.path.join(ROOT, "README.md"), encoding="utf-8").read()
    blocks = re.findall(r"```python\n(.*?)```", text, flags=re.S)
    assert len(blocks) >= 2
    print(f"[README] {len(blocks)} python blocks", flush=True)
    torch.manual_seed(0)
    env = {}
    for code in blocks:
        exec(compile(code, "README.md", "exec"), env)
    torch.cuda.synchronize()
    for name in ("out", "res_new", "red"):
        t = env[name]
        assert t.is_cuda and bool(torch.isfinite(t.float()).all()), name
    assert env["gathers"][0][3 * 1024:4 * 1024].float().abs().sum().item() > 0
