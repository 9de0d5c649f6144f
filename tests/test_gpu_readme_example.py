"""The Python usage example of README.md, run as written: tree attention on
two chain-shaped trees through the C ABI, checked inside the example against
causal attention in float32 PyTorch on the CPU."""

import re
from pathlib import Path

import pytest
import torch

README = Path(__file__).resolve().parents[1] / "README.md"


def _python_blocks(text: str):
    return re.findall(r"```python\n(.*?)```", text, re.S)


def test_readme_has_one_python_example():
    assert len(_python_blocks(README.read_text())) == 1


@pytest.mark.gpu
def test_readme_example_runs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.manual_seed(0)
    code = _python_blocks(README.read_text())[0]
    print("[gpu] README example", flush=True)
    exec(compile(code, str(README), "exec"), {"__name__": "readme_example"})
    torch.cuda.synchronize()
