"""The Python example in README.md runs as written (GPU): the ABI calls and
FP8Linear's training forward, backward and decode-sized inference."""

import os

import pytest

from tests._gpu import note, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _readme_example():
    text = open(os.path.join(ROOT, "README.md")).read()
    start = text.index("From Python")
    lines = text[start:].splitlines()[1:]
    block, seen = [], False
    for line in lines:
        if line.startswith("    "):
            block.append(line[4:])
            seen = True
        elif line.strip() == "":
            if seen:
                block.append("")
        elif seen:
            break
    return "\n".join(block)


def test_readme_python_example_runs():
    import torch
    code = _readme_example()
    assert "fp8_gemm_fwd" in code and "FP8Linear" in code
    note("README Python example")
    env = {}
    exec(compile(code, "README.md", "exec"), env)
    torch.cuda.synchronize()
    assert tuple(env["y"].shape) == (4096, 7168)
    assert tuple(env["y_decode"].shape) == (64, 7168)
    assert env["layer"].weight.grad is not None and env["x"].grad is not None
