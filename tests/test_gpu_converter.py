"""The quantizers' unclamped use of the hardware E4M3 converter.

The kernels pass every quotient q (|q| < 449, see the exhaustive CPU proof)
to v_cvt_pk_fp8_f32 without clamping it to +-448 first. The program
tests/gpu/e4m3_converter_check (built with the library) converts every fp32
value with |v| < 449, both signs, with and without the clamp and counts the
bytes that differ; the count must be zero.
"""

import os
import subprocess

import pytest

from tests._gpu import note, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gpu", "e4m3_converter_check")


def test_converter_needs_no_clamp_below_449():
    if not os.path.exists(EXE):
        raise FileNotFoundError(f"{EXE} is not built; run __graft_entry__.build() first")
    note("e4m3 converter, every |v| < 449 with and without the clamp")
    r = subprocess.run([EXE], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    assert r.returncode == 0, r.stdout
    assert "converter_mismatches=0" in r.stdout, r.stdout
