"""CPU proof that the quantizers' division-free quotient equals IEEE fp32 division.

Builds tests/cpu/quotient_exhaustive.c with gcc and runs it: it enumerates
every pair of bf16 values (x, amax) with |x| <= amax, both signs of x, and
checks that the kernels' reciprocal-and-correction sequence gives the same
E4M3 byte (and the same float32 whenever the quotient is at least 2^-11) as
fl32(x / fl32(amax / 448)), and that no quotient reaches 449 in magnitude
(the kernels pass quotients to the hardware converter unclamped).
"""

import os
import shutil
import subprocess
import tempfile

import pytest

SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "cpu", "quotient_exhaustive.c")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_quotient_sequence_is_exact_division():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "qx")
        subprocess.run(["gcc", "-O2", "-mfma", "-ffp-contract=off", "-fopenmp", SRC, "-o", exe, "-lm"], check=True)
        r = subprocess.run([exe], stdout=subprocess.PIPE, text=True, timeout=600)
    assert r.returncode == 0, r.stdout
    assert "byte_mismatch=0 f32_mismatch=0" in r.stdout
    assert "pairs=1065402238" in r.stdout
    maxq = float(r.stdout.split("max_abs_q=")[1].split()[0])
    assert 448.0 <= maxq < 449.0, maxq
