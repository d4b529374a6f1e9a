"""Build libfp8bsq.so (the C-ABI library) in-tree with hipcc for gfx950.

    python -m fp8_block_scaled_quantize_amd.build

Compiles every csrc/*.hip to an object file, then links one shared library
next to this file; also builds the stand-alone GPU check programs under
tests/gpu (each tests/gpu/<name>.hip -> tests/gpu/<name>), which GPU tests run,
and the ceilings micro-benchmark bench_ceilings.hip -> bench_ceilings at the
repository root, which bench.py runs.
Flags:
  --offload-arch=gfx950                  MI355X only
  -O3 -std=c++17 -fPIC
  -fhip-fp32-correctly-rounded-divide-sqrt   IEEE fp32 division for the scales
  -Xclang -target-feature -Xclang -packed-fp32-ops   no packed fp32 VALU ops
No fast-math and no denormal flushing: the quantizers rely on IEEE fp32
division and fma with gradual underflow.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libfp8bsq.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
BUILD_DIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-Wno-unused-command-line-argument",
]


# Stand-alone GPU check programs that tests run (not part of the library).
CHECKS_DIR = os.path.join(ROOT, "tests", "gpu")


CEILINGS_SRC = os.path.join(ROOT, "bench_ceilings.hip")
CEILINGS_EXE = os.path.join(ROOT, "bench_ceilings")


def check_programs():
    """(source, executable) pairs of the stand-alone HIP programs: the GPU
    checks under tests/gpu and the ceilings micro-benchmark."""
    progs = []
    if os.path.isdir(CHECKS_DIR):
        progs = [(os.path.join(CHECKS_DIR, f), os.path.join(CHECKS_DIR, f[:-4]))
                 for f in sorted(os.listdir(CHECKS_DIR)) if f.endswith(".hip")]
    if os.path.exists(CEILINGS_SRC):
        progs.append((CEILINGS_SRC, CEILINGS_EXE))
    return progs


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def build(verbose=False):
    """Compile and link the library; returns the path of the .so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in sources():
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        objs.append(obj)
        cmds.append([HIPCC, *COMMON_FLAGS, "-c", src, "-o", obj])
    for src, exe in check_programs():
        cmds.append([HIPCC, *COMMON_FLAGS, src, "-o", exe])
    with ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
