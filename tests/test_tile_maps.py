"""CPU check that the kernels' workgroup -> tile maps are bijections.

Builds tests/cpu/tile_map_bijection.cpp host-only with hipcc; the program
includes the kernels' own csrc/tile_map.h (host and device functions), so the
maps checked here are the code the GEMM and 128x1 quantizer kernels run. Cases:

* every tile grid up to 40 x 40, in both GEMM orders (per-XCD bands and the
  chip-wide 16 x 16 supertiles);
* the tile grid of every GEMM of every configured workload (forward, DGrad and
  WGrad of each linear), in all four tile shapes and both orders, so whichever
  configuration a launch picks is covered;
* the grouped WGrad launch of each multi-linear workload (the benchmark's
  dominant launch at 32768 tokens), with 256-aligned ranges and the order
  each problem's contraction length selects, plus the 8-aligned small-tile
  layout and the shapes of the grouped GPU tests;
* the 128x1 / dual quantizer grids of every activation and gradient tensor.
"""

import os
import shutil
import subprocess

import pytest

from fp8_block_scaled_quantize_amd import inputs

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "cpu", "tile_map_bijection.cpp")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

TILES = {"large": (256, 256), "medium": (256, 128), "small": (128, 64), "tiny": (64, 64)}
SUPERTILE_MIN_KB = 64


def _cdiv(a, b):
    return -(-a // b)


def _gemm_dims(role, M, N, K):
    """(I, J, contraction) of the kernel for one role: out[j][i], P has I rows, Q has J rows."""
    Np, Kp = _cdiv(N, 128) * 128, _cdiv(K, 128) * 128
    if role == "fwd":
        return Np, M, Kp
    if role == "dgrad":
        return Kp, M, Np
    return K, N, _cdiv(M, 128) * 128


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("needs hipcc")
    exe = str(tmp_path_factory.mktemp("tilemap") / "tile_map_bijection")
    subprocess.run([HIPCC, "-x", "hip", "--offload-host-only", "-O2", "-std=c++17", SRC, "-o", exe], check=True)
    return exe


def _run(exe, lines):
    r = subprocess.run([exe], input="\n".join(lines) + "\n", stdout=subprocess.PIPE, text=True, timeout=600)
    out = r.stdout.splitlines()
    assert r.returncode == 0, "\n".join(l for l in out if l.startswith("FAIL"))[:2000]
    assert len(out) == len(lines) and all(l.startswith("ok ") for l in out), out[:5]
    return out


def test_every_small_grid(checker):
    out = _run(checker, ["all 40"])
    assert out == [f"ok all {2 * sum(i * j for i in range(1, 41) for j in range(1, 41))}"]


def test_workload_gemm_grids(checker):
    lines = set()
    for wl in inputs.WORKLOADS.values():
        for lin in wl["linears"]:
            for role in wl["passes"]:
                I, J, _ = _gemm_dims(role, lin["M"], lin["N"], lin["K"])
                for bi, bj in TILES.values():
                    ti, tj = _cdiv(I, bi), _cdiv(J, bj)
                    lines.add(f"plain {ti} {tj}")
                    lines.add(f"super {ti} {tj}")
    _run(checker, sorted(lines))


def _group_line(align, problems, tile):
    bi, bj = tile
    parts = []
    for role, M, N, K in problems:
        I, J, red = _gemm_dims(role, M, N, K)
        sup = int(tile[0] * tile[1] >= 256 * 128 and red // 128 >= SUPERTILE_MIN_KB)
        parts.append(f"{_cdiv(I, bi)} {_cdiv(J, bj)} {sup}")
    return f"group {align} {len(problems)} " + " ".join(parts)


def test_grouped_layouts(checker):
    lines = []
    for wl in inputs.WORKLOADS.values():
        if "wgrad" not in wl["passes"] or len(wl["linears"]) < 2:
            continue
        probs = [("wgrad", l["M"], l["N"], l["K"]) for l in wl["linears"]]
        lines.append(_group_line(256, probs, TILES["large"]))
        lines.append(_group_line(8, probs, TILES["small"]))
        for role in ("fwd", "dgrad"):
            if role in wl["passes"]:
                p = [(role, l["M"], l["N"], l["K"]) for l in wl["linears"]]
                lines.append(_group_line(256, p, TILES["large"]))
                lines.append(_group_line(8, p, TILES["small"]))
    # the grouped GPU tests' shapes
    for shapes in ([(256, 512, 384), (128, 256, 640), (384, 128, 128), (256, 384, 256)],
                   [(256, 4096, 4096), (512, 4224, 2048), (256, 2048, 4096)],
                   [(8192, 4096, 4224), (8192, 1152, 8192), (8192, 5120, 896)]):
        for role in ("fwd", "dgrad", "wgrad"):
            p = [(role, M, N, K) for (M, N, K) in shapes]
            lines.append(_group_line(256, p, TILES["large"]))
            lines.append(_group_line(8, p, TILES["small"]))
    _run(checker, lines)


def test_quantizer_grids(checker):
    lines = set()
    for wl in inputs.WORKLOADS.values():
        for lin in wl["linears"]:
            M = lin["M"]
            for C in (lin["K"], lin["N"]):
                lines.add(f"quant {_cdiv(M, 128)} {min(_cdiv(C, 128), 65535)}")
    for nx in (1, 2, 31, 32, 33, 255, 256, 257):
        for ny in (1, 3, 8, 9):
            lines.add(f"quant {nx} {ny}")
    _run(checker, sorted(lines))


def test_checker_detects_a_broken_map(checker, tmp_path):
    """The checker itself: a copy of the header with one id remapped must fail."""
    hdr = os.path.join(os.path.dirname(HERE), "fp8_block_scaled_quantize_amd", "csrc", "tile_map.h")
    src = open(hdr).read()
    broken = src.replace("ti = first_i + in_group % gsize;", "ti = first_i + in_group % gsize; if (bid == 3) ti = (ti + 1) % tiles_i;")
    assert broken != src
    d = tmp_path / "csrc"
    d.mkdir()
    (d / "tile_map.h").write_text(broken)
    prog = open(SRC).read().replace('"../../fp8_block_scaled_quantize_amd/csrc/tile_map.h"', f'"{d}/tile_map.h"')
    (tmp_path / "p.cpp").write_text(prog)
    exe = str(tmp_path / "p")
    subprocess.run([HIPCC, "-x", "hip", "--offload-host-only", "-O2", "-std=c++17", str(tmp_path / "p.cpp"), "-o", exe],
                   check=True)
    r = subprocess.run([exe], input="plain 5 7\n", stdout=subprocess.PIPE, text=True, timeout=60)
    assert r.returncode == 1 and r.stdout.startswith("FAIL")
