"""Seeded synthetic inputs for the FP8 linear-layer flow.

This module only draws numbers: it holds none of the quantization or GEMM
arithmetic. Both the HIP-path tests/bench and the CPU oracle take their inputs
from here, so that both sides see the same bf16 bytes.

Recipe (the pages print no shapes or values; the workloads below stand in for
the linear layers of the models the Jet-RL pages evaluate -- Llama3.1-8B,
Qwen2.5-7B and a 32B model -- at their real shapes):

* every tensor is drawn as float32 from numpy's PCG64, ``standard_normal``
  times the standard deviation, then rounded once to bf16 (nearest, ties to
  even);
* "outlier channels": round(0.01 * C) distinct columns of the last dimension,
  chosen without replacement from the same generator, are multiplied by 20 in
  float32 before the bf16 rounding;
* per-tensor generators are spawned from ``SeedSequence(seed)`` in a fixed
  tensor order, so each tensor is reproducible on its own.
"""

import numpy as np

GROUP = 128


def f32_to_bf16_bits(x):
    """Round float32 to bf16 (nearest, ties to even); finite inputs only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_normal(rng, shape, std, outlier_frac=0.0, outlier_gain=20.0):
    """bf16 bit patterns (uint16) of N(0, std^2) values, with optional outlier columns."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    x *= np.float32(std)
    if outlier_frac > 0:
        C = shape[-1]
        n_out = int(round(outlier_frac * C))
        cols = rng.choice(C, size=n_out, replace=False)
        x[..., cols] *= np.float32(outlier_gain)
    return f32_to_bf16_bits(x)


def tensor_streams(seed, n):
    """n independent generators spawned from SeedSequence(seed)."""
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


# ---------------------------------------------------------------------------
# Workloads: linear layers named by model and shape.
#   A linear maps K input features to N outputs; X is [M, K], W is [N, K],
#   dY is [M, N]. Standard deviations: X 1.0, W 0.02, dY 1e-3 unless noted.
# ---------------------------------------------------------------------------

def _lin(name, M, N, K, x_outliers=True, dy_std=1e-3, dy_outliers=False):
    return {"name": name, "M": M, "N": N, "K": K, "x_std": 1.0, "w_std": 0.02,
            "x_outliers": x_outliers, "dy_std": dy_std, "dy_outliers": dy_outliers}


WORKLOADS = {
    # Tiny forward-only case, seed 0.
    "tiny_fwd_128x256x256": {
        "passes": ("fwd",),
        "linears": [_lin("tiny", 128, 256, 256, x_outliers=False)],
    },
    # Rollout decode step through Llama-3.1-8B's fused gate+up projection.
    "llama31_8b_decode_gate_up_m64": {
        "passes": ("fwd",),
        "linears": [_lin("gate_up", 64, 28672, 4096)],
    },
    # Training / prefill forward of Llama-3.1-8B's MLP, 2 x 8192 tokens.
    "llama31_8b_prefill_mlp_m16384": {
        "passes": ("fwd",),
        "linears": [_lin("up", 16384, 14336, 4096), _lin("down", 16384, 4096, 14336)],
    },
    # Backward of Qwen2.5-7B's MLP (hidden 3584, intermediate 18944).
    "qwen25_7b_mlp_backward_m16384": {
        "passes": ("dgrad", "wgrad"),
        "linears": [_lin("up", 16384, 18944, 3584), _lin("down", 16384, 3584, 18944)],
    },
}

# Qwen2.5-32B-shaped linears (hidden 5120, intermediate 27648, GQA qkv
# 5120 + 2 * 1024 = 7168 outputs, o-proj 5120 x 5120), full fwd + DGrad +
# WGrad, at three token counts. Gradients here also carry 1% outlier columns.
for _M in (256, 4096, 32768):
    WORKLOADS[f"qwen25_32b_linears_m{_M}"] = {
        "passes": ("fwd", "dgrad", "wgrad"),
        "linears": [
            _lin("qkv", _M, 7168, 5120, dy_std=1.0, dy_outliers=True),
            _lin("o", _M, 5120, 5120, dy_std=1.0, dy_outliers=True),
            _lin("up", _M, 27648, 5120, dy_std=1.0, dy_outliers=True),
            _lin("down", _M, 5120, 27648, dy_std=1.0, dy_outliers=True),
        ],
    }


def linear_tensors(lin, seed=0, which=("x", "w", "dy"), rows=None):
    """Generate bf16 bit patterns for one linear: dict with x [M,K], w [N,K], dy [M,N].

    Each tensor has its own generator (spawned in the order x, w, dy), so the
    result does not depend on ``which``. ``rows`` (optional) limits the token
    count M, e.g. to build the first rows of a large activation cheaply; the
    rows produced are the first rows of the full tensor only when no outlier
    columns are drawn, so tests that slice use the full generator instead.
    """
    M = lin["M"] if rows is None else rows
    N, K = lin["N"], lin["K"]
    gx, gw, gdy = tensor_streams(seed, 3)
    out = {}
    if "x" in which:
        out["x"] = bf16_normal(gx, (M, K), lin["x_std"], 0.01 if lin["x_outliers"] else 0.0)
    if "w" in which:
        out["w"] = bf16_normal(gw, (N, K), lin["w_std"])
    if "dy" in which:
        out["dy"] = bf16_normal(gdy, (M, N), lin["dy_std"], 0.01 if lin["dy_outliers"] else 0.0)
    return out


# ---------------------------------------------------------------------------
# Inputs whose quantization is lossless and whose GEMMs are exact in fp32.
# ---------------------------------------------------------------------------

def _small_grid():
    """k/4 for 0 <= k <= 64 with k of at most 4 significant bits (all E4M3 values)."""
    vals = []
    for k in range(0, 65):
        odd = k
        while odd and odd % 2 == 0:
            odd //= 2
        if odd < 16:
            vals.append(k / 4.0)
    return np.array(vals, dtype=np.float32)


SMALL_GRID = _small_grid()


# Values 448 * 2^-j (j = 0..2) and 0: products are multiples of 448^2 / 16, so
# every partial sum of up to 2048 terms needs at most 16 significant bits.
NARROW_GRID = np.array([0.0, 112.0, 224.0, 448.0], dtype=np.float32)


def exact_operand(rng, rows, cols, block_exp, grid=None):
    """bf16 bits of a [rows, cols] tensor built so that FP8 quantization is lossless.

    ``block_exp`` is an int array [rows/128, cols/128]; every element of block
    (i, j) is v * 2^block_exp[i, j] with v drawn from ``grid`` (SMALL_GRID by
    default; random sign),
    and the elements with r % 128 == c % 128 are +-448 * 2^block_exp[i, j].
    Every 1x128 row group, 128x1 column group and 128x128 block therefore has
    amax exactly 448 * 2^e, so its scale is the power of two 2^e and every
    element divided by it is an E4M3 value.
    """
    if rows % GROUP or cols % GROUP:
        raise ValueError("rows and cols must be multiples of 128")
    v = rng.choice(SMALL_GRID if grid is None else grid, size=(rows, cols)).astype(np.float32)
    diag = (np.arange(rows)[:, None] % GROUP) == (np.arange(cols)[None, :] % GROUP)
    v = np.where(diag, np.float32(448.0), v)
    v *= rng.choice(np.array([-1.0, 1.0], dtype=np.float32), size=(rows, cols))
    e = np.repeat(np.repeat(np.asarray(block_exp, dtype=np.int64), GROUP, axis=0), GROUP, axis=1)
    v = v * np.exp2(e).astype(np.float32)
    return f32_to_bf16_bits(v)


# ---------------------------------------------------------------------------
# Device-side generator for full-size tensors (same recipe, torch's Philox
# generator on the GPU). Used where a tensor is too large to draw on the host
# quickly; tests copy the slices they check back to the host.
# ---------------------------------------------------------------------------

def bf16_normal_device(shape, std, outlier_frac=0.0, seed=0, device="cuda", outlier_gain=20.0):
    """bf16 torch tensor of N(0, std^2) values with optional outlier columns, drawn on `device`."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    x.mul_(std)
    if outlier_frac > 0:
        C = shape[-1]
        n_out = int(round(outlier_frac * C))
        gc = torch.Generator(device="cpu")
        gc.manual_seed(int(seed) + 1)
        cols = torch.randperm(C, generator=gc)[:n_out].to(device)
        x[..., cols] *= outlier_gain
    return x.to(torch.bfloat16)


def linear_tensors_device(lin, seed=0, which=("x", "w", "dy"), device="cuda"):
    """Device bf16 tensors x [M,K], w [N,K], dy [M,N] of one linear (seeds seed, seed+10, seed+20)."""
    M, N, K = lin["M"], lin["N"], lin["K"]
    out = {}
    if "x" in which:
        out["x"] = bf16_normal_device((M, K), lin["x_std"], 0.01 if lin["x_outliers"] else 0.0, seed, device)
    if "w" in which:
        out["w"] = bf16_normal_device((N, K), lin["w_std"], 0.0, seed + 10, device)
    if "dy" in which:
        out["dy"] = bf16_normal_device((M, N), lin["dy_std"], 0.01 if lin["dy_outliers"] else 0.0, seed + 20, device)
    return out
