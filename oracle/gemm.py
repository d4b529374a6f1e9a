"""fp64 reference GEMMs over dequantized FP8 operands (oracle; test infrastructure only).

Source: Resumen Técnico: Jet-RL (gist.science), "Esquema de Cuantización":
the linear layers are FP8 GEMMs; forward Y = X W^T on 1x128-quantized X and
128x128-quantized W; DGrad dX = dY W with dY quantized 1x128 and the same
quantized W; WGrad dW = dY^T X with both operands grouped along the token
dimension (1x128 for dY^T, 128x1 for X). Gradients leave in bf16.

The reference value of every output element is the exact dot product of the
dequantized operands: x_hat = decode(q) * s (exact in float64, since a code
has at most 4 significant bits and a scale 24). It is accumulated in float64;
any summation order differs from the exact sum by ~1e-13 relative, far below
the tolerance. The GPU result (fp32 accumulation, bf16 output) is compared
with it by ``within_tolerance``:

    |gpu - ref| <= 2^-7 * |ref| + 1e-3 * rms(ref)     for every element,

rms taken over the whole output of the call (or over the sampled entries
when only a sample is computed).
"""

import numpy as np

from .e4m3 import decode

GROUP = 128
REL_TOL = 2.0 ** -7
RMS_TOL = 1e-3


def dequant_rows(q, s):
    """Row-grouped operand: q [R, L] codes, s [R, L/128] scales -> float64 [R, L]."""
    q = np.asarray(q)
    s = np.asarray(s, dtype=np.float32).astype(np.float64)
    return decode(q) * np.repeat(s, GROUP, axis=1)


def dequant_blocks(q, s):
    """128x128-block operand: q [N, K] codes, s [N/128, K/128] scales -> float64 [N, K]."""
    q = np.asarray(q)
    s = np.asarray(s, dtype=np.float32).astype(np.float64)
    return decode(q) * np.repeat(np.repeat(s, GROUP, axis=0), GROUP, axis=1)


def gemm_fwd(xq, xs, wq, ws, n=None):
    """Forward / rollout: Y[m, n] = sum_k x_hat[m, k] * w_hat[n, k]  (Y = X W^T).

    The code tensors may be padded to whole 128-groups (xq [M, Kp], wq [Np, Kp],
    +0 codes outside the tensor); `n` (default: every row of wq) is the number
    of output columns N kept.
    """
    y = dequant_rows(xq, xs) @ dequant_blocks(wq, ws).T
    return y if n is None else y[:, :n]


def gemm_dgrad(dyq, dys, wq, ws, k=None):
    """DGrad: dX[m, k] = sum_n dy_hat[m, n] * w_hat[n, k]  (dX = dY W).

    Takes the weight in its forward layout wq [N, K]; the contraction runs
    over N, so the 128x128 block scale ws[n/128, k/128] is reused unchanged.
    With padded code tensors (dyq [M, Np], wq [Np, Kp]) `k` is the number of
    output columns K kept (default: all).
    """
    dx = dequant_rows(dyq, dys) @ dequant_blocks(wq, ws)
    return dx if k is None else dx[:, :k]


def gemm_wgrad(dyq_t, dys_t, xq_t, xs_t):
    """WGrad: dW[n, k] = sum_m dy_hat[m, n] * x_hat[m, k]  (dW = dY^T X).

    Both operands come transposed, token-contiguous: dyq_t [N, M] with scales
    dys_t [N, M/128] and xq_t [K, M] with scales xs_t [K, M/128].
    """
    return dequant_rows(dyq_t, dys_t) @ dequant_rows(xq_t, xs_t).T


def bf16_rne(values):
    """Round float64 values to bf16 (nearest, ties to even); return uint16 bits.

    bf16 has 8 significant bits and float32's exponent range, with gradual
    underflow below 2^-126 (spacing 2^-133). Rounding is done once, directly
    from float64 (no intermediate float32 rounding). Values beyond the largest
    finite bf16 are rejected: they do not arise here.
    """
    v = np.asarray(values, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("bf16_rne: non-finite input")
    a = np.abs(v)
    _, exp2 = np.frexp(a)
    e = np.maximum(exp2.astype(np.int64) - 1, -126)    # binade, clamped at the subnormal range
    ulp = np.exp2((e - 7).astype(np.float64))
    r = np.rint(a / ulp) * ulp                           # exact scaling, ties to even
    if np.any(r >= 2.0 ** 128):
        raise ValueError("bf16_rne: overflow")
    r32 = r.astype(np.float32)                           # exact: r is a bf16 value
    bits = (r32.view(np.uint32) >> 16).astype(np.uint16)
    neg = np.signbit(v)
    return np.where(neg, bits | np.uint16(0x8000), bits).astype(np.uint16)


def bf16_bits_to_f64(bits):
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def within_tolerance(out_bf16_bits, ref, rms=None):
    """Check |out - ref| <= 2^-7 |ref| + 1e-3 rms(ref) element by element.

    Returns (all_ok, details) where details holds the worst ratio of error to
    bound and the number of violations. ``rms`` defaults to the rms of ref.
    """
    out = bf16_bits_to_f64(out_bf16_bits)
    ref = np.asarray(ref, dtype=np.float64)
    if rms is None:
        rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    bound = REL_TOL * np.abs(ref) + RMS_TOL * rms
    err = np.abs(out - ref)
    bad = ~(err <= bound)
    worst = float(np.max(np.where(bound > 0, err / np.where(bound > 0, bound, 1), np.where(err > 0, np.inf, 0.0)))) if ref.size else 0.0
    return (not bool(np.any(bad))), {"violations": int(np.sum(bad)), "worst_err_over_bound": worst, "rms": rms}
