"""The operators whose outputs are quantized in place (oracle; test infrastructure only).

Source: Resumen Técnico: Jet-RL (gist.science). "Esquema de Cuantización":
activations saved for the backward pass are stored in FP8, with the
quantization fused into the operator that produces them. "Implementación":
the quantization kernels are fused with the activation and RMSNorm operators.

The two producers in front of the linear layers of a Llama/Qwen block:

* RMSNorm of the residual stream x [M, K] with a bf16 weight gamma [K]:
      rstd_m = 1 / sqrt( (1/K) * sum_k x[m,k]^2 + eps )
      y[m,k] = bf16( x[m,k] * rstd_m * gamma[k] )
* the gated activation (SwiGLU) of the gate and up projections g, u [M, N]:
      h[m,n] = bf16( silu(g[m,n]) * u[m,n] ),   silu(t) = t / (1 + exp(-t))

The fused kernels then quantize y (or h) exactly as the 1x128 / 128x1
quantizers of ``quant`` do. Here the operators are evaluated in float64 and
rounded once to bf16 (nearest, ties to even); the GPU evaluates them in
float32, so its bf16 output may differ from this one by one bf16 unit in the
last place where the exact value lies within float32 error of a rounding
boundary (the tolerance is derived in the design notes).

Inputs are bf16 bit patterns (uint16 arrays); outputs are bf16 bit patterns
and, for RMSNorm, the float64 rstd.
"""

import numpy as np

from .gemm import bf16_bits_to_f64, bf16_rne


def rms_rstd(x_bits, eps):
    """rstd_m = (mean_k x[m,k]^2 + eps)^(-1/2) in float64, one value per row."""
    x = bf16_bits_to_f64(x_bits)
    ms = np.mean(x * x, axis=-1)
    return 1.0 / np.sqrt(ms + float(eps))


def rmsnorm_bf16(x_bits, gamma_bits, eps):
    """RMSNorm over the last dimension; returns (y bf16 bits, rstd float64)."""
    x = bf16_bits_to_f64(x_bits)
    g = bf16_bits_to_f64(gamma_bits)
    if x.shape[-1] != g.shape[-1]:
        raise ValueError("gamma must have the length of the normalized dimension")
    r = rms_rstd(x_bits, eps)
    return bf16_rne(x * r[..., None] * g), r


def silu(t):
    """t * sigmoid(t) = t / (1 + exp(-t)) in float64 (exp overflow gives -0 or 0 as the limit)."""
    t = np.asarray(t, dtype=np.float64)
    with np.errstate(over="ignore"):
        return t / (1.0 + np.exp(-t))


def swiglu_bf16(g_bits, u_bits):
    """h = bf16(silu(g) * u) elementwise; returns bf16 bits."""
    g = bf16_bits_to_f64(g_bits)
    u = bf16_bits_to_f64(u_bits)
    if g.shape != u.shape:
        raise ValueError("gate and up must have the same shape")
    return bf16_rne(silu(g) * u)


def bf16_ulp(bits):
    """Spacing of bf16 values at the magnitude of each element (subnormal spacing 2^-133)."""
    v = np.abs(bf16_bits_to_f64(bits))
    _, e2 = np.frexp(v)
    e = np.maximum(e2.astype(np.int64) - 1, -126)
    return np.exp2((e - 7).astype(np.float64))
