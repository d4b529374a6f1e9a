"""The three group quantizers of the FP8 linear-layer flow (oracle; test infrastructure only).

Source: Resumen Técnico: Jet-RL (gist.science), section "Esquema de
Cuantización" -- activations are quantized in 1x128 groups, weights in 128x128
blocks, and the WGrad operands in 1x128 / 128x1 groups; "Arquitectura
Central" -- master weights are bf16 and one quantization flow serves rollout
and training.

One group G of bf16 values is quantized as follows (every step in IEEE
binary32, round-to-nearest-even, no flush-to-zero):

    x_j  = float32(G_j)                    exact widening of bf16
    amax = max_j |x_j|                     exact
    s    = 1.0                 if amax == 0   (an all-zero group; reading: keeps
                                               the rule uniform and decodes to 0)
         = fl32(amax / 448)    otherwise      (one float32 division)
    q_j  = E4M3_RNE( fl32(x_j / s) )          (one float32 division per element,
                                               then the codec in e4m3.encode)

A group is 128 consecutive elements of a row (1x128), a 128x128 tile
(128x128), or 128 consecutive rows of one column (128x1). A dimension that is
not a multiple of 128 ends in a partial group holding the remaining elements:
its amax is theirs, and the code tensors are padded to whole groups along that
dimension with code 0x00 (+0), which a contraction reads as zero products.
(Reading: the pages fix no layout for a partial group; quantizing the tensor
zero-padded to whole groups gives exactly these codes and scales, since +0
never raises an amax and encodes to 0x00.)

Inputs are bf16 bit patterns (uint16 arrays); outputs are E4M3 bytes (uint8)
and float32 scales.
"""

import numpy as np

from .e4m3 import bf16_bits_to_f32, encode

GROUP = 128
FP8_MAX = np.float32(448.0)


def _grouped_scales_and_codes(groups):
    """Quantize every row of a [G, n] float32 array as one group (the rule in
    the module docstring): the amax is per row, the scale is one float32
    division per row (1.0 for an all-zero row), the quotient one float32
    division per element, then the E4M3 encoder.
    """
    g = np.asarray(groups, dtype=np.float32)
    amax = np.max(np.abs(g), axis=1)
    s = np.where(amax == 0, np.float32(1.0),
                 (amax / FP8_MAX).astype(np.float32)).astype(np.float32)
    q = encode((g / s[:, None]).astype(np.float32))
    return q, s


def _groups(n):
    """Number of 128-element groups covering n elements, and the padded length."""
    g = (n + GROUP - 1) // GROUP
    return g, g * GROUP


def quantize_act_1x128(x_bits):
    """1x128 per-token group quantization of a bf16 [M, K] activation.

    Source: "Esquema de Cuantización", activations bullet (1x128 per group);
    the same quantizer serves dY before DGrad (backward GEMMs in FP8).

    Any K is accepted. With Kg = ceil(K / 128) and Kp = 128 * Kg, returns
    xq uint8 [M, Kp] and xs float32 [M, Kg], where xs[m, g] is the scale of
    x[m, 128g : min(128g + 128, K)] and xq[m, k] = 0x00 for k >= K.
    """
    x = bf16_bits_to_f32(x_bits)
    M, K = x.shape
    Kg, Kp = _groups(K)
    xp = np.zeros((M, Kp), dtype=np.float32)              # +0 beyond the last channel
    xp[:, :K] = x
    q, s = _grouped_scales_and_codes(xp.reshape(M * Kg, GROUP))
    return q.reshape(M, Kp), s.reshape(M, Kg)


def quantize_weight_128x128(w_bits):
    """128x128 per-block quantization of a bf16 [N, K] weight.

    Source: "Esquema de Cuantización", weights bullet (128x128 per block);
    "Arquitectura Central", bf16 master weights re-quantized for each use.

    Any N and K are accepted. With Nb = ceil(N / 128), Np = 128 * Nb (and Kb,
    Kp likewise), returns wq uint8 [Np, Kp], ws float32 [Nb, Kb] (ws[i, j] is
    the scale of the block w[128i : min(128i + 128, N), 128j : min(128j + 128, K)])
    and wq_t = wq transposed ([Kp, Np]), the operand layout DGrad reads; codes
    outside [0, N) x [0, K) are 0x00. A 128x128 block has the same amax
    transposed, so wq_t is exactly the byte transpose of wq.
    """
    w = bf16_bits_to_f32(w_bits)
    N, K = w.shape
    Nb, Np = _groups(N)
    Kb, Kp = _groups(K)
    wp = np.zeros((Np, Kp), dtype=np.float32)             # +0 outside the weight
    wp[:N, :K] = w
    blocks = wp.reshape(Nb, GROUP, Kb, GROUP).transpose(0, 2, 1, 3)
    q, s = _grouped_scales_and_codes(blocks.reshape(Nb * Kb, GROUP * GROUP))
    wq = q.reshape(Nb, Kb, GROUP, GROUP).transpose(0, 2, 1, 3).reshape(Np, Kp)
    ws = s.reshape(Nb, Kb)
    return wq, ws, np.ascontiguousarray(wq.T)


def transpose_quantize_128x1(x_bits):
    """128x1 group quantization of a bf16 [M, C] tensor, written transposed.

    Source: "Esquema de Cuantización", backward bullets: WGrad runs in FP8
    with 1x128 / 128x1 operand groups, and saved activations are kept in FP8.
    Each group is 128 consecutive tokens of one channel, i.e. it runs along
    the token dimension, which is WGrad's contraction dimension.

    Any token count M and channel count C are accepted (C is not grouped
    here). With Mp = 128 * ceil(M / 128), returns
    xq_t uint8 [C, Mp] and xs_t float32 [C, Mp/128]: xq_t[c, m] is the code of
    x[m, c] and xs_t[c, b] the scale of the group x[128b : min(128b + 128, M), c].
    When M is not a multiple of 128 the last group holds the remaining tokens
    (its amax is theirs) and the positions m >= M hold code 0x00 (+0), which a
    contraction over the tokens reads as zero products. (Reading: the pages
    fix no layout for a ragged tail; padding the transposed copy keeps WGrad's
    contraction a whole number of 128-token blocks.)
    """
    x = bf16_bits_to_f32(x_bits)
    M, C = x.shape
    Mb, Mp = _groups(M)
    xt = np.zeros((C, Mp), dtype=np.float32)            # +0 beyond the last token
    xt[:, :M] = x.T
    q, s = _grouped_scales_and_codes(xt.reshape(C * Mb, GROUP))
    return q.reshape(C, Mp), s.reshape(C, Mb)
