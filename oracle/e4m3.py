"""OCP 8-bit E4M3 codec and bf16 helpers (oracle; test infrastructure only).

The pages only say "FP8" (Resumen Técnico: Jet-RL, "Esquema de Cuantización").
The format used throughout is OCP E4M3 with the finite-only convention
("E4M3FN"): exponent bias 7, 3 mantissa bits, no infinities, NaN only at
0x7F / 0xFF, largest finite magnitude 448 (0x7E), smallest normal 2^-6,
subnormals k * 2^-9 for k = 1..7, and a signed zero (0x00 / 0x80).

Everything here is written from that definition with plain numpy, value by
value, so that it can be read against the definition by eye.
"""

import numpy as np

E4M3_MAX = 448.0
MIN_NORMAL = 2.0 ** -6
SUBNORMAL_STEP = 2.0 ** -9


def decode(codes):
    """Map E4M3 bytes to their exact values (float64; NaN for 0x7F / 0xFF).

    Byte layout: sign bit 7, exponent field E = bits 6..3, mantissa T = bits
    2..0. E == 0 is subnormal: T * 2^-9. Otherwise (8 + T) * 2^(E - 10),
    i.e. (1 + T/8) * 2^(E - 7). E == 15 with T == 7 is NaN.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    negative = (c & 0x80) != 0
    E = (c >> 3) & 0xF
    T = c & 0x7
    magnitude = np.where(E == 0,
                         T * SUBNORMAL_STEP,
                         (8 + T) * np.exp2(E.astype(np.float64) - 10.0))
    value = np.where(negative, -magnitude, magnitude)
    return np.where((E == 15) & (T == 7), np.nan, value)


def encode(values):
    """Round float32 values to E4M3 bytes, nearest value, ties to even mantissa.

    Steps, following the format definition:
      1. the sign bit of the input is kept, also for -0.0 and for negative
         values that round to zero;
      2. a = |v| is taken exactly (float64 holds every float32);
      3. below the smallest normal 2^-6 the grid is k * 2^-9; k = RNE(a * 2^9)
         lies in 0..8, and k == 8 is exactly the code of 2^-6;
      4. otherwise e = floor(log2 a) is read from the float's exponent,
         m = RNE(a * 2^(3 - e)) lies in 8..16, and m == 16 carries into the
         next binade (e + 1, m = 8); the byte is ((e + 7) << 3) | (m - 8).
    Magnitudes above 464 (the midpoint between 448 and the NaN slot) have no
    finite nearest code; they never arise from the quantizers and are
    rejected. Non-finite inputs are rejected too.
    """
    v = np.asarray(values, dtype=np.float32)
    if not np.all(np.isfinite(v)):
        raise ValueError("E4M3 encode: non-finite input")
    sign = ((v.view(np.uint32) >> 31).astype(np.uint8) << 7).astype(np.uint8)
    a = np.abs(v.astype(np.float64))
    if np.any(a > 464.0):
        raise ValueError("E4M3 encode: magnitude above 464 has no finite code")

    out = np.zeros(v.shape, dtype=np.uint8)
    small = a < MIN_NORMAL
    # np.rint rounds half to even; the scaling by 2^9 is exact in float64.
    out[small] = np.rint(a[small] / SUBNORMAL_STEP).astype(np.uint8)

    big = ~small
    ab = a[big]
    frac, exp2 = np.frexp(ab)          # ab = frac * 2^exp2, frac in [0.5, 1)
    e = exp2.astype(np.int64) - 1      # floor(log2 ab), exact
    m = np.rint(ab * np.exp2(3.0 - e)).astype(np.int64)
    carry = m == 16
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 8, m)
    out[big] = (((e + 7) << 3) | (m - 8)).astype(np.uint8)
    return out | sign


def bf16_bits_to_f32(bits):
    """bf16 bit patterns (uint16) -> float32, exactly (a 16-bit left shift)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)
