"""Exact-arithmetic helpers for pinning the oracle (tests only).

Everything here works on fractions.Fraction, so it shares no floating-point
behaviour with the oracle it checks.
"""

import math
from fractions import Fraction


def e4m3_values():
    """All finite non-negative E4M3 values with their codes, built by enumeration.

    Listed from the format's grid rather than from a decode formula: the
    subnormal binade holds k/512 (k = 0..7); binade e = -6..8 holds
    (8 + t) * 2^(e - 3) for t = 0..7, except the top slot (e = 8, t = 7),
    which is NaN. Codes count up with the value.
    """
    vals = [Fraction(k, 512) for k in range(8)]
    for e in range(-6, 9):
        for t in range(8):
            if e == 8 and t == 7:
                continue
            vals.append(Fraction(8 + t) * Fraction(2) ** (e - 3))
    return list(enumerate(vals))          # code == position for the positive half


_E4M3 = e4m3_values()


def nearest_e4m3_code(v):
    """Brute-force nearest E4M3 code to the rational v (ties to the even code), sign kept."""
    neg = v < 0
    a = -v if neg else v
    best = None
    for code, val in _E4M3:
        d = abs(val - a)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    return best[1] | (0x80 if neg else 0)


def _floor_log2(a):
    """floor(log2 a) for a positive rational, exactly."""
    e = math.frexp(float(a))[1] - 1 if float(a) > 0 else -1100
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def _round_to_grid(v, mant_bits, min_exp):
    """Round rational v to a binary grid with mant_bits significant bits, ties to even."""
    if v == 0:
        return Fraction(0)
    s = -1 if v < 0 else 1
    a = abs(v)
    e = max(_floor_log2(a), min_exp)
    ulp = Fraction(2) ** (e - (mant_bits - 1))
    q, r = divmod(a, ulp)
    n = int(q)
    if r * 2 > ulp or (r * 2 == ulp and n % 2 == 1):
        n += 1
    return s * n * ulp


def rn_float32(v):
    """Nearest float32 to a rational (ties to even; gradual underflow below 2^-126)."""
    return _round_to_grid(v, 24, -126)


def rn_bf16(v):
    """Nearest bf16 to a rational (ties to even; gradual underflow below 2^-126)."""
    return _round_to_grid(v, 8, -126)
