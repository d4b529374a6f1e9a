"""Pins of the oracle's E4M3 codec against things other than itself.

* the decode table against torch's float8_e4m3fn (an independent library)
  and against a grid enumerated in exact rationals;
* the encoder against a brute-force nearest-value search (exact rationals)
  at every midpoint and its float32 neighbours, on every bf16 value, and
  against torch's float8_e4m3fn cast on a structured sweep of float32.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import e4m3
from tests._exact import e4m3_values, nearest_e4m3_code


def _torch_cast(v32):
    return torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_matches_torch_and_enumerated_grid():
    codes = np.arange(256, dtype=np.uint8)
    dec = e4m3.decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(dec), nan)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(dec[~nan], ref[~nan])
    assert np.array_equal(np.signbit(dec[~nan]), np.signbit(ref[~nan]))
    for code, val in e4m3_values():
        assert Fraction(float(dec[code])) == val
        assert Fraction(float(dec[code | 0x80])) == -val


def test_decode_named_values():
    d = e4m3.decode(np.array([0x7E, 0xFE, 0x08, 0x01, 0x07, 0x38, 0x00, 0x80], dtype=np.uint8))
    assert list(d[:6]) == [448.0, -448.0, 2.0 ** -6, 2.0 ** -9, 7 * 2.0 ** -9, 1.0]
    assert d[6] == 0 and not np.signbit(d[6])
    assert d[7] == 0 and np.signbit(d[7])
    finite = np.isfinite(e4m3.decode(np.arange(256, dtype=np.uint8)))
    assert finite.sum() == 254


def _midpoint_probe_set():
    """Every midpoint between adjacent non-negative codes, and its float32 neighbours."""
    vals = [float(v) for _, v in e4m3_values()]
    probes = []
    for lo, hi in zip(vals[:-1], vals[1:]):
        mid = np.float32((lo + hi) / 2)          # exact: midpoints have 5 significant bits
        assert float(mid) == (lo + hi) / 2
        probes += [mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))]
    probes += [np.float32(v) for v in vals]
    top_mid = np.float32(464.0)                  # between 448 and the NaN slot: ties down to 448
    probes += [top_mid, np.nextafter(top_mid, np.float32(0))]
    return np.array(probes, dtype=np.float32)


def test_encode_brute_force_at_midpoints():
    p = _midpoint_probe_set()
    p = np.concatenate([p, -p])
    got = e4m3.encode(p)
    for v, g in zip(p, got):
        want = nearest_e4m3_code(Fraction(float(v)))
        if np.signbit(v) and want == 0:
            want = 0x80
        assert g == want, (float(v), hex(g), hex(want))


def test_encode_brute_force_every_bf16_in_range():
    bits = np.arange(0x10000, dtype=np.uint32) << 16
    v = bits.astype(np.uint32).view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 464)]
    got = e4m3.encode(v)
    # Brute force: distance from |v| to every finite code value, ties to the even code.
    grid = np.array([float(x) for _, x in e4m3_values()])
    a = np.abs(v.astype(np.float64))
    dist = np.abs(a[:, None] - grid[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    even = cand & (np.arange(grid.size)[None, :] % 2 == 0)
    code = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1)).astype(np.uint8)
    code |= np.where(np.signbit(v), 0x80, 0).astype(np.uint8)
    assert np.array_equal(got, code)


def test_encode_matches_torch_on_float32_sweep():
    # Every float32 with |v| <= 464 whose low 12 bits are one of a few
    # patterns (covers every tie and both neighbours of every tie, since a tie
    # has at least 19 trailing zero bits) plus a dense random sample.
    hi = np.arange(0, 0x43E81, dtype=np.uint32) << 12
    lows = np.array([0x000, 0x001, 0x7FF, 0x800, 0x801, 0xFFF], dtype=np.uint32)
    bits = (hi[:, None] | lows[None, :]).ravel()
    rng = np.random.default_rng(1234)
    bits = np.concatenate([bits, rng.integers(0, 0x43E80001, size=2_000_000, dtype=np.uint32)])
    v = bits.view(np.float32)
    v = v[np.abs(v) <= 464]
    v = np.concatenate([v, -v])
    assert np.array_equal(e4m3.encode(v), _torch_cast(v))


def test_encode_sign_of_zero():
    got = e4m3.encode(np.array([0.0, -0.0, 1e-4, -1e-4, -2.0 ** -10, 2.0 ** -10], dtype=np.float32))
    assert list(got) == [0x00, 0x80, 0x00, 0x80, 0x80, 0x00]


def test_encode_rejects_out_of_contract():
    with pytest.raises(ValueError):
        e4m3.encode(np.array([464.01], dtype=np.float32))
    with pytest.raises(ValueError):
        e4m3.encode(np.array([np.nan], dtype=np.float32))


def test_bf16_widening_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0001, 0x7F7F, 0x8000], dtype=np.uint16)
    v = e4m3.bf16_bits_to_f32(bits)
    assert list(v[:2]) == [1.0, -1.0]
    assert v[2] == np.float32(2.0 ** -133)
    assert v[3] == np.float32(3.3895313892515355e38)
    assert np.signbit(v[4]) and v[4] == 0
