"""Pins of the RMSNorm and SwiGLU oracle (CPU only).

Each check compares the oracle with something other than its own formula:
closed forms, exact high-precision arithmetic (``decimal`` at 60 digits),
torch's float64 implementations, and exact invariances.
"""

import decimal
from decimal import Decimal

import numpy as np
import pytest
import torch

from fp8_block_scaled_quantize_amd import inputs
from oracle import fused
from oracle.gemm import bf16_bits_to_f64

decimal.getcontext().prec = 60


def _bits(v):
    return inputs.f32_to_bf16_bits(np.asarray(v, dtype=np.float32))


def _dec(bits):
    return Decimal(float(bf16_bits_to_f64(np.uint16(bits))))


def _assert_rounded_once(cand_bits, exact):
    """cand (bf16) is the nearest bf16 to the Decimal `exact`, ties to even mantissa."""
    for cb, ex in zip(np.ravel(cand_bits), np.ravel(exact)):
        c = _dec(cb)
        ulp = Decimal(float(fused.bf16_ulp(np.uint16(cb))))
        # the spacing below a power of two is half as large
        mag = abs(c)
        if mag != 0 and (float(mag) == 2.0 ** np.floor(np.log2(float(mag)))) and abs(ex) < mag:
            ulp = ulp / 2
        err = abs(ex - c)
        assert err <= ulp / 2, (hex(int(cb)), float(c), float(ex))
        if err == ulp / 2:
            assert (int(cb) & 1) == 0, "tie not rounded to even"


# ---------------------------------------------------------------- RMSNorm --

@pytest.mark.parametrize("c", [1.0, -3.0, 0.15625, 2.0 ** -20, -448.0])
def test_rmsnorm_constant_row_closed_form(c):
    K = 256
    x = _bits(np.full((2, K), c))
    g = _bits(np.ones(K))
    y, r = fused.rmsnorm_bf16(x, g, 0.0)
    cb = float(bf16_bits_to_f64(x[0, 0]))
    assert np.all(r == 1.0 / abs(cb))                     # mean of squares is c^2
    want = 0x3F80 if cb > 0 else 0xBF80                     # exactly +-1
    assert np.all(y == want)
    eps = 0.25
    y2, _ = fused.rmsnorm_bf16(x, g, eps)
    exact = _dec(x[0, 0]) / (_dec(x[0, 0]) ** 2 + Decimal(eps)).sqrt()
    _assert_rounded_once(y2[0, :3], [exact] * 3)


def test_rmsnorm_matches_exact_arithmetic():
    (rng,) = inputs.tensor_streams(71, 1)
    for K in (8, 128, 384):
        x = inputs.bf16_normal(rng, (3, K), 1.5, 0.0)
        g = inputs.bf16_normal(rng, (K,), 1.0, 0.0)
        eps = 1e-6
        y, r = fused.rmsnorm_bf16(x, g, eps)
        for m in range(3):
            xs = [_dec(b) for b in x[m]]
            ms = sum(v * v for v in xs) / K
            rstd = 1 / (ms + Decimal(eps)).sqrt()
            assert abs(float(rstd) - r[m]) <= 4e-16 * r[m]
            exact = [xs[k] * rstd * _dec(g[k]) for k in range(K)]
            _assert_rounded_once(y[m], exact)


def test_rmsnorm_matches_torch_float64():
    (rng,) = inputs.tensor_streams(72, 1)
    x = inputs.bf16_normal(rng, (16, 5120), 1.0, 0.01)
    g = inputs.bf16_normal(rng, (5120,), 0.5, 0.0)
    y, r = fused.rmsnorm_bf16(x, g, 1e-6)
    xt = torch.from_numpy(bf16_bits_to_f64(x))
    gt = torch.from_numpy(bf16_bits_to_f64(g))
    ref = torch.nn.functional.rms_norm(xt, (5120,), weight=gt, eps=1e-6).numpy()
    got = bf16_bits_to_f64(y)
    assert np.all(np.abs(got - ref) <= fused.bf16_ulp(y) / 2 * (1 + 1e-9) + 1e-300)


def test_rmsnorm_invariances():
    (rng,) = inputs.tensor_streams(73, 1)
    x = inputs.bf16_normal(rng, (8, 640), 1.0, 0.01)
    g = inputs.bf16_normal(rng, (640,), 1.0, 0.0)
    y, _ = fused.rmsnorm_bf16(x, g, 0.0)
    x8 = _bits(bf16_bits_to_f64(x) * 8.0)                  # exact power-of-two scaling
    y8, _ = fused.rmsnorm_bf16(x8, g, 0.0)
    assert np.array_equal(y, y8)                           # scale invariance (eps = 0)
    g4 = _bits(bf16_bits_to_f64(g) * 0.25)
    y4, _ = fused.rmsnorm_bf16(x, g4, 0.0)
    assert np.array_equal(bf16_bits_to_f64(y4), bf16_bits_to_f64(y) * 0.25)


# ----------------------------------------------------------------- SwiGLU --

def test_silu_special_values_and_limits():
    t = np.array([0.0, -0.0, 64.0, 300.0, -200.0, -1000.0])
    s = fused.silu(t)
    assert s[0] == 0.0 and s[1] == 0.0
    assert abs(s[2] - 64.0) < 1e-24 and s[3] == 300.0
    assert s[4] < 0 and s[4] > -1e-80 and s[5] == 0.0 and np.signbit(s[5])
    h = fused.swiglu_bf16(_bits([-200.0, 300.0, 64.0]), _bits([1.0, 1.0, -2.0]))
    assert list(h) == [0x8000, 0x4396, 0xC300]            # -0, 300, -128


def test_silu_identity_and_torch():
    t = np.linspace(-30, 30, 2001)
    s = fused.silu(t)
    assert np.allclose(s - fused.silu(-t), t, rtol=1e-14, atol=1e-14)
    ref = torch.nn.functional.silu(torch.from_numpy(t)).numpy()
    assert np.allclose(s, ref, rtol=1e-15, atol=1e-300)


def test_swiglu_matches_exact_arithmetic():
    (rng,) = inputs.tensor_streams(74, 1)
    g = inputs.bf16_normal(rng, (64,), 2.0, 0.0)
    u = inputs.bf16_normal(rng, (64,), 1.0, 0.0)
    h = fused.swiglu_bf16(g, u)
    exact = []
    for gb, ub in zip(g, u):
        gd, ud = _dec(gb), _dec(ub)
        exact.append(gd / (1 + (-gd).exp()) * ud)
    _assert_rounded_once(h, exact)


def test_swiglu_linear_in_up():
    (rng,) = inputs.tensor_streams(75, 1)
    g = inputs.bf16_normal(rng, (4, 256), 2.0, 0.0)
    u = inputs.bf16_normal(rng, (4, 256), 1.0, 0.0)
    h = fused.swiglu_bf16(g, u)
    h2 = fused.swiglu_bf16(g, _bits(bf16_bits_to_f64(u) * -2.0))
    assert np.array_equal(bf16_bits_to_f64(h2), bf16_bits_to_f64(h) * -2.0)
