"""GPU parity of the fused producers (RMSNorm and SwiGLU with their outputs quantized).

Two parts, as the contract of the entry points states:
* the produced bf16 values (y / h, written when asked) against the fp64
  oracle: at most one bf16 unit in the last place apart, since the kernels
  evaluate in fp32 (the bound and its derivation are in the design notes);
  the RMSNorm row statistic rstd within its fp32 summation bound;
* the FP8 codes and scales bit for bit against the oracle's quantizers applied
  to the GPU's own bf16 values, and unchanged when those values are not written.
Calls go through the C ABI (via the Python binding).
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_quantize_amd as fq
from fp8_block_scaled_quantize_amd import inputs
from oracle import fused, quant
from oracle.gemm import bf16_bits_to_f64
from tests._gpu import assert_bytes_equal, dev_bf16, host, host_bits, note, requires_gpu, sample_indices

pytestmark = [pytest.mark.gpu, requires_gpu]


def _np_bf16(shape, seed, std=1.0, outliers=0.0):
    (g,) = inputs.tensor_streams(seed, 1)
    return inputs.bf16_normal(g, shape, std, outliers)


def _assert_within_one_ulp(got_bits, ref_bits, what):
    got, ref = bf16_bits_to_f64(got_bits), bf16_bits_to_f64(ref_bits)
    ulp = np.maximum(fused.bf16_ulp(ref_bits), fused.bf16_ulp(got_bits))
    bad = np.abs(got - ref) > ulp
    assert not bad.any(), f"{what}: {bad.sum()} values more than one bf16 ulp from the oracle"
    exact = np.mean(got_bits == ref_bits)
    assert exact > 0.99, f"{what}: only {exact:.4f} of the values equal the oracle's"


def _check_codes(y_bits, xq, xs, xq_t, xs_t, what):
    oq, os_ = quant.quantize_act_1x128(y_bits)
    assert_bytes_equal(host(xs), os_, f"{what} xs")
    assert_bytes_equal(host(xq), oq, f"{what} xq", y_bits)
    if xq_t is not None:
        oqt, ost = quant.transpose_quantize_128x1(y_bits)
        assert np.array_equal(host(xs_t), ost)
        assert np.array_equal(host(xq_t), oqt)


def _rstd_bound(K):
    # fp32 sum of K squares: each lane adds K/512 chunks of 8 in order, then a
    # 6-level butterfly; plus the division, sqrt and reciprocal (a few ulps).
    return (K / 64 + 16) * 2.0 ** -24


@pytest.mark.parametrize("M,K,transposed", [(3, 384, False), (128, 640, True), (257, 1280, False),
                                            (256, 5120, True), (300, 640, True)])
def test_rmsnorm_quantize_matches_oracle(M, K, transposed):
    note(f"rmsnorm_quantize M={M} K={K} transposed={transposed}")
    x = _np_bf16((M, K), seed=M + K, outliers=0.01)
    g = _np_bf16((K,), seed=M + K + 1, std=0.5)
    eps = 1e-6
    xq, xs, xq_t, xs_t, rstd, y = fq.rmsnorm_quantize_1x128(dev_bf16(x), dev_bf16(g), eps, transposed, True)
    a = fq.rmsnorm_quantize_1x128(dev_bf16(x), dev_bf16(g), eps, transposed, False)
    torch.cuda.synchronize()
    yref, rref = fused.rmsnorm_bf16(x, g, eps)
    rel = np.abs(host(rstd).astype(np.float64) / rref - 1.0)
    assert rel.max() <= _rstd_bound(K), rel.max()
    yb = host_bits(y)
    _assert_within_one_ulp(yb, yref, "rmsnorm y")
    _check_codes(yb, xq, xs, xq_t, xs_t, "rmsnorm")
    assert torch.equal(a[0], xq) and torch.equal(a[1], xs) and torch.equal(a[4], rstd)
    if transposed:
        assert torch.equal(a[2], xq_t) and torch.equal(a[3], xs_t)


def test_rmsnorm_edge_rows():
    note("rmsnorm_quantize: zero row, constant rows, tiny and huge rows, eps = 0")
    K = 256
    x = _np_bf16((128, K), seed=91)
    x[0] = 0                                                 # all zero: rstd = 1/sqrt(eps)
    x[1] = inputs.f32_to_bf16_bits(np.full(K, 3.0, np.float32))
    x[2] = inputs.f32_to_bf16_bits(np.full(K, -0.5, np.float32))
    x[3] = inputs.f32_to_bf16_bits(bf16_bits_to_f64(x[3]).astype(np.float32) * np.float32(2.0 ** -60))
    x[4] = inputs.f32_to_bf16_bits(bf16_bits_to_f64(x[4]).astype(np.float32) * np.float32(2.0 ** 50))
    g = inputs.f32_to_bf16_bits(np.ones(K, np.float32))
    for eps in (1e-6, 0.0):
        xx = x[1:] if eps == 0.0 else x                        # eps = 0 on a zero row divides by zero
        xq, xs, _, _, rstd, y = fq.rmsnorm_quantize_1x128(dev_bf16(xx), dev_bf16(g), eps, False, True)
        torch.cuda.synchronize()
        yref, rref = fused.rmsnorm_bf16(xx, g, eps)
        yb = host_bits(y)
        got, ref = bf16_bits_to_f64(yb), bf16_bits_to_f64(yref)
        assert np.all(np.abs(got - ref) <= np.maximum(fused.bf16_ulp(yref), fused.bf16_ulp(yb)))
        _check_codes(yb, xq, xs, None, None, f"rmsnorm eps={eps}")
    # constant rows with gamma = 1 and eps = 0 normalize to exactly +-1
    assert np.all(yb[0] == 0x3F80) and np.all(yb[1] == 0xBF80)


@pytest.mark.parametrize("M,N,transposed", [(5, 384, False), (128, 640, True), (256, 27648, True),
                                            (200, 384, True)])
def test_swiglu_quantize_matches_oracle(M, N, transposed):
    note(f"swiglu_quantize M={M} N={N} transposed={transposed}")
    gt = _np_bf16((M, N), seed=3 * M + N, std=2.0)
    up = _np_bf16((M, N), seed=3 * M + N + 1)
    gt[0, :8] = inputs.f32_to_bf16_bits(np.array([0, -0.0, 100, -100, 88.5, -88.5, 1e-30, -1e-30], np.float32))
    hq, hs, hq_t, hs_t, h = fq.swiglu_quantize_1x128(dev_bf16(gt), dev_bf16(up), transposed, True)
    a = fq.swiglu_quantize_1x128(dev_bf16(gt), dev_bf16(up), transposed, False)
    torch.cuda.synchronize()
    href = fused.swiglu_bf16(gt, up)
    hb = host_bits(h)
    _assert_within_one_ulp(hb, href, "swiglu h")
    _check_codes(hb, hq, hs, hq_t, hs_t, "swiglu")
    assert torch.equal(a[0], hq) and torch.equal(a[1], hs)
    if transposed:
        assert torch.equal(a[2], hq_t) and torch.equal(a[3], hs_t)


def test_fused_full_size_codes_equal_dual_quantizer():
    M, K, N = 32768, 5120, 27648
    note(f"rmsnorm [{M},{K}] and swiglu [{M},{N}] at full size: codes vs the dual quantizer of y, y sampled vs oracle")
    x = inputs.bf16_normal_device((M, K), 1.0, 0.01, seed=31)
    g = inputs.bf16_normal_device((K,), 0.5, 0.0, seed=32)
    xq, xs, xq_t, xs_t, rstd, y = fq.rmsnorm_quantize_1x128(x, g, 1e-6, True, True)
    d = fq.quantize_dual_1x128_128x1(y)
    torch.cuda.synchronize()
    assert torch.equal(xq, d[0]) and torch.equal(xs, d[1]) and torch.equal(xq_t, d[2]) and torch.equal(xs_t, d[3])
    rows = sample_indices(M, 24, seed=6)
    yref, rref = fused.rmsnorm_bf16(host_bits(x[rows]), host_bits(g), 1e-6)
    _assert_within_one_ulp(host_bits(y[rows]), yref, "rmsnorm y (sampled rows)")
    assert np.max(np.abs(host(rstd[rows]).astype(np.float64) / rref - 1)) <= _rstd_bound(K)
    del x, y, xq, xs, xq_t, xs_t, d
    gt = inputs.bf16_normal_device((M, N), 2.0, 0.0, seed=33)
    up = inputs.bf16_normal_device((M, N), 1.0, 0.0, seed=34)
    hq, hs, hq_t, hs_t, h = fq.swiglu_quantize_1x128(gt, up, True, True)
    d = fq.quantize_dual_1x128_128x1(h)
    torch.cuda.synchronize()
    assert torch.equal(hq, d[0]) and torch.equal(hs, d[1]) and torch.equal(hq_t, d[2]) and torch.equal(hs_t, d[3])
    href = fused.swiglu_bf16(host_bits(gt[rows]), host_bits(up[rows]))
    _assert_within_one_ulp(host_bits(h[rows]), href, "swiglu h (sampled rows)")
