"""GPU parity for channel counts that are not a multiple of 128 (partial groups).

The last 1x128 group of a row, the last 128x128 blocks of a weight and the
last channel block of the 128x1 / dual / fused quantizers are partial: codes
and scales bit-exact against the oracle (whose padded codes are +0), GEMMs
within the tolerance, the grouped calls equal to the plain ones, and
FP8Linear training with such feature counts. Calls go through the C ABI.
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_quantize_amd as fq
from fp8_block_scaled_quantize_amd import inputs
from fp8_block_scaled_quantize_amd.linear import FP8Linear
from oracle import fused, gemm, quant
from tests._gpu import assert_bytes_equal, dev_bf16, dev_f32, dev_u8, host, host_bits, note, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def _np_bf16(rows, cols, seed, std=1.0, outliers=0.01):
    (g,) = inputs.tensor_streams(seed, 1)
    return inputs.bf16_normal(g, (rows, cols), std, outliers)


def _assert_close(got_bits, ref, what):
    ok, info = gemm.within_tolerance(got_bits, ref)
    assert ok, f"{what}: {info}"


@pytest.mark.parametrize("M,K", [(3, 8), (130, 200), (64, 264), (257, 1032), (1, 4104)])
def test_act_partial_group(M, K):
    note(f"act_1x128 partial group M={M} K={K}")
    x = _np_bf16(M, K, seed=M + 3 * K)
    xq, xs = fq.quantize_act_1x128(dev_bf16(x))
    torch.cuda.synchronize()
    oq, os_ = quant.quantize_act_1x128(x)
    assert_bytes_equal(host(xs), os_, "xs")
    assert_bytes_equal(host(xq), oq, "xq")


@pytest.mark.parametrize("N,K", [(8, 8), (136, 200), (296, 1032), (1000, 264)])
def test_weight_partial_blocks(N, K):
    note(f"weight_128x128 partial blocks N={N} K={K}")
    w = _np_bf16(N, K, seed=N + 5 * K, std=0.02)
    wq, ws, wq_t = fq.quantize_weight_128x128(dev_bf16(w))
    wq2, ws2, none = fq.quantize_weight_128x128(dev_bf16(w), transposed=False)
    torch.cuda.synchronize()
    oq, os_, oqt = quant.quantize_weight_128x128(w)
    assert_bytes_equal(host(ws), os_, "ws")
    assert_bytes_equal(host(wq), oq, "wq")
    assert_bytes_equal(host(wq_t), oqt, "wq_t")
    assert none is None and torch.equal(wq2, wq) and torch.equal(ws2, ws)


@pytest.mark.parametrize("M,C", [(128, 8), (300, 200), (256, 1032)])
def test_transpose_partial_channel_block(M, C):
    note(f"transpose_128x1 partial channel block M={M} C={C}")
    x = _np_bf16(M, C, seed=7 * M + C)
    qt, st = fq.transpose_quantize_128x1(dev_bf16(x))
    torch.cuda.synchronize()
    oqt, ost = quant.transpose_quantize_128x1(x)
    assert_bytes_equal(host(st), ost, "xs_t")
    assert_bytes_equal(host(qt), oqt, "xq_t")


@pytest.mark.parametrize("M,K", [(77, 200), (256, 8), (300, 1032)])
def test_dual_partial_group(M, K):
    note(f"dual partial group M={M} K={K}")
    x = _np_bf16(M, K, seed=11 * M + K)
    xq, xs, qt, st = fq.quantize_dual_1x128_128x1(dev_bf16(x))
    torch.cuda.synchronize()
    oq, os_ = quant.quantize_act_1x128(x)
    oqt, ost = quant.transpose_quantize_128x1(x)
    assert_bytes_equal(host(xq), oq, "xq")
    assert_bytes_equal(host(xs), os_, "xs")
    assert_bytes_equal(host(qt), oqt, "xq_t")
    assert_bytes_equal(host(st), ost, "xs_t")


@pytest.mark.parametrize("M,K", [(130, 200), (3, 1032)])
def test_rmsnorm_partial_group(M, K):
    note(f"rmsnorm_quantize partial group M={M} K={K}")
    x = _np_bf16(M, K, seed=M + K, outliers=0.01)
    g = _np_bf16(1, K, seed=M + K + 1, std=0.5, outliers=0.0)[0]
    xq, xs, xq_t, xs_t, rstd, y = fq.rmsnorm_quantize_1x128(dev_bf16(x), dev_bf16(g), 1e-6, True, True)
    torch.cuda.synchronize()
    yb = host_bits(y)
    yref, rref = fused.rmsnorm_bf16(x, g, 1e-6)
    ulp = np.maximum(fused.bf16_ulp(yref), fused.bf16_ulp(yb))
    assert np.all(np.abs(gemm.bf16_bits_to_f64(yb) - gemm.bf16_bits_to_f64(yref)) <= ulp)
    assert np.max(np.abs(host(rstd).astype(np.float64) / rref - 1)) <= (K / 64 + 16) * 2.0 ** -24
    oq, os_ = quant.quantize_act_1x128(yb)                    # codes of the GPU's own y
    oqt, ost = quant.transpose_quantize_128x1(yb)
    assert_bytes_equal(host(xq), oq, "xq")
    assert_bytes_equal(host(xs), os_, "xs")
    assert_bytes_equal(host(xq_t), oqt, "xq_t")
    assert_bytes_equal(host(xs_t), ost, "xs_t")


@pytest.mark.parametrize("M,N", [(5, 264), (200, 136)])
def test_swiglu_partial_group(M, N):
    note(f"swiglu_quantize partial group M={M} N={N}")
    gt = _np_bf16(M, N, seed=3 * M + N, std=2.0, outliers=0.0)
    up = _np_bf16(M, N, seed=3 * M + N + 1, outliers=0.0)
    hq, hs, hq_t, hs_t, h = fq.swiglu_quantize_1x128(dev_bf16(gt), dev_bf16(up), True, True)
    torch.cuda.synchronize()
    hb = host_bits(h)
    href = fused.swiglu_bf16(gt, up)
    ulp = np.maximum(fused.bf16_ulp(href), fused.bf16_ulp(hb))
    assert np.all(np.abs(gemm.bf16_bits_to_f64(hb) - gemm.bf16_bits_to_f64(href)) <= ulp)
    oq, os_ = quant.quantize_act_1x128(hb)
    oqt, ost = quant.transpose_quantize_128x1(hb)
    assert_bytes_equal(host(hq), oq, "hq")
    assert_bytes_equal(host(hs), os_, "hs")
    assert_bytes_equal(host(hq_t), oqt, "hq_t")
    assert_bytes_equal(host(hs_t), ost, "hs_t")


# Shapes: small-tile and clamped configurations, and (last) one large enough
# for the 256 x 256 tiles, whose last tile along N / K holds the masked columns.
GEMM_SHAPES = [(1, 8, 8), (17, 136, 200), (300, 264, 1032), (64, 1000, 520), (4096, 4104, 520)]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_fwd_dgrad_partial_groups(M, N, K):
    note(f"fwd/dgrad partial groups M={M} N={N} K={K}")
    g1, g2, g3 = inputs.tensor_streams(M + N + K, 3)
    x = inputs.bf16_normal(g1, (M, K), 1.0, 0.01)
    w = inputs.bf16_normal(g2, (N, K), 0.02)
    dy = inputs.bf16_normal(g3, (M, N), 1e-3)
    xq, xs = quant.quantize_act_1x128(x)
    wq, ws, wq_t = quant.quantize_weight_128x128(w)
    dyq, dys = quant.quantize_act_1x128(dy)
    y = fq.fp8_gemm_fwd(dev_u8(xq), dev_f32(xs), dev_u8(wq), dev_f32(ws), n=N)
    dx = fq.fp8_gemm_dgrad(dev_u8(dyq), dev_f32(dys), dev_u8(wq_t), dev_f32(ws), k=K)
    torch.cuda.synchronize()
    assert y.shape == (M, N) and dx.shape == (M, K)
    _assert_close(host_bits(y), gemm.gemm_fwd(xq, xs, wq, ws, n=N), "fwd")
    _assert_close(host_bits(dx), gemm.gemm_dgrad(dyq, dys, wq, ws, k=K), "dgrad")


@pytest.mark.parametrize("M,N,K", [(128, 8, 8), (300, 136, 200), (256, 1000, 264), (1024, 4104, 520)])
def test_wgrad_partial_output(M, N, K):
    note(f"wgrad with N={N} K={K} (M={M})")
    g1, g2 = inputs.tensor_streams(3 * M + N + K, 2)
    x = inputs.bf16_normal(g1, (M, K), 1.0, 0.01)
    dy = inputs.bf16_normal(g2, (M, N), 1.0, 0.01)
    xq_t, xs_t = quant.transpose_quantize_128x1(x)
    dyq_t, dys_t = quant.transpose_quantize_128x1(dy)
    dw = fq.fp8_gemm_wgrad(dev_u8(dyq_t), dev_f32(dys_t), dev_u8(xq_t), dev_f32(xs_t))
    torch.cuda.synchronize()
    assert dw.shape == (N, K)
    _assert_close(host_bits(dw), gemm.gemm_wgrad(dyq_t, dys_t, xq_t, xs_t), "wgrad")


def test_grouped_with_partial_groups_equals_plain():
    note("grouped fwd / dgrad with partial-group problems vs the plain calls")
    shapes = [(256, 136, 200), (300, 264, 1032), (4096, 4104, 520)]
    fwd_p, dg_p = [], []
    for i, (M, N, K) in enumerate(shapes):
        x = inputs.bf16_normal_device((M, K), 1.0, 0.01, seed=90 + i)
        w = inputs.bf16_normal_device((N, K), 0.02, 0.0, seed=95 + i)
        dy = inputs.bf16_normal_device((M, N), 1e-3, 0.0, seed=99 + i)
        xq, xs = fq.quantize_act_1x128(x)
        wq, ws, wq_t = fq.quantize_weight_128x128(w)
        dyq, dys = fq.quantize_act_1x128(dy)
        fwd_p.append((xq, xs, wq, ws, N))
        dg_p.append((dyq, dys, wq_t, ws, K))
    fo = fq.fp8_gemm_fwd_grouped(fwd_p)
    do = fq.fp8_gemm_dgrad_grouped(dg_p)
    fr = [fq.fp8_gemm_fwd(*p[:4], n=p[4]) for p in fwd_p]
    dr = [fq.fp8_gemm_dgrad(*p[:4], k=p[4]) for p in dg_p]
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        assert torch.equal(fo[i], fr[i]), f"fwd problem {i}"
        assert torch.equal(do[i], dr[i]), f"dgrad problem {i}"


def test_fp8linear_partial_features():
    M, K, N = 300, 200, 136
    note(f"FP8Linear training with in_features={K}, out_features={N}, M={M}")
    w = inputs.bf16_normal_device((N, K), 0.02, 0.0, seed=61)
    lin = FP8Linear(K, N, weight=w)
    x = inputs.bf16_normal_device((M, K), 1.0, 0.01, seed=62).requires_grad_(True)
    dy = inputs.bf16_normal_device((M, N), 1e-3, 0.0, seed=63)
    y = lin(x)
    y.backward(dy)
    with torch.no_grad():
        y_inf = lin(x.detach())
    torch.cuda.synchronize()
    assert y.shape == (M, N) and x.grad.shape == (M, K) and lin.weight.grad.shape == (N, K)
    assert torch.equal(y, y_inf)
    xb, wb, db = host_bits(x.detach()), host_bits(lin.weight.detach()), host_bits(dy)
    oxq, oxs = quant.quantize_act_1x128(xb)
    owq, ows, _ = quant.quantize_weight_128x128(wb)
    odq, ods = quant.quantize_act_1x128(db)
    _assert_close(host_bits(y), gemm.gemm_fwd(oxq, oxs, owq, ows, n=N), "fwd")
    _assert_close(host_bits(x.grad), gemm.gemm_dgrad(odq, ods, owq, ows, k=K), "dgrad")
    o1, s1 = quant.transpose_quantize_128x1(db)
    o2, s2 = quant.transpose_quantize_128x1(xb)
    _assert_close(host_bits(lin.weight.grad), gemm.gemm_wgrad(o1, s1, o2, s2), "wgrad")
