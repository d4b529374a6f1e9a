"""FP8Linear (the autograd op over the C ABI): rollout/training consistency,
batch invariance, and the backward against direct calls and the oracle."""

import numpy as np
import pytest
import torch

import fp8_block_scaled_quantize_amd as fq
from fp8_block_scaled_quantize_amd import inputs
from fp8_block_scaled_quantize_amd.linear import FP8Linear
from oracle import gemm, quant
from tests._gpu import host_bits, note, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def _layer(K, N, seed):
    w = inputs.bf16_normal_device((N, K), 0.02, 0.0, seed=seed)
    return FP8Linear(K, N, weight=w)


def test_forward_equals_the_abi_calls_and_inference_equals_training():
    M, K, N = 512, 640, 384
    note(f"FP8Linear forward M={M} K={K} N={N}")
    lin = _layer(K, N, seed=51)
    x = inputs.bf16_normal_device((M, K), 1.0, 0.01, seed=52)
    y_train = lin(x)
    with torch.no_grad():
        y_infer = lin(x)
    xq, xs = fq.quantize_act_1x128(x)
    wq, ws, _ = fq.quantize_weight_128x128(lin.weight.detach(), transposed=False)
    y_abi = fq.fp8_gemm_fwd(xq, xs, wq, ws)
    torch.cuda.synchronize()
    assert torch.equal(y_train, y_abi)
    assert torch.equal(y_infer, y_train)          # one quantization flow for rollout and training


@pytest.mark.parametrize("big", [256, 4096])
def test_batch_invariance(big):
    K, N = 4096, 4096
    note(f"FP8Linear batch invariance: rows of a {big}-token batch vs alone (64 tokens) and permuted")
    lin = _layer(K, N, seed=53)
    x = inputs.bf16_normal_device((big, K), 1.0, 0.01, seed=54)
    with torch.no_grad():
        y_big = lin(x)
        y_small = lin(x[:64].contiguous())
        perm = torch.randperm(big, generator=torch.Generator().manual_seed(5)).cuda()
        y_perm = lin(x[perm].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(y_small, y_big[:64])
    assert torch.equal(y_perm, y_big[perm])


def test_backward_equals_the_abi_calls_and_the_oracle():
    M, K, N = 384, 512, 256
    note(f"FP8Linear backward M={M} K={K} N={N}")
    lin = _layer(K, N, seed=55)
    x = inputs.bf16_normal_device((M, K), 1.0, 0.01, seed=56).requires_grad_(True)
    dy = inputs.bf16_normal_device((M, N), 1e-3, 0.0, seed=57)
    y = lin(x)
    y.backward(dy)
    torch.cuda.synchronize()
    w = lin.weight.detach()
    dyq, dys, dyq_t, dys_t = fq.quantize_dual_1x128_128x1(dy)
    _, xs_unused, xq_t, xs_t = fq.quantize_dual_1x128_128x1(x.detach())
    wq, ws, wq_t = fq.quantize_weight_128x128(w)
    dx = fq.fp8_gemm_dgrad(dyq, dys, wq_t, ws)
    dw = fq.fp8_gemm_wgrad(dyq_t, dys_t, xq_t, xs_t)
    torch.cuda.synchronize()
    assert torch.equal(x.grad, dx)
    assert torch.equal(lin.weight.grad, dw)
    xb, wb, db = host_bits(x.detach()), host_bits(w), host_bits(dy)
    oq, os_ = quant.quantize_act_1x128(db)
    owq, ows, _ = quant.quantize_weight_128x128(wb)
    ok, info = gemm.within_tolerance(host_bits(x.grad), gemm.gemm_dgrad(oq, os_, owq, ows))
    assert ok, info
    o1, s1 = quant.transpose_quantize_128x1(db)
    o2, s2 = quant.transpose_quantize_128x1(xb)
    ok, info = gemm.within_tolerance(host_bits(lin.weight.grad), gemm.gemm_wgrad(o1, s1, o2, s2))
    assert ok, info


def test_weight_update_requantizes():
    M, K, N = 128, 256, 256
    note("FP8Linear: an in-place weight update invalidates the cached codes")
    lin = _layer(K, N, seed=58)
    x = inputs.bf16_normal_device((M, K), 1.0, 0.0, seed=59)
    with torch.no_grad():
        y0 = lin(x)
        lin.weight.mul_(2.0)                      # exact: every scale doubles, codes unchanged
        y1 = lin(x)
    torch.cuda.synchronize()
    assert torch.equal(y1.float(), 2.0 * y0.float())


def test_training_with_a_ragged_token_count():
    M, K, N = 300, 256, 384
    note(f"FP8Linear training with M={M} tokens (transposed copies padded to 384)")
    lin = _layer(K, N, seed=60)
    x = inputs.bf16_normal_device((M, K), 1.0, 0.0, seed=61).requires_grad_(True)
    dy = inputs.bf16_normal_device((M, N), 1e-3, 0.0, seed=62)
    y = lin(x)
    y.backward(dy)
    with torch.no_grad():
        y_inf = lin(x.detach())
    torch.cuda.synchronize()
    assert torch.equal(y, y_inf)
    xb, wb, db = host_bits(x.detach()), host_bits(lin.weight.detach()), host_bits(dy)
    oq, os_ = quant.quantize_act_1x128(db)
    owq, ows, _ = quant.quantize_weight_128x128(wb)
    ok, info = gemm.within_tolerance(host_bits(x.grad), gemm.gemm_dgrad(oq, os_, owq, ows))
    assert ok, info
    o1, s1 = quant.transpose_quantize_128x1(db)          # [N, 384], +0 past token 300
    o2, s2 = quant.transpose_quantize_128x1(xb)
    ok, info = gemm.within_tolerance(host_bits(lin.weight.grad), gemm.gemm_wgrad(o1, s1, o2, s2))
    assert ok, info


@pytest.mark.parametrize("tokens", [1, 17, 64])
def test_decode_inference_on_the_streaming_layout(tokens):
    """Rollout with at most 64 tokens runs the weight-streaming forward; its rows
    equal the training forward's, and after an in-place weight update it uses
    the new codes (the streaming copy is remade)."""
    K, N = 1024, 768
    note(f"FP8Linear decode inference, {tokens} tokens, on the streaming layout")
    lin = _layer(K, N, seed=63)
    x = inputs.bf16_normal_device((tokens, K), 1.0, 0.01, seed=64)
    y_train = lin(x.clone().requires_grad_(True))
    w2 = inputs.bf16_normal_device((N, K), 0.02, 0.0, seed=65)
    with torch.no_grad():
        y_dec = lin(x)
        assert lin._codes.wq_s is not None                  # the streaming path ran
        lin.weight.copy_(w2)                                # new codes and scales
        y_dec2 = lin(x)
    xq, xs = fq.quantize_act_1x128(x)
    wq, ws, _ = fq.quantize_weight_128x128(w2, transposed=False)
    y_abi2 = fq.fp8_gemm_fwd(xq, xs, wq, ws)
    torch.cuda.synchronize()
    assert torch.equal(y_dec, y_train.detach())
    assert torch.equal(y_dec2, y_abi2)
