"""GPU parity of the weight-streaming forward (decode, at most 64 token rows).

* the stream layout is a permutation of the row-major codes: checked element
  by element against the layout's definition (tests/_layout.py, pinned by
  tests/test_stream_order.py) on codes the oracle made, both for the conversion (fp8_weight_stream_layout) and for the
  quantizer that writes the layout itself (quantize_weight_128x128_stream,
  whose scales must also equal the oracle's);
* fp8_gemm_fwd_stream gives the bytes of fp8_gemm_fwd for every token count
  1..64 tried, on shapes that run each workgroup width (1..7 weight
  fragments), K lengths that run the ring's main loop, its tail or both, and
  ragged N / K;
* decode-sized linears at full size (the benchmark's gate/up workload and
  narrower weights that run the multi-chunk token ring), quantized and
  multiplied as the benchmark runs them, on one output in every 16 x 64 band
  against the oracle.
Calls go through the C ABI (via the Python binding).
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_quantize_amd as fq
from fp8_block_scaled_quantize_amd import inputs
from oracle import gemm, quant
from tests._gpu import (assert_bytes_equal, dev_bf16, dev_u8, host, host_bits, note, one_per_tile,
                        oracle_weight, requires_gpu)
from tests._layout import stream_order

pytestmark = [pytest.mark.gpu, requires_gpu]


@pytest.mark.parametrize("N,K", [(128, 128), (256, 384), (136, 200), (1000, 1000), (8, 8)])
def test_stream_layout_of_oracle_codes(N, K):
    note(f"stream layout N={N} K={K}")
    (gw,) = inputs.tensor_streams(N * 7 + K, 1)
    w = inputs.bf16_normal(gw, (N, K), 0.02)
    owq, ows, _ = quant.quantize_weight_128x128(w)
    want = stream_order(owq)
    conv = fq.weight_stream_layout(dev_u8(owq))
    wq_s, ws = fq.quantize_weight_128x128_stream(dev_bf16(w))
    torch.cuda.synchronize()
    assert_bytes_equal(host(conv), want, "fp8_weight_stream_layout")
    assert_bytes_equal(host(wq_s), want, "quantize_weight_128x128_stream codes")
    assert_bytes_equal(host(ws).view(np.uint32), ows.view(np.uint32), "quantize_weight_128x128_stream scales")


# (N, K): the workgroup width the launch picks for N (weight fragments per
# workgroup, 1..7) and the K blocks Kb, against the weight ring (12 blocks
# for wide weights and for one token block, else 8: Kb below it runs the
# ring's tail only, a multiple of it the main loop only) and the token ring
# (4-block chunks, up to 6 in flight: Kb below 24 ends inside the first
# chunks in flight).
SHAPES = [
    (8, 8),            # width 1, Kb 1, everything ragged
    (128, 128),        # width 1, Kb 1
    (1000, 1000),      # width 1, Kb 8, ragged
    (384, 1152),       # width 1, Kb 9
    (2048, 1536),      # width 1, Kb 12
    (5120, 5120),      # width 2, Kb 40
    (12288, 1024),     # width 3, Kb 8
    (14336, 4096),     # width 4, Kb 32
    (20480, 256),      # width 5, Kb 2
    (24576, 384),      # width 6, Kb 3
    (28672, 4096),     # width 7, Kb 32
]


@pytest.mark.parametrize("N,K", SHAPES)
def test_stream_fwd_equals_tile_fwd(N, K):
    # every token-block count (1-4 blocks of 16) on every shape
    tokens = (1, 5, 16, 17, 33, 48, 64) if N * K <= 1 << 24 else (1, 17, 40, 64)
    note(f"stream fwd vs fp8_gemm_fwd N={N} K={K} tokens {tokens}")
    x = inputs.bf16_normal_device((64, K), 1.0, 0.01, seed=N + K)
    w = inputs.bf16_normal_device((N, K), 0.02, 0.0, seed=N + 2 * K)
    xq, xs = fq.quantize_act_1x128(x)
    wq, ws, _ = fq.quantize_weight_128x128(w, transposed=False)
    wq_s, ws_s = fq.quantize_weight_128x128_stream(w)
    full = fq.fp8_gemm_fwd_stream(xq, xs, wq_s, ws_s, n=N)
    for M in tokens:
        a, a_s = xq[:M].contiguous(), xs[:M].contiguous()
        y_tile = fq.fp8_gemm_fwd(a, a_s, wq, ws, n=N)
        y_stream = fq.fp8_gemm_fwd_stream(a, a_s, wq_s, ws_s, n=N)
        torch.cuda.synchronize()
        assert torch.equal(y_stream, y_tile), f"N={N} K={K} M={M}: stream and tile forwards differ"
        assert torch.equal(y_stream, full[:M]), f"N={N} K={K} M={M}: rows differ from the 64-row call"
    assert torch.equal(ws_s, ws)


# Decode-sized linears at full size: the benchmark's gate/up workload (7
# fragments per workgroup, one token chunk in flight), the 8B down projection
# (one fragment per workgroup, 3 staging wavefronts, 28 chunks), the 32B o
# projection (2 fragments per workgroup, 10 chunks) and the 8B qkv
# projection at 40 tokens (3 token blocks, 2 staging wavefronts).
DECODE_LINEARS = [
    ("gate_up", 64, 28672, 4096),
    ("down_8b", 64, 4096, 14336),
    ("o_32b", 64, 5120, 5120),
    ("qkv_8b", 40, 6144, 4096),
]


@pytest.mark.parametrize("name,M,N,K", DECODE_LINEARS)
def test_decode_linear_full_size(name, M, N, K):
    """A rollout decode linear as the benchmark runs it: 1x128 activations, the
    weight quantized straight into the stream layout, the stream forward; one
    output in every 16-token x 64-channel band against the oracle."""
    lin = dict(inputs.WORKLOADS["llama31_8b_decode_gate_up_m64"]["linears"][0], name=name, M=M, N=N, K=K)
    note(f"decode stream fwd {name} M={M} N={N} K={K}")
    t = inputs.linear_tensors_device(lin, seed=1000)
    x, w = t["x"], t["w"]
    xq, xs = fq.quantize_act_1x128(x)
    wq_s, ws = fq.quantize_weight_128x128_stream(w)
    y = fq.fp8_gemm_fwd_stream(xq, xs, wq_s, ws)
    torch.cuda.synchronize()
    owq, ows = oracle_weight(w)
    assert_bytes_equal(host(ws).view(np.uint32), ows.view(np.uint32), "weight scales")
    assert_bytes_equal(host(wq_s), stream_order(owq), "weight codes (stream layout)")
    rows = one_per_tile(M, 7, band=16)
    cols = one_per_tile(N, 8, band=64)
    oxq, oxs = quant.quantize_act_1x128(host_bits(x[rows]))
    ref = gemm.dequant_rows(oxq, oxs) @ gemm.dequant_rows(owq[cols], ows[cols // 128]).T
    ok, info = gemm.within_tolerance(host_bits(y[rows][:, cols]), ref)
    assert ok, f"decode stream fwd {name}, {len(rows)} x {len(cols)} outputs: {info}"


def _random_shapes(n, seed):
    """n seeded (M, N, K): M in 1..64, N and K multiples of 8 up to 2048, ragged or not."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.integers(1, 65))
        N = 8 * int(rng.integers(1, 257))
        K = 8 * int(rng.integers(1, 257))
        out.append((M, N, K))
    return out


@pytest.mark.parametrize("M,N,K", _random_shapes(24, 2027))
def test_stream_random_shapes(M, N, K):
    note(f"stream path on a random shape M={M} N={N} K={K}")
    x = inputs.bf16_normal_device((M, K), 1.0, 0.01, seed=M * 7 + N + K)
    w = inputs.bf16_normal_device((N, K), 0.02, 0.0, seed=M + N * 3 + K)
    xq, xs = fq.quantize_act_1x128(x)
    wq, ws, _ = fq.quantize_weight_128x128(w, transposed=False)
    wq_s, ws_s = fq.quantize_weight_128x128_stream(w)
    conv = fq.weight_stream_layout(wq)
    y_tile = fq.fp8_gemm_fwd(xq, xs, wq, ws, n=N)
    y_stream = fq.fp8_gemm_fwd_stream(xq, xs, wq_s, ws_s, n=N)
    torch.cuda.synchronize()
    assert torch.equal(wq_s, conv), "stream quantizer codes differ from the converted row-major codes"
    assert torch.equal(ws_s, ws)
    assert torch.equal(y_stream, y_tile), "stream and tile forwards differ"
    if N * K <= 1 << 20:
        owq, ows, _ = quant.quantize_weight_128x128(host_bits(w))
        assert_bytes_equal(host(wq_s), stream_order(owq), "stream codes vs the oracle")
        oxq, oxs = quant.quantize_act_1x128(host_bits(x))
        ok, info = gemm.within_tolerance(host_bits(y_stream), gemm.gemm_fwd(oxq, oxs, owq, ows, n=N))
        assert ok, info
