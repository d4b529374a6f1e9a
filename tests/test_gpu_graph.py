"""The library's calls inside a captured HIP graph (torch.cuda.graph).

The entry points only enqueue kernels on the given stream (no allocation, no
memset, no synchronisation), so a sequence of them can be captured once and
replayed. Every replay is checked bit for bit against the eager results, with
unrelated eager work and synchronisations between the replays.
"""

import pytest
import torch

import fp8_block_scaled_quantize_amd as fq
from fp8_block_scaled_quantize_amd import inputs
from tests._gpu import note, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def _step(x, w, dy, out):
    """One linear layer's flow into preallocated outputs (the calls a graph records)."""
    fq.quantize_weight_128x128(w, True, out["wq"], out["ws"], out["wq_t"])
    fq.quantize_dual_1x128_128x1(x, out["xq"], out["xs"], out["xq_t"], out["xs_t"])
    fq.fp8_gemm_fwd(out["xq"], out["xs"], out["wq"], out["ws"], out=out["y"])
    fq.quantize_dual_1x128_128x1(dy, out["dyq"], out["dys"], out["dyq_t"], out["dys_t"])
    fq.fp8_gemm_dgrad(out["dyq"], out["dys"], out["wq_t"], out["ws"], out=out["dx"])
    fq.fp8_gemm_wgrad(out["dyq_t"], out["dys_t"], out["xq_t"], out["xs_t"], out=out["dw"])
    fq.quantize_act_1x128(x[:64], out["dq"], out["ds"])           # a decode-sized pair
    fq.fp8_gemm_fwd(out["dq"], out["ds"], out["wq"], out["ws"], out=out["dy64"])
    fq.quantize_weight_128x128_stream(w, out["wq_s"], out["ws_s"])  # the decode path on the stream layout
    fq.fp8_gemm_fwd_stream(out["dq"], out["ds"], out["wq_s"], out["ws_s"], out=out["ds64"])


def _buffers(M, N, K):
    e = lambda shape, dt: torch.empty(shape, dtype=dt, device="cuda")
    u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16
    return {"wq": e((N, K), u8), "ws": e((N // 128, K // 128), f32), "wq_t": e((K, N), u8),
            "xq": e((M, K), u8), "xs": e((M, K // 128), f32), "xq_t": e((K, M), u8), "xs_t": e((K, M // 128), f32),
            "dyq": e((M, N), u8), "dys": e((M, N // 128), f32), "dyq_t": e((N, M), u8),
            "dys_t": e((N, M // 128), f32), "y": e((M, N), bf), "dx": e((M, K), bf), "dw": e((N, K), bf),
            "dq": e((64, K), u8), "ds": e((64, K // 128), f32), "dy64": e((64, N), bf),
            "wq_s": e((N, K), u8), "ws_s": e((N // 128, K // 128), f32), "ds64": e((64, N), bf)}


def test_graph_replays_equal_eager():
    M, N, K = 1024, 768, 512
    note(f"graph capture of the linear-layer flow M={M} N={N} K={K}, 4 replays vs eager")
    x = inputs.bf16_normal_device((M, K), 1.0, 0.01, seed=81)
    w = inputs.bf16_normal_device((N, K), 0.02, 0.0, seed=82)
    dy = inputs.bf16_normal_device((M, N), 1e-3, 0.0, seed=83)
    eager = _buffers(M, N, K)
    _step(x, w, dy, eager)
    torch.cuda.synchronize()

    graphed = _buffers(M, N, K)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                  # warm-up on the capture stream, as torch advises
        _step(x, w, dy, graphed)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(x, w, dy, graphed)
    torch.cuda.synchronize()
    for rep in range(4):
        for t in graphed.values():                 # every output is rewritten by the replay
            t.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()   # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for name, ref in eager.items():
            assert torch.equal(graphed[name], ref), f"replay {rep}: {name} differs from the eager call"
    assert torch.equal(eager["ds64"], eager["dy64"])   # the stream forward equals the tile forward
