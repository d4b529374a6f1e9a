"""GPU parity of the three quantizers and the E4M3 encoder: bit-exact against the oracle.

Calls go through the C ABI (via the Python binding). Inputs are seeded; the
oracle sees the same bf16 bytes as the GPU.
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_quantize_amd as fq
from fp8_block_scaled_quantize_amd import inputs
from oracle import e4m3, quant
from tests._gpu import assert_bytes_equal, dev_bf16, dev_f32, host, host_bits, note, requires_gpu, sample_indices

pytestmark = [pytest.mark.gpu, requires_gpu]


def _np_bf16(rows, cols, seed, std=1.0, outliers=0.01):
    (g,) = inputs.tensor_streams(seed, 1)
    return inputs.bf16_normal(g, (rows, cols), std, outliers)


# ------------------------------------------------------------------ 1x128 --

@pytest.mark.parametrize("shape", [(1, 128), (3, 384), (130, 256), (128, 256), (64, 4096), (257, 1280)])
def test_act_matches_oracle(shape):
    note(f"act_1x128 {shape}")
    x = _np_bf16(*shape, seed=sum(shape))
    xq, xs = fq.quantize_act_1x128(dev_bf16(x))
    torch.cuda.synchronize()
    oq, os_ = quant.quantize_act_1x128(x)
    assert_bytes_equal(host(xq), oq, "xq", x)
    assert_bytes_equal(host(xs), os_, "xs")


def test_act_every_bf16_amax_and_edge_groups():
    note("act_1x128 every positive bf16 amax + tiny/zero/-0 groups")
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    G = np.zeros((bits.size, 128), dtype=np.uint16)
    G[:, 0] = bits
    G[:, 77] = bits | 0x8000
    rng = np.random.default_rng(3)
    # other entries: random bf16 values at or below the group's amax
    frac = rng.random((bits.size, 126)).astype(np.float32)
    amax = e4m3.bf16_bits_to_f32(bits)
    vals = inputs.f32_to_bf16_bits(frac * amax[:, None] * np.where(rng.random((bits.size, 126)) < 0.5, -1, 1).astype(np.float32))
    keep = np.abs(e4m3.bf16_bits_to_f32(vals)) <= amax[:, None]
    vals = np.where(keep, vals, 0).astype(np.uint16)
    G[:, 1:77] = vals[:, :76]
    G[:, 78:] = vals[:, 76:]
    extra = np.zeros((4, 128), dtype=np.uint16)
    extra[1, 5] = 0x8000                       # a -0.0 in a zero group
    extra[2, :] = 0x0001                       # smallest subnormal everywhere
    extra[3, ::2] = 0x8001
    X = np.concatenate([G, extra])
    xq, xs = fq.quantize_act_1x128(dev_bf16(X))
    torch.cuda.synchronize()
    oq, os_ = quant.quantize_act_1x128(X)
    assert_bytes_equal(host(xs), os_, "xs")
    assert_bytes_equal(host(xq), oq, "xq", X)


def test_act_full_size_sampled_rows():
    M, K = 16384, 14336
    note(f"act_1x128 full size [{M},{K}] sampled rows")
    x = inputs.bf16_normal_device((M, K), 1.0, 0.01, seed=7)
    xq, xs = fq.quantize_act_1x128(x)
    torch.cuda.synchronize()
    rows = sample_indices(M, 96, seed=1)
    xb = host_bits(x[rows])
    oq, os_ = quant.quantize_act_1x128(xb)
    assert np.array_equal(host(xq[rows]), oq)
    assert np.array_equal(host(xs[rows]), os_)


def test_act_scale_range_sweep():
    note("act_1x128 groups scaled by 2^e, e in [-140, 120]")
    base = _np_bf16(261, 128, seed=9, outliers=0.0)
    f = e4m3.bf16_bits_to_f32(base)
    e = np.arange(-140, 121, dtype=np.float64)
    X = inputs.f32_to_bf16_bits((f.astype(np.float64) * np.exp2(e)[:, None]).astype(np.float32))
    xq, xs = fq.quantize_act_1x128(dev_bf16(X))
    torch.cuda.synchronize()
    oq, os_ = quant.quantize_act_1x128(X)
    assert_bytes_equal(host(xs), os_, "xs")
    assert_bytes_equal(host(xq), oq, "xq", X)


# ---------------------------------------------------------------- 128x128 --

@pytest.mark.parametrize("shape", [(128, 128), (256, 256), (384, 640), (1024, 512)])
def test_weight_matches_oracle(shape):
    note(f"weight_128x128 {shape}")
    (g,) = inputs.tensor_streams(sum(shape), 1)
    w = inputs.bf16_normal(g, shape, 0.02)
    wq, ws, wq_t = fq.quantize_weight_128x128(dev_bf16(w))
    torch.cuda.synchronize()
    oq, os_, ot = quant.quantize_weight_128x128(w)
    assert np.array_equal(host(wq), oq)
    assert np.array_equal(host(ws), os_)
    assert np.array_equal(host(wq_t), ot)


def test_weight_without_transpose_and_full_size():
    N, K = 28672, 4096
    note(f"weight_128x128 full size [{N},{K}] sampled bands")
    w = inputs.bf16_normal_device((N, K), 0.02, 0.0, seed=11)
    wq, ws, wq_t = fq.quantize_weight_128x128(w)
    wq2, ws2, none = fq.quantize_weight_128x128(w, transposed=False)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(wq, wq2) and torch.equal(ws, ws2)
    assert torch.equal(wq_t, wq.t().contiguous())
    for band in (0, 97, N // 128 - 1):
        rows = slice(128 * band, 128 * band + 128)
        oq, os_, _ = quant.quantize_weight_128x128(host_bits(w[rows]))
        assert np.array_equal(host(wq[rows]), oq)
        assert np.array_equal(host(ws[band:band + 1]), os_)


# ------------------------------------------------------------------ 128x1 --

@pytest.mark.parametrize("shape", [(128, 128), (256, 384), (384, 256), (512, 1152)])
def test_transpose_matches_oracle(shape):
    note(f"transpose_128x1 {shape}")
    x = _np_bf16(*shape, seed=3 * sum(shape))
    qt, st = fq.transpose_quantize_128x1(dev_bf16(x))
    torch.cuda.synchronize()
    oq, os_ = quant.transpose_quantize_128x1(x)
    assert np.array_equal(host(st), os_)
    assert np.array_equal(host(qt), oq)


def test_transpose_full_size_sampled_and_identity():
    M, C = 32768, 27648
    note(f"transpose_128x1 full size [{M},{C}] sampled channels")
    x = inputs.bf16_normal_device((M, C), 1.0, 0.01, seed=13)
    qt, st = fq.transpose_quantize_128x1(x)
    torch.cuda.synchronize()
    cols = sample_indices(C, 48, seed=2)
    oq, os_ = quant.transpose_quantize_128x1(host_bits(x[:, cols]))
    assert np.array_equal(host(qt[cols]), oq)
    assert np.array_equal(host(st[cols]), os_)
    note("transpose_128x1 == act_1x128 of the transpose (GPU vs GPU, [4096, 5120])")
    y = x[:4096, :5120].contiguous()
    qt2, st2 = fq.transpose_quantize_128x1(y)
    q1, s1 = fq.quantize_act_1x128(y.t().contiguous())
    torch.cuda.synchronize()
    assert torch.equal(qt2, q1) and torch.equal(st2, s1)


@pytest.mark.parametrize("M", [1, 100, 300, 1000])
def test_transpose_ragged_token_count(M):
    note(f"transpose_128x1 ragged M={M}")
    x = _np_bf16(M, 384, seed=7 * M)
    qt, st = fq.transpose_quantize_128x1(dev_bf16(x))
    torch.cuda.synchronize()
    oq, os_ = quant.transpose_quantize_128x1(x)
    assert np.array_equal(host(st), os_)
    assert np.array_equal(host(qt), oq)


# ------------------------------------------------------------ dual output --

@pytest.mark.parametrize("shape", [(128, 128), (256, 384), (384, 640), (512, 1152)])
def test_dual_matches_oracle(shape):
    note(f"dual 1x128 + 128x1 {shape}")
    x = _np_bf16(*shape, seed=5 * sum(shape))
    xq, xs, qt, st = fq.quantize_dual_1x128_128x1(dev_bf16(x))
    torch.cuda.synchronize()
    oq, os_ = quant.quantize_act_1x128(x)
    oqt, ost = quant.transpose_quantize_128x1(x)
    assert_bytes_equal(host(xq), oq, "xq", x)
    assert_bytes_equal(host(xs), os_, "xs")
    assert np.array_equal(host(qt), oqt)
    assert np.array_equal(host(st), ost)


@pytest.mark.parametrize("M", [77, 300])
def test_dual_ragged_token_count(M):
    note(f"dual ragged M={M}")
    x = _np_bf16(M, 640, seed=11 * M)
    xq, xs, qt, st = fq.quantize_dual_1x128_128x1(dev_bf16(x))
    torch.cuda.synchronize()
    oq, os_ = quant.quantize_act_1x128(x)
    oqt, ost = quant.transpose_quantize_128x1(x)
    assert_bytes_equal(host(xq), oq, "xq", x)
    assert_bytes_equal(host(xs), os_, "xs")
    assert np.array_equal(host(qt), oqt)
    assert np.array_equal(host(st), ost)


def test_dual_edge_groups():
    note("dual: zero, -0, subnormal, tiny and bf16-max groups along both groupings")
    x = _np_bf16(256, 384, seed=41)
    x[0, :] = 0                                   # an all-zero row
    x[1, :] = 0x8000                              # an all -0.0 row
    x[2, :] = 0x0001                              # smallest subnormal everywhere
    x[3, ::3] = 0x8001
    x[4:20, :] = inputs.f32_to_bf16_bits(                 # amax far below 2^-64
        e4m3.bf16_bits_to_f32(x[4:20, :]) * np.float32(2.0 ** -100))
    x[:, 5] = 0x7F7F                              # largest finite bf16 in one channel
    x[128:, 130] = 0                              # a zero 128x1 group
    x[128:, 131] = 0x8000                         # a -0.0 128x1 group
    xq, xs, qt, st = fq.quantize_dual_1x128_128x1(dev_bf16(x))
    torch.cuda.synchronize()
    oq, os_ = quant.quantize_act_1x128(x)
    oqt, ost = quant.transpose_quantize_128x1(x)
    assert_bytes_equal(host(xs), os_, "xs")
    assert_bytes_equal(host(xq), oq, "xq", x)
    assert np.array_equal(host(st), ost)
    assert np.array_equal(host(qt), oqt)


@pytest.mark.parametrize("shape", [(4224, 1152), (4200, 1144)])
def test_dual_and_transpose_every_byte_past_256_workgroups(shape):
    # 33 token blocks x 9 channel blocks = 297 workgroups: the first 256 are
    # renumbered so each XCD takes 32 consecutive token blocks, the last 41
    # keep their order; the second shape is ragged in both dimensions (the
    # TAIL instantiation). Every code and scale byte is compared.
    M, C = shape
    note(f"dual and transpose_128x1, every byte, {M}x{C}")
    x = _np_bf16(M, C, seed=M + C)
    xd = dev_bf16(x)
    xq, xs, qt, st = fq.quantize_dual_1x128_128x1(xd)
    qt2, st2 = fq.transpose_quantize_128x1(xd)
    torch.cuda.synchronize()
    oq, os_ = quant.quantize_act_1x128(x)
    oqt, ost = quant.transpose_quantize_128x1(x)
    assert_bytes_equal(host(xq), oq, "dual xq")
    assert_bytes_equal(host(xs), os_, "dual xs")
    assert_bytes_equal(host(qt), oqt, "dual xq_t")
    assert_bytes_equal(host(st), ost, "dual xs_t")
    assert_bytes_equal(host(qt2), oqt, "transpose xq_t")
    assert_bytes_equal(host(st2), ost, "transpose xs_t")


def test_dual_full_size_equals_single_output_kernels():
    M, C = 32768, 27648
    note(f"dual full size [{M},{C}] vs the single-output kernels (all bytes) and the oracle (sampled)")
    x = inputs.bf16_normal_device((M, C), 1.0, 0.01, seed=23)
    xq, xs, qt, st = fq.quantize_dual_1x128_128x1(x)
    q1, s1 = fq.quantize_act_1x128(x)
    q2, s2 = fq.transpose_quantize_128x1(x)
    torch.cuda.synchronize()
    assert torch.equal(xq, q1) and torch.equal(xs, s1)
    assert torch.equal(qt, q2) and torch.equal(st, s2)
    rows = sample_indices(M, 24, seed=3)
    oq, os_ = quant.quantize_act_1x128(host_bits(x[rows]))
    assert np.array_equal(host(xq[rows]), oq) and np.array_equal(host(xs[rows]), os_)
    cols = sample_indices(C, 24, seed=4)
    oqt, ost = quant.transpose_quantize_128x1(host_bits(x[:, cols]))
    assert np.array_equal(host(qt[cols]), oqt) and np.array_equal(host(st[cols]), ost)


# ------------------------------------------------- grid-limit launch split --

def test_launch_split_beyond_grid_y_limit():
    # 65536 channel (or row) blocks: one more than a launch's y extent, so the
    # launchers issue a second launch with a block offset.
    C = 65536 * 128
    note(f"transpose / dual / weight quantizers past the grid limit: [128, {C}] and [{C}, 128]")
    x = inputs.bf16_normal_device((128, C), 1.0, 0.01, seed=29)
    cols = np.unique(np.concatenate([sample_indices(C, 24, seed=5), np.arange(C - 130, C)]))
    qt, st = fq.transpose_quantize_128x1(x)
    torch.cuda.synchronize()
    oqt, ost = quant.transpose_quantize_128x1(host_bits(x[:, cols]))
    assert np.array_equal(host(qt[cols]), oqt) and np.array_equal(host(st[cols]), ost)
    del qt, st
    xq, xs, qt, st = fq.quantize_dual_1x128_128x1(x)
    torch.cuda.synchronize()
    assert np.array_equal(host(qt[cols]), oqt) and np.array_equal(host(st[cols]), ost)
    band = slice(C - 128 * 3, C)
    oq, os_ = quant.quantize_act_1x128(host_bits(x[:, band]))
    assert np.array_equal(host(xq[:, band]), oq)
    assert np.array_equal(host(xs[:, (C - 384) // 128:]), os_)
    del xq, xs, qt, st
    w = x.t().contiguous()
    del x
    wq, ws, wq_t = fq.quantize_weight_128x128(w)
    torch.cuda.synchronize()
    for rb in (0, 31337, 65535):
        rows = slice(128 * rb, 128 * rb + 128)
        owq, ows, owq_t = quant.quantize_weight_128x128(host_bits(w[rows]))
        assert np.array_equal(host(wq[rows]), owq)
        assert np.array_equal(host(ws[rb:rb + 1]), ows)
        assert np.array_equal(host(wq_t[:, rows]), owq_t)


# ------------------------------------------------------------------ codec --

def test_cast_sweep_matches_oracle():
    note("cast_f32_e4m3 structured float32 sweep")
    hi = np.arange(0, 0x43E81, dtype=np.uint32) << 12
    lows = np.array([0x000, 0x001, 0x7FF, 0x800, 0x801, 0xFFF], dtype=np.uint32)
    bits = (hi[:, None] | lows[None, :]).ravel()
    v = bits.view(np.float32)
    v = v[np.abs(v) <= 464]
    v = np.concatenate([v, -v, np.zeros((-2 * v.size) % 4, np.float32)])
    out = fq.cast_f32_e4m3(dev_f32(v))
    torch.cuda.synchronize()
    assert_bytes_equal(host(out), e4m3.encode(v), "cast")


def test_determinism():
    note("quantizers: repeated calls give identical bytes")
    x = inputs.bf16_normal_device((4096, 5120), 1.0, 0.01, seed=17)
    a = fq.quantize_act_1x128(x)
    b = fq.quantize_act_1x128(x)
    c = fq.transpose_quantize_128x1(x)
    d = fq.transpose_quantize_128x1(x)
    e = fq.quantize_weight_128x128(x)
    f = fq.quantize_weight_128x128(x)
    g = fq.quantize_dual_1x128_128x1(x)
    h = fq.quantize_dual_1x128_128x1(x)
    torch.cuda.synchronize()
    for u, w in ((a, b), (c, d), (e, f), (g, h)):
        for s, t in zip(u, w):
            assert torch.equal(s, t)
