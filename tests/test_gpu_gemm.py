"""GPU parity of the three FP8 GEMMs against the fp64 oracle.

* exact operands (every group's amax is 448 * 2^e, so quantization is
  lossless and every partial sum is exact in fp32): with the narrow value set
  (0, +-112, +-224, +-448 times 2^e) the bf16 output must equal the oracle's
  bf16 rounding bit for bit. With the wide value set (multiples of 1/4 up to
  16, plus the +-448 amax) the FP8 MFMA itself is not exact (one 16x16x128
  fp8 MFMA deviates from the exact sum by a small fraction of its largest
  product; tests/test_gpu_mfma_exactness.py pins the bound), so that set is
  held to the bound that follows from it;
* oracle-quantized operands fed straight into the GEMMs at small, ragged
  shapes: within the tolerance |err| <= 2^-7 |ref| + 1e-3 rms(ref);
* every workload at full size, quantized and multiplied on the GPU in the
  launch configuration the benchmark uses, checked on sampled outputs that
  the oracle computes from the same bf16 inputs.
Calls go through the C ABI (via the Python binding).
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_quantize_amd as fq
from fp8_block_scaled_quantize_amd import inputs
from oracle import gemm, quant
from tests._gpu import dev_bf16, dev_f32, dev_u8, host_bits, note, one_per_tile, oracle_weight, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def _assert_close(out_bits, ref, what):
    ok, info = gemm.within_tolerance(out_bits, ref)
    assert ok, f"{what}: {info}"


def _assert_bits_equal(out_bits, want_bits, ref, what):
    """Bit-exact bf16 comparison with a report of the first differences."""
    bad = np.argwhere(out_bits != want_bits)
    if bad.size:
        got = gemm.bf16_bits_to_f64(out_bits)
        lines = [f"{what}: {len(bad)} of {out_bits.size} outputs differ"]
        for i, j in bad[:8]:
            lines.append(f"  [{i},{j}] gpu={got[i, j]!r} ref={ref[i, j]!r} "
                         f"bits gpu={out_bits[i, j]:04x} want={want_bits[i, j]:04x}")
        rel = np.abs(got - ref)[out_bits != want_bits] / np.maximum(np.abs(ref[out_bits != want_bits]), 1e-300)
        lines.append(f"  max rel diff {rel.max():.3e}")
        raise AssertionError("\n".join(lines))


# ------------------------------------------------------------------ exact --

GRIDS = {"narrow": inputs.NARROW_GRID, "wide": None}


def _check_exact_or_close(out_bits, ref, grid, what, amax_prod):
    """Narrow grid: bit-exact. Wide grid: within the MFMA's own error bound.

    The wide grid puts +-448 values among small ones (so some blocks hold a
    448 x 448 product next to products as small as 2^-4) and lets the products
    cancel, which stresses the matrix core's internal accumulation. One fp8
    16x16x128 MFMA does not add such products exactly:
    tests/test_gpu_mfma_exactness.py pins each block's deviation from the
    exact sum to at most 2^-10 of the block's largest product magnitude. The
    bound here is that term summed over the blocks, taken at the largest
    possible product (amax_x * amax_w = 448^2 * sx * sw), plus the bf16
    rounding of the result (2^-8 |ref|).

    The number of outputs outside the tolerance band 2^-7 |ref| + 1e-3
    rms(ref) is printed: on these adversarial operands the MFMA's own error
    can exceed that band where the products cancel to a small result.
    """
    if grid == "narrow":
        _assert_bits_equal(out_bits, gemm.bf16_rne(ref), ref, f"exact {what}")
        return
    got = gemm.bf16_bits_to_f64(out_bits)
    _, ns = gemm.within_tolerance(out_bits, ref)
    print(f"[gpu] wide-grid {what}: {ns['violations']} of {ref.size} outputs outside the tolerance band "
          f"(worst err/bound {ns['worst_err_over_bound']:.3g})", flush=True)
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -10 * amax_prod
    bad = np.abs(got - ref) > bound
    assert not bad.any(), f"wide-grid {what}: {bad.sum()} outputs beyond the MFMA bound"


@pytest.mark.parametrize("grid", list(GRIDS))
def test_exact_fwd(grid):
    M, N, K = 320, 640, 512
    note(f"exact fwd ({grid}) M={M} N={N} K={K}")
    g1, g2 = inputs.tensor_streams(101, 2)
    x = inputs.exact_operand(g1, 384, K, np.array([[-2] * 4, [1] * 4, [0] * 4]), GRIDS[grid])[:M]
    w = inputs.exact_operand(g2, N, K, np.array([[-7] * 4, [-5] * 4, [-6] * 4, [-8] * 4, [-4] * 4]), GRIDS[grid])
    xq, xs = fq.quantize_act_1x128(dev_bf16(x))
    wq, ws, _ = fq.quantize_weight_128x128(dev_bf16(w), transposed=False)
    y = fq.fp8_gemm_fwd(xq, xs, wq, ws)
    torch.cuda.synchronize()
    oxq, oxs = quant.quantize_act_1x128(x)
    owq, ows, _ = quant.quantize_weight_128x128(w)
    ref = gemm.gemm_fwd(oxq, oxs, owq, ows)
    _check_exact_or_close(host_bits(y), ref, grid, "fwd", 448.0 ** 2 * (oxs.astype(np.float64) @ ows.astype(np.float64).repeat(128, axis=0).T))


@pytest.mark.parametrize("grid", list(GRIDS))
def test_exact_dgrad(grid):
    M, N, K = 320, 512, 640
    note(f"exact dgrad ({grid}) M={M} N={N} K={K}")
    g1, g2 = inputs.tensor_streams(102, 2)
    dy = inputs.exact_operand(g1, 384, N, np.array([[-3] * 4, [0] * 4, [2] * 4]), GRIDS[grid])[:M]
    w = inputs.exact_operand(g2, N, K, np.array([[-6, -7, -5, -6, -8]] * 4), GRIDS[grid])
    dyq, dys = fq.quantize_act_1x128(dev_bf16(dy))
    wq, ws, wq_t = fq.quantize_weight_128x128(dev_bf16(w))
    dx = fq.fp8_gemm_dgrad(dyq, dys, wq_t, ws)
    torch.cuda.synchronize()
    odq, ods = quant.quantize_act_1x128(dy)
    owq, ows, _ = quant.quantize_weight_128x128(w)
    ref = gemm.gemm_dgrad(odq, ods, owq, ows)
    _check_exact_or_close(host_bits(dx), ref, grid, "dgrad", 448.0 ** 2 * (ods.astype(np.float64) @ ows.astype(np.float64).repeat(128, axis=1)))


@pytest.mark.parametrize("grid", list(GRIDS))
def test_exact_wgrad(grid):
    M, N, K = 512, 384, 640
    note(f"exact wgrad ({grid}) M={M} N={N} K={K}")
    g1, g2 = inputs.tensor_streams(103, 2)
    dy = inputs.exact_operand(g1, M, N, np.array([[-4, -2, -3]] * 4), GRIDS[grid])
    x = inputs.exact_operand(g2, M, K, np.array([[0, 1, -1, 2, 0]] * 4), GRIDS[grid])
    dyq_t, dys_t = fq.transpose_quantize_128x1(dev_bf16(dy))
    xq_t, xs_t = fq.transpose_quantize_128x1(dev_bf16(x))
    dw = fq.fp8_gemm_wgrad(dyq_t, dys_t, xq_t, xs_t)
    torch.cuda.synchronize()
    oq1, os1 = quant.transpose_quantize_128x1(dy)
    oq2, os2 = quant.transpose_quantize_128x1(x)
    ref = gemm.gemm_wgrad(oq1, os1, oq2, os2)
    _check_exact_or_close(host_bits(dw), ref, grid, "wgrad", 448.0 ** 2 * (os1.astype(np.float64) @ os2.astype(np.float64).T))


# Shapes that route to the large (256 x 256) tile configuration: at least 256
# large tiles and a ragged dimension (33 x 128 rows: the last tile is shifted
# back and overlaps its neighbour). The ones above run the small configuration.

# Block exponents vary only along the non-contracted dimension, so that every
# K block of one output carries the same power-of-two scale product and the
# fp32 sums stay exact (as in the tests above).

def _exps_by_row(rng, rb, cb, lo, hi):
    return np.repeat(rng.integers(lo, hi, size=(rb, 1)), cb, axis=1)


def _exps_by_col(rng, rb, cb, lo, hi):
    return np.repeat(rng.integers(lo, hi, size=(1, cb)), rb, axis=0)


@pytest.mark.parametrize("grid", list(GRIDS))
def test_exact_large_tiles_fwd(grid):
    M, N, K = 4224, 4096, 256
    note(f"exact fwd, large tiles ({grid}) M={M} N={N} K={K}")
    g1, g2, g3 = inputs.tensor_streams(111, 3)
    x = inputs.exact_operand(g1, M, K, _exps_by_row(g3, M // 128, K // 128, -3, 2), GRIDS[grid])
    w = inputs.exact_operand(g2, N, K, _exps_by_row(g3, N // 128, K // 128, -8, -4), GRIDS[grid])
    xq, xs = fq.quantize_act_1x128(dev_bf16(x))
    wq, ws, _ = fq.quantize_weight_128x128(dev_bf16(w), transposed=False)
    y = fq.fp8_gemm_fwd(xq, xs, wq, ws)
    torch.cuda.synchronize()
    oxq, oxs = quant.quantize_act_1x128(x)
    owq, ows, _ = quant.quantize_weight_128x128(w)
    ref = gemm.gemm_fwd(oxq, oxs, owq, ows)
    _check_exact_or_close(host_bits(y), ref, grid, "fwd large tiles",
                          448.0 ** 2 * (oxs.astype(np.float64) @ ows.astype(np.float64).repeat(128, axis=0).T))


@pytest.mark.parametrize("grid", list(GRIDS))
def test_exact_large_tiles_dgrad(grid):
    M, N, K = 4224, 256, 4096
    note(f"exact dgrad, large tiles ({grid}) M={M} N={N} K={K}")
    g1, g2, g3 = inputs.tensor_streams(112, 3)
    dy = inputs.exact_operand(g1, M, N, _exps_by_row(g3, M // 128, N // 128, -3, 2), GRIDS[grid])
    w = inputs.exact_operand(g2, N, K, _exps_by_col(g3, N // 128, K // 128, -8, -4), GRIDS[grid])
    dyq, dys = fq.quantize_act_1x128(dev_bf16(dy))
    wq, ws, wq_t = fq.quantize_weight_128x128(dev_bf16(w))
    dx = fq.fp8_gemm_dgrad(dyq, dys, wq_t, ws)
    torch.cuda.synchronize()
    odq, ods = quant.quantize_act_1x128(dy)
    owq, ows, _ = quant.quantize_weight_128x128(w)
    ref = gemm.gemm_dgrad(odq, ods, owq, ows)
    _check_exact_or_close(host_bits(dx), ref, grid, "dgrad large tiles",
                          448.0 ** 2 * (ods.astype(np.float64) @ ows.astype(np.float64).repeat(128, axis=1)))


@pytest.mark.parametrize("grid", list(GRIDS))
def test_exact_large_tiles_wgrad(grid):
    M, N, K = 256, 4096, 4224
    note(f"exact wgrad, large tiles ({grid}) M={M} N={N} K={K}")
    g1, g2, g3 = inputs.tensor_streams(113, 3)
    dy = inputs.exact_operand(g1, M, N, _exps_by_col(g3, M // 128, N // 128, -4, 0), GRIDS[grid])
    x = inputs.exact_operand(g2, M, K, _exps_by_col(g3, M // 128, K // 128, -1, 3), GRIDS[grid])
    dyq_t, dys_t = fq.transpose_quantize_128x1(dev_bf16(dy))
    xq_t, xs_t = fq.transpose_quantize_128x1(dev_bf16(x))
    dw = fq.fp8_gemm_wgrad(dyq_t, dys_t, xq_t, xs_t)
    torch.cuda.synchronize()
    oq1, os1 = quant.transpose_quantize_128x1(dy)
    oq2, os2 = quant.transpose_quantize_128x1(x)
    ref = gemm.gemm_wgrad(oq1, os1, oq2, os2)
    _check_exact_or_close(host_bits(dw), ref, grid, "wgrad large tiles",
                          448.0 ** 2 * (os1.astype(np.float64) @ os2.astype(np.float64).T))


# Long contractions (K / 128 >= 64) put the large and medium configurations on
# their chip-wide tile order: whole 16 x 16 blocks of tiles shared by the eight
# XCDs, the remaining partial rows and columns of tiles in the plain order. The
# large case is a 19 x 22 grid of 256 x 256 tiles (418 tiles, two rounds of the
# chip); the medium case a 19 x 28 grid of 256 x 128 tiles (266 large tiles
# would take two rounds, 532 medium ones take three at about half the cost).
# Both have one or two whole blocks plus both kinds of remainder and a ragged
# last tile along j. At least one output of every tile (one sample per tile
# extent in each dimension) is checked against the oracle, so a tile computed
# in the wrong place or not at all would show.

@pytest.mark.parametrize("config,rows_j", [("large", 5504), ("medium", 3520)])
@pytest.mark.parametrize("role", ["fwd", "dgrad", "wgrad"])
def test_every_tile_long_contraction(role, config, rows_j):
    long_k, cols_i = 8192, 4864                    # 64 K blocks; 19 tiles along i
    jband = 256 if config == "large" else 128      # tile extent along the output rows
    if role == "fwd":
        M, N, K = rows_j, cols_i, long_k
    elif role == "dgrad":
        M, N, K = rows_j, long_k, cols_i
    else:
        M, N, K = long_k, rows_j, cols_i
    note(f"every tile, long contraction ({config} tiles): {role} M={M} N={N} K={K}")
    x = inputs.bf16_normal_device((M, K), 1.0, 0.01, seed=71)
    w = inputs.bf16_normal_device((N, K), 0.02, 0.0, seed=72)
    dy = inputs.bf16_normal_device((M, N), 1e-3, 0.0, seed=73)
    if role == "fwd":
        xq, xs = fq.quantize_act_1x128(x)
        wq, ws, _ = fq.quantize_weight_128x128(w, transposed=False)
        out = fq.fp8_gemm_fwd(xq, xs, wq, ws)
        torch.cuda.synchronize()
        r, c = one_per_tile(M, 1, band=jband), one_per_tile(N, 2, group=128)
        oxq, oxs = quant.quantize_act_1x128(host_bits(x[r]))
        owq, ows, _ = quant.quantize_weight_128x128(host_bits(w[c]))
        ref = gemm.gemm_fwd(oxq, oxs, owq, ows)
    elif role == "dgrad":
        dyq, dys = fq.quantize_act_1x128(dy)
        wq, ws, wq_t = fq.quantize_weight_128x128(w)
        out = fq.fp8_gemm_dgrad(dyq, dys, wq_t, ws)
        torch.cuda.synchronize()
        r, c = one_per_tile(M, 3, band=jband), one_per_tile(K, 4, group=128)
        odq, ods = quant.quantize_act_1x128(host_bits(dy[r]))
        owq, ows, _ = quant.quantize_weight_128x128(host_bits(w[:, c]))
        ref = gemm.gemm_dgrad(odq, ods, owq, ows)
    else:
        dyq_t, dys_t = fq.transpose_quantize_128x1(dy)
        xq_t, xs_t = fq.transpose_quantize_128x1(x)
        out = fq.fp8_gemm_wgrad(dyq_t, dys_t, xq_t, xs_t)
        torch.cuda.synchronize()
        r, c = one_per_tile(N, 5, band=jband), one_per_tile(K, 6)
        oq1, os1 = quant.transpose_quantize_128x1(host_bits(dy[:, r]))
        oq2, os2 = quant.transpose_quantize_128x1(host_bits(x[:, c]))
        ref = gemm.gemm_wgrad(oq1, os1, oq2, os2)
    _assert_close(host_bits(out[r][:, c]), ref, f"{role} every tile, long contraction, {config} tiles")


# ---------------------------------------------------------- grouped calls --

def _quantized_problem(role, M, N, K, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    u8 = lambda *sh: torch.randint(0, 0x7E, sh, dtype=torch.uint8, device="cuda", generator=g) | (
        torch.randint(0, 2, sh, dtype=torch.uint8, device="cuda", generator=g) << 7)
    f32 = lambda *sh: torch.rand(sh, device="cuda", generator=g) * 0.01 + 1e-3
    if role == "fwd":
        return (u8(M, K), f32(M, K // 128), u8(N, K), f32(N // 128, K // 128))
    if role == "dgrad":
        return (u8(M, N), f32(M, N // 128), u8(K, N), f32(N // 128, K // 128))
    return (u8(N, M), f32(N, M // 128), u8(K, M), f32(K, M // 128))


@pytest.mark.parametrize("role", ["fwd", "dgrad", "wgrad"])
@pytest.mark.parametrize("shapes", [
    [(256, 512, 384), (128, 256, 640), (384, 128, 128), (256, 384, 256)],      # small tiles
    [(256, 4096, 4096), (512, 4224, 2048), (256, 2048, 4096)],                # large tiles
    [(128, 256, 256)] * 20,                                                   # more than one launch
    # 8192 tokens: long contractions in WGrad (64 K blocks: the supertile
    # order inside a grouped launch), 392 large tiles in all, tile counts of
    # 272, 40 and 80 (not multiples of the 256-aligned ranges), ragged tiles
    [(8192, 4096, 4224), (8192, 1152, 8192), (8192, 5120, 896)],
])
def test_grouped_equals_plain_calls(role, shapes):
    note(f"grouped {role}: {len(shapes)} problems {shapes[:3]}")
    problems = [_quantized_problem(role, M, N, K, seed=7 * i + len(shapes)) for i, (M, N, K) in enumerate(shapes)]
    outs = getattr(fq, f"fp8_gemm_{role}_grouped")(problems)
    plain = getattr(fq, f"fp8_gemm_{role}")
    refs = [plain(*pr) for pr in problems]
    torch.cuda.synchronize()
    for i, (o, r) in enumerate(zip(outs, refs)):
        assert torch.equal(o, r), f"{role} problem {i}"


# ----------------------------------- K / 128 not a multiple of 4 (any K) --
#
# The per-row scales of 4 consecutive K blocks reach LDS with one 16-byte copy
# per row when the contraction has a multiple of 4 blocks, and with 4-byte
# copies (a kernel of its own) otherwise. Padding the contraction with +0
# codes up to the next multiple of 4 blocks (scale 1 there) only adds exact
# zeros to every running sum, so the two forms must give the same bits; the
# plain form is checked against the oracle everywhere else.

def _pad_contraction(role, ops, kb_to):
    """The same problem with its contraction padded by +0 codes to kb_to blocks."""
    def pad_codes(t):            # contraction along dim 1
        out = torch.zeros(t.shape[0], 128 * kb_to, dtype=t.dtype, device=t.device)
        out[:, :t.shape[1]] = t
        return out

    def pad_cols(s):             # scales with the contraction along dim 1
        out = torch.ones(s.shape[0], kb_to, dtype=s.dtype, device=s.device)
        out[:, :s.shape[1]] = s
        return out

    def pad_rows(s):             # block scales with the contraction along dim 0
        out = torch.ones(kb_to, s.shape[1], dtype=s.dtype, device=s.device)
        out[:s.shape[0]] = s
        return out

    a, sa, b, sb = ops
    if role == "fwd":
        return pad_codes(a), pad_cols(sa), pad_codes(b), pad_cols(sb)
    if role == "dgrad":
        return pad_codes(a), pad_cols(sa), pad_codes(b), pad_rows(sb)
    return pad_codes(a), pad_cols(sa), pad_codes(b), pad_cols(sb)


@pytest.mark.parametrize("role", ["fwd", "dgrad", "wgrad"])
@pytest.mark.parametrize("rows,cols,kb", [
    (4096, 4096, 3),      # large tiles, one partial group
    (4096, 4096, 9),      # large tiles, two whole groups and a partial one
    (4096, 4096, 65),     # large tiles, long contraction (chip-wide tile order)
    (4096, 2048, 6),      # small tiles
    (200, 640, 5),        # tiny tiles, a ragged dimension
    (40, 128, 2),         # clamped tiny tiles
])
def test_any_k_block_count_equals_zero_padded(role, rows, cols, kb):
    kb_to = (kb + 3) // 4 * 4
    L = 128 * kb
    M, N, K = {"fwd": (rows, cols, L), "dgrad": (rows, L, cols), "wgrad": (L, rows, cols)}[role]
    note(f"{role} with {kb} K blocks vs zero-padded to {kb_to}: M={M} N={N} K={K}")
    ops = _quantized_problem(role, M, N, K, seed=1000 + kb)
    plain = getattr(fq, f"fp8_gemm_{role}")
    out = plain(*ops)
    padded = plain(*_pad_contraction(role, ops, kb_to))
    torch.cuda.synchronize()
    assert torch.equal(out, padded), f"{role} {kb} K blocks: differs from the zero-padded contraction"


# ------------------------------------------- oracle operands, small shapes --

@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (17, 384, 256), (300, 640, 1152), (64, 256, 4096)])
def test_fwd_and_dgrad_on_oracle_operands(M, N, K):
    note(f"fwd/dgrad on oracle operands M={M} N={N} K={K}")
    g1, g2, g3 = inputs.tensor_streams(M + N + K, 3)
    x = inputs.bf16_normal(g1, (M, K), 1.0, 0.01)
    w = inputs.bf16_normal(g2, (N, K), 0.02)
    dy = inputs.bf16_normal(g3, (M, N), 1e-3)
    xq, xs = quant.quantize_act_1x128(x)
    wq, ws, wq_t = quant.quantize_weight_128x128(w)
    dyq, dys = quant.quantize_act_1x128(dy)
    y = fq.fp8_gemm_fwd(dev_u8(xq), dev_f32(xs), dev_u8(wq), dev_f32(ws))
    dx = fq.fp8_gemm_dgrad(dev_u8(dyq), dev_f32(dys), dev_u8(wq_t), dev_f32(ws))
    torch.cuda.synchronize()
    _assert_close(host_bits(y), gemm.gemm_fwd(xq, xs, wq, ws), "fwd")
    _assert_close(host_bits(dx), gemm.gemm_dgrad(dyq, dys, wq, ws), "dgrad")


@pytest.mark.parametrize("M,N,K", [(128, 128, 128), (384, 256, 640), (1024, 384, 128)])
def test_wgrad_on_oracle_operands(M, N, K):
    note(f"wgrad on oracle operands M={M} N={N} K={K}")
    g1, g2 = inputs.tensor_streams(M * 3 + N + K, 2)
    x = inputs.bf16_normal(g1, (M, K), 1.0, 0.01)
    dy = inputs.bf16_normal(g2, (M, N), 1.0, 0.01)
    xq_t, xs_t = quant.transpose_quantize_128x1(x)
    dyq_t, dys_t = quant.transpose_quantize_128x1(dy)
    dw = fq.fp8_gemm_wgrad(dev_u8(dyq_t), dev_f32(dys_t), dev_u8(xq_t), dev_f32(xs_t))
    torch.cuda.synchronize()
    _assert_close(host_bits(dw), gemm.gemm_wgrad(dyq_t, dys_t, xq_t, xs_t), "wgrad")


def test_identity_weight():
    note("fwd with W = 448 I: Y is 448 * x_hat")
    N = K = 384
    w = np.zeros((N, K), np.uint16)
    w[np.arange(N), np.arange(N)] = inputs.f32_to_bf16_bits(np.array([448.0], np.float32))[0]
    (g,) = inputs.tensor_streams(5, 1)
    x = inputs.bf16_normal(g, (200, K), 1.0, 0.01)
    xq, xs = fq.quantize_act_1x128(dev_bf16(x))
    wq, ws, wq_t = fq.quantize_weight_128x128(dev_bf16(w))
    y = fq.fp8_gemm_fwd(xq, xs, wq, ws)
    dx = fq.fp8_gemm_dgrad(xq, xs, wq_t, ws)
    torch.cuda.synchronize()
    oxq, oxs = quant.quantize_act_1x128(x)
    ref = 448.0 * gemm.dequant_rows(oxq, oxs)
    _assert_close(host_bits(y), ref, "fwd identity")
    _assert_close(host_bits(dx), ref, "dgrad identity")


@pytest.mark.parametrize("role", ["fwd", "dgrad"])
def test_rows_identical_across_tile_configurations(role):
    # Every tile configuration reduces K in the same order, so a token's output
    # row does not depend on how many tokens share the call. With N = K = 4096:
    # 4352 tokens run the 256x128 tiles (272 large tiles would take two rounds
    # of the chip, 544 medium ones take three at about half the cost each),
    # 4096 the 256x256 tiles, 1024 the 128x64 tiles, 256 and 64 the 64x64
    # tiles, 17 the 64x64 tiles with clamped rows.
    M, N, K = 4352, 4096, 4096
    note(f"{role}: rows of a {M}-token call vs 4096/1024/256/64/17-token calls (every tile configuration)")
    a, as_, b, bs = _quantized_problem(role, M, N, K, seed=77)
    f = getattr(fq, f"fp8_gemm_{role}")
    full = f(a, as_, b, bs)
    parts = {rows: f(a[:rows].contiguous(), as_[:rows].contiguous(), b, bs) for rows in (4096, 1024, 256, 64, 17)}
    torch.cuda.synchronize()
    for rows, part in parts.items():
        assert torch.equal(part, full[:rows]), f"{role}: {rows} rows differ from the {M}-row call"


@pytest.mark.parametrize("role", ["fwd", "dgrad"])
def test_rows_identical_wide_weight_few_tokens(role):
    # 256 tokens against 27648 weight rows run the 256x128 tiles (216 of them,
    # one round of the chip); 1024 tokens the 256x256 tiles, 64 and 17 the
    # 64x64 tiles. A token's row is the same bits in every one.
    M, N, K = 256, 27648, 1024
    if role == "dgrad":
        N, K = 1024, 27648
    note(f"{role}: rows of a {M}-token call vs 1024/64/17-token calls, 27648 weight rows")
    a_full, as_full, b, bs = _quantized_problem(role, 1024, N, K, seed=78)
    f = getattr(fq, f"fp8_gemm_{role}")
    big = f(a_full, as_full, b, bs)
    full = f(a_full[:M].contiguous(), as_full[:M].contiguous(), b, bs)
    parts = {rows: f(a_full[:rows].contiguous(), as_full[:rows].contiguous(), b, bs) for rows in (64, 17)}
    torch.cuda.synchronize()
    assert torch.equal(full, big[:M]), f"{role}: the {M}-row call differs from the 1024-row call"
    for rows, part in parts.items():
        assert torch.equal(part, full[:rows]), f"{role}: {rows} rows differ from the {M}-row call"


def test_gemm_determinism():
    note("GEMMs: repeated calls give identical bytes")
    x = inputs.bf16_normal_device((2048, 4096), 1.0, 0.01, seed=21)
    w = inputs.bf16_normal_device((4096, 4096), 0.02, 0.0, seed=22)
    xq, xs = fq.quantize_act_1x128(x)
    wq, ws, wq_t = fq.quantize_weight_128x128(w)
    xq_t, xs_t = fq.transpose_quantize_128x1(x)
    a = fq.fp8_gemm_fwd(xq, xs, wq, ws)
    b = fq.fp8_gemm_fwd(xq, xs, wq, ws)
    c = fq.fp8_gemm_dgrad(xq, xs, wq_t, ws)
    d = fq.fp8_gemm_dgrad(xq, xs, wq_t, ws)
    e = fq.fp8_gemm_wgrad(xq_t, xs_t, xq_t, xs_t)
    f = fq.fp8_gemm_wgrad(xq_t, xs_t, xq_t, xs_t)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(c, d) and torch.equal(e, f)


# --------------------------------------------- full-size workloads, sampled --
#
# Every GEMM of every workload runs at full size, quantized on the GPU as the
# benchmark quantizes (the dual quantizer wherever a tensor needs both
# groupings), and at least one output of every output tile is checked against
# the oracle, whatever tile configuration the launch picks: the smallest tile
# extent along either output dimension is 64, so the check takes one row and
# one column in every 64-wide band (plus the last ones). A tile computed in
# the wrong place, twice or not at all by the tile maps, the supertile order
# or the grouped offsets would show. The oracle quantizes every input from the
# same bf16 bytes (the whole weight: its 128x128 blocks are independent, so
# 128-row bands are quantized in parallel threads and stacked).

TILE_BAND = 64

def _quantize_for_passes(x, dy, w, passes):
    """GPU quantization of one linear's operands, the way the benchmark step does it."""
    fwd, dgrad, wgrad = "fwd" in passes, "dgrad" in passes, "wgrad" in passes
    q = {}
    if fwd and wgrad:
        q["xq"], q["xs"], q["xq_t"], q["xs_t"] = fq.quantize_dual_1x128_128x1(x)
    elif fwd:
        q["xq"], q["xs"] = fq.quantize_act_1x128(x)
    if dgrad and wgrad:
        q["dyq"], q["dys"], q["dyq_t"], q["dys_t"] = fq.quantize_dual_1x128_128x1(dy)
    elif dgrad:
        q["dyq"], q["dys"] = fq.quantize_act_1x128(dy)
    if wgrad and "xq_t" not in q:
        q["xq_t"], q["xs_t"] = fq.transpose_quantize_128x1(x)
    if wgrad and "dyq_t" not in q:
        q["dyq_t"], q["dys_t"] = fq.transpose_quantize_128x1(dy)
    if fwd or dgrad:
        q["wq"], q["ws"], q["wq_t"] = fq.quantize_weight_128x128(w, transposed=dgrad)
    return q


def _check_linear(lin, passes, seed, keep_wgrad=False):
    """Run the linear's passes on the GPU at full size and check one output
    in every 64 x 64 band of each output against the oracle. Returns the
    WGrad operands and output when keep_wgrad is set."""
    M, N, K = lin["M"], lin["N"], lin["K"]
    t = inputs.linear_tensors_device(lin, seed=seed)
    x, w, dy = t["x"], t["w"], t["dy"]
    q = _quantize_for_passes(x, dy, w, passes)
    kept = None
    if "fwd" in passes or "dgrad" in passes:
        owq, ows = oracle_weight(w)
    if "fwd" in passes:
        note(f"{lin['name']} fwd M={M} N={N} K={K}")
        y = fq.fp8_gemm_fwd(q["xq"], q["xs"], q["wq"], q["ws"])
        torch.cuda.synchronize()
        rows = one_per_tile(M, seed, band=TILE_BAND)
        cols = one_per_tile(N, seed + 1, band=TILE_BAND)
        oxq, oxs = quant.quantize_act_1x128(host_bits(x[rows]))
        # rows `cols` of the dequantized weight: each weight row with its block's scales
        w_sel = gemm.dequant_rows(owq[cols], ows[cols // 128])
        ref = gemm.dequant_rows(oxq, oxs) @ w_sel.T
        _assert_close(host_bits(y[rows][:, cols]), ref, f"{lin['name']} fwd, {len(rows)} x {len(cols)} outputs")
        del y
    if "dgrad" in passes:
        note(f"{lin['name']} dgrad M={M} N={N} K={K}")
        dx = fq.fp8_gemm_dgrad(q["dyq"], q["dys"], q["wq_t"], q["ws"])
        torch.cuda.synchronize()
        rows = one_per_tile(M, seed + 2, band=TILE_BAND)
        cols = one_per_tile(K, seed + 3, band=TILE_BAND)
        odq, ods = quant.quantize_act_1x128(host_bits(dy[rows]))
        # columns `cols` of the dequantized weight, as rows (contraction over N)
        w_sel = gemm.dequant_rows(np.ascontiguousarray(owq[:, cols].T), np.ascontiguousarray(ows[:, cols // 128].T))
        ref = gemm.dequant_rows(odq, ods) @ w_sel.T
        _assert_close(host_bits(dx[rows][:, cols]), ref, f"{lin['name']} dgrad, {len(rows)} x {len(cols)} outputs")
        del dx
    if "wgrad" in passes:
        note(f"{lin['name']} wgrad M={M} N={N} K={K}")
        dw = fq.fp8_gemm_wgrad(q["dyq_t"], q["dys_t"], q["xq_t"], q["xs_t"])
        torch.cuda.synchronize()
        ns = one_per_tile(N, seed + 4, band=TILE_BAND)
        ks = one_per_tile(K, seed + 5, band=TILE_BAND)
        oq1, os1 = quant.transpose_quantize_128x1(host_bits(dy[:, ns]))
        oq2, os2 = quant.transpose_quantize_128x1(host_bits(x[:, ks]))
        ref = gemm.gemm_wgrad(oq1, os1, oq2, os2)
        _assert_close(host_bits(dw[ns][:, ks]), ref, f"{lin['name']} wgrad, {len(ns)} x {len(ks)} outputs")
        if keep_wgrad:
            kept = ((q["dyq_t"], q["dys_t"], q["xq_t"], q["xs_t"]), dw)
        else:
            del dw
    del t, x, w, dy, q
    torch.cuda.empty_cache()
    return kept


@pytest.mark.parametrize("workload", list(inputs.WORKLOADS))
def test_workload_full_size(workload):
    wl = inputs.WORKLOADS[workload]
    grouped = "wgrad" in wl["passes"] and len(wl["linears"]) > 1
    kept = [_check_linear(lin, wl["passes"], seed=1000 + 17 * idx, keep_wgrad=grouped)
            for idx, lin in enumerate(wl["linears"])]
    if grouped:
        # the benchmark's launch: every linear's WGrad in one grouped launch,
        # bit-identical to the plain calls checked above
        note(f"{workload}: grouped WGrad of {len(kept)} linears vs the plain calls")
        outs = fq.fp8_gemm_wgrad_grouped([k[0] for k in kept])
        torch.cuda.synchronize()
        for lin, k, o in zip(wl["linears"], kept, outs):
            assert torch.equal(o, k[1]), f"{workload} {lin['name']}: grouped WGrad differs from the plain call"
        del kept, outs
        torch.cuda.empty_cache()


def test_tiny_fwd_every_output():
    """The tiny forward case checked on every output element, numpy inputs (seed 0)."""
    lin = inputs.WORKLOADS["tiny_fwd_128x256x256"]["linears"][0]
    note("tiny fwd 128x256x256, every output")
    t = inputs.linear_tensors(lin, seed=0)
    xq, xs = fq.quantize_act_1x128(dev_bf16(t["x"]))
    wq, ws, _ = fq.quantize_weight_128x128(dev_bf16(t["w"]))
    y = fq.fp8_gemm_fwd(xq, xs, wq, ws)
    torch.cuda.synchronize()
    oxq, oxs = quant.quantize_act_1x128(t["x"])
    owq, ows, _ = quant.quantize_weight_128x128(t["w"])
    _assert_close(host_bits(y), gemm.gemm_fwd(oxq, oxs, owq, ows), "tiny fwd")
