"""Pins of the oracle's three group quantizers.

What fixes each check (none of them re-runs the oracle's own formula):
* exact rational arithmetic for the fp32 scale and quotient, and a
  brute-force nearest-code search, on sampled groups (the rounding pipeline);
* invariants: every group's largest element maps to +-448 for every possible
  bf16 amax; power-of-two equivariance; all-zero groups;
* brute force on one-hot tensors for the group/block geometry;
* transpose identities between the three quantizers;
* an independent implementation of the whole pipeline in torch;
* hand-derived fixtures under tests/golden/.
"""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from fp8_block_scaled_quantize_amd.inputs import bf16_normal, f32_to_bf16_bits, tensor_streams
from oracle import e4m3, quant
from tests._exact import nearest_e4m3_code, rn_float32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(x32):
    return f32_to_bf16_bits(np.asarray(x32, dtype=np.float32))


def _llama_like(rows, cols, seed=0):
    (g,) = tensor_streams(seed, 1)
    return bf16_normal(g, (rows, cols), 1.0, 0.01)


# ---------------------------------------------------------------- pipeline --

def _exact_group(vals_f32):
    """Scale and codes of one group by exact rationals + brute-force rounding."""
    xs = [Fraction(float(v)) for v in vals_f32]
    amax = max(abs(v) for v in xs)
    s = Fraction(1) if amax == 0 else rn_float32(amax / 448)
    codes = []
    for v, v32 in zip(xs, vals_f32):
        qf = rn_float32(v / s)
        c = nearest_e4m3_code(qf)
        if np.signbit(v32) and c == 0:
            c = 0x80
        codes.append(c)
    return s, codes


def test_rounding_pipeline_matches_exact_rationals():
    x = _llama_like(16, 512)                       # 64 groups of 128
    xq, xs = quant.quantize_act_1x128(x)
    xf = e4m3.bf16_bits_to_f32(x)
    for m in range(16):
        for g in range(4):
            s, codes = _exact_group(xf[m, 128 * g:128 * g + 128])
            assert Fraction(float(xs[m, g])) == s
            assert list(xq[m, 128 * g:128 * g + 128]) == codes


def test_rounding_pipeline_double_rounding_cases():
    """Where fl32(x/s) lands on an E4M3 tie, the code follows the float32 quotient.

    This is the reading the oracle takes (one float32 division, then the
    codec). Such cases exist in realistic data, and on them rounding the exact
    quotient once would give a different byte; the check makes sure the
    sample contains some and that the oracle sides with the float32 quotient.
    """
    x = _llama_like(256, 4096, seed=3)
    xq, xs = quant.quantize_act_1x128(x)
    xf = e4m3.bf16_bits_to_f32(x).reshape(-1, 128)
    s = xs.reshape(-1).astype(np.float32)
    qf = (xf / s[:, None]).astype(np.float32)
    # Is the float32 quotient exactly a midpoint of two E4M3 neighbours?
    a = np.abs(qf.astype(np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6)
    step = np.exp2(e - 3)
    ties = (a > 0) & (np.mod(a / step, 1.0) == 0.5)
    idx = np.argwhere(ties)
    assert len(idx) > 0
    differ = 0
    codes = xq.reshape(-1, 128)
    for gi, j in idx[:200]:
        v = Fraction(float(xf[gi, j]))
        sf = Fraction(float(s[gi]))
        want = nearest_e4m3_code(rn_float32(v / sf))
        single = nearest_e4m3_code(v / sf)
        if v < 0:
            want |= 0x80
            single |= 0x80
        assert codes[gi, j] == want
        differ += int(want != single)
    assert differ > 0


# --------------------------------------------------------------- invariants --

def test_amax_maps_to_448_for_every_bf16_amax():
    bits = np.arange(1, 0x7F80, dtype=np.uint16)          # every positive finite bf16
    amax = e4m3.bf16_bits_to_f32(bits)
    G = np.zeros((bits.size, 128), dtype=np.uint16)
    G[:, 0] = bits
    G[:, 77] = bits | 0x8000                               # -amax in the same group
    G[:, 5] = _bits(amax * np.float32(0.3))
    xq, xs = quant.quantize_act_1x128(G)
    assert np.all(xq[:, 0] == 0x7E) and np.all(xq[:, 77] == 0xFE)
    ratio = amax.astype(np.float64) / xs[:, 0].astype(np.float64)
    assert ratio.min() >= 447.3 and ratio.max() <= 448.9
    normal_s = xs[:, 0] >= np.float32(2.0 ** -126)
    assert np.all(np.abs(ratio[normal_s] - 448.0) <= 448.0 * 2.0 ** -22)


def test_power_of_two_equivariance():
    x = _llama_like(64, 256, seed=5)
    xq, xs = quant.quantize_act_1x128(x)
    xf = e4m3.bf16_bits_to_f32(x)
    for j in (-20, -7, -1, 1, 3, 11):
        y = _bits(xf * np.float32(2.0 ** j))              # exact: stays bf16, stays normal
        assert np.array_equal(e4m3.bf16_bits_to_f32(y), xf * np.float32(2.0 ** j))
        yq, ys = quant.quantize_act_1x128(y)
        assert np.array_equal(yq, xq)
        assert np.array_equal(ys, xs * np.float32(2.0 ** j))


def test_all_zero_groups():
    x = np.zeros((128, 256), dtype=np.uint16)
    x[3, 200] = 0x8000                                     # a -0.0 in an otherwise zero group
    for q, s in (quant.quantize_act_1x128(x), quant.transpose_quantize_128x1(x),
                 quant.quantize_weight_128x128(x)[:2]):
        assert np.all(s == 1.0)
        assert set(np.unique(q)) <= {0x00, 0x80}
    xq, _ = quant.quantize_act_1x128(x)
    assert xq[3, 200] == 0x80 and np.count_nonzero(xq) == 1


# ----------------------------------------------------------------- geometry --

def _one_hot_positions():
    rng = np.random.default_rng(7)
    edges = [0, 1, 126, 127, 128, 129, 254, 255]
    pos = [(r, c) for r in edges for c in edges]
    pos += [tuple(p) for p in rng.integers(0, 256, size=(64, 2))]
    return pos


@pytest.mark.parametrize("value", [3.0, -0.015625, 1.2e-38])
def test_geometry_one_hot(value):
    vb = _bits([value])[0]
    v = e4m3.bf16_bits_to_f32(np.array([vb]))[0]
    expect_s = np.float32(np.float32(abs(v)) / np.float32(448.0))
    code = 0xFE if v < 0 else 0x7E
    for r, c in _one_hot_positions():
        x = np.zeros((256, 256), dtype=np.uint16)
        x[r, c] = vb
        # 1x128: one scale per (row, 128-column group)
        q, s = quant.quantize_act_1x128(x)
        want_s = np.ones((256, 2), np.float32)
        want_s[r, c // 128] = expect_s
        assert np.array_equal(s, want_s)
        want_q = np.zeros((256, 256), np.uint8)
        want_q[r, c] = code
        assert np.array_equal(q, want_q)
        # 128x128: one scale per block
        wq, ws, wq_t = quant.quantize_weight_128x128(x)
        want_ws = np.ones((2, 2), np.float32)
        want_ws[r // 128, c // 128] = expect_s
        assert np.array_equal(ws, want_ws)
        assert np.array_equal(wq, want_q) and np.array_equal(wq_t, want_q.T)
        # 128x1 transposed: xs_t[c, r // 128]
        qt, st = quant.transpose_quantize_128x1(x)
        want_st = np.ones((256, 2), np.float32)
        want_st[c, r // 128] = expect_s
        assert np.array_equal(st, want_st)
        assert np.array_equal(qt, want_q.T)


def test_transpose_identities():
    x = _llama_like(256, 384, seed=11)
    q1, s1 = quant.quantize_act_1x128(np.ascontiguousarray(x.T))
    qt, st = quant.transpose_quantize_128x1(x)
    assert np.array_equal(q1, qt) and np.array_equal(s1, st)
    wq, ws, wq_t = quant.quantize_weight_128x128(x)
    wq2, ws2, wq2_t = quant.quantize_weight_128x128(np.ascontiguousarray(x.T))
    assert np.array_equal(wq2, wq.T) and np.array_equal(ws2, ws.T) and np.array_equal(wq_t, wq.T)
    assert np.array_equal(wq2_t, wq)


@pytest.mark.parametrize("M", [1, 100, 127, 129, 300])
def test_transpose_ragged_token_count(M):
    # A tail of fewer than 128 tokens: per channel, the group of the remaining
    # tokens is quantized on its own (exact rationals + brute-force rounding)
    # and the padded positions hold +0 codes.
    x = _llama_like(M, 256, seed=M)
    qt, st = quant.transpose_quantize_128x1(x)
    Mp = -(-M // 128) * 128
    assert qt.shape == (256, Mp) and st.shape == (256, Mp // 128)
    assert np.all(qt[:, M:] == 0)
    xf = e4m3.bf16_bits_to_f32(x)
    for c in (0, 77, 255):
        for b in range(Mp // 128):
            vals = xf[128 * b:min(128 * b + 128, M), c]
            sc, codes = _exact_group(vals)
            assert float(st[c, b]) == float(sc)
            assert list(qt[c, 128 * b:128 * b + len(vals)]) == codes
    if M > 128:                       # the whole groups agree with the 1x128 rule on X^T
        full = (M // 128) * 128
        q1, s1 = quant.quantize_act_1x128(np.ascontiguousarray(x[:full].T))
        assert np.array_equal(qt[:, :full], q1) and np.array_equal(st[:, :full // 128], s1)


# -------------------------------------------------------- independent impl --

def test_matches_torch_pipeline():
    """The whole 1x128 pipeline re-implemented with torch ops and its fp8 cast."""
    x = _llama_like(512, 1024, seed=13)
    xq, xs = quant.quantize_act_1x128(x)
    t = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float().reshape(512, 8, 128)
    amax = t.abs().amax(dim=-1, keepdim=True)
    s = torch.where(amax == 0, torch.ones_like(amax), amax / torch.tensor(448.0))
    q = (t / s).to(torch.float8_e4m3fn).view(torch.uint8).reshape(512, 1024).numpy()
    assert np.array_equal(q, xq)
    assert np.array_equal(s.reshape(512, 8).numpy(), xs)


# ------------------------------------------------------------------ golden --

def _read_fixture(name):
    scale, rows = None, []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        if line.startswith("scale"):
            scale = float(line.split()[1])
        else:
            rows.append(line.split())
    return scale, rows


def test_golden_act_group():
    scale, rows = _read_fixture("act_1x128_hand.txt")
    x = np.zeros((1, 128), np.uint16)
    want = np.zeros(128, np.uint8)
    for col, b, code in rows:
        x[0, int(col)] = int(b, 16)
        want[int(col)] = int(code, 16)
    q, s = quant.quantize_act_1x128(x)
    assert s[0, 0] == np.float32(scale)
    assert np.array_equal(q[0], want)


def test_golden_weight_block():
    scale, rows = _read_fixture("weight_128x128_hand.txt")
    w = np.zeros((128, 128), np.uint16)
    want = np.zeros((128, 128), np.uint8)
    for r, c, b, code in rows:
        w[int(r), int(c)] = int(b, 16)
        want[int(r), int(c)] = int(code, 16)
    wq, ws, wq_t = quant.quantize_weight_128x128(w)
    assert ws[0, 0] == np.float32(scale)
    assert np.array_equal(wq, want) and np.array_equal(wq_t, want.T)


# ------------------------------------------------ partial channel groups --

@pytest.mark.parametrize("K", [1, 8, 100, 200, 264])
def test_act_partial_channel_group(K):
    # A row length that is not a multiple of 128 ends in a partial group: its
    # scale and codes are those of the remaining elements alone (exact
    # rationals + brute-force rounding) and the padded positions hold +0 codes.
    x = _llama_like(5, K, seed=K)
    xq, xs = quant.quantize_act_1x128(x)
    Kg = -(-K // 128)
    assert xq.shape == (5, 128 * Kg) and xs.shape == (5, Kg)
    assert np.all(xq[:, K:] == 0)
    xf = e4m3.bf16_bits_to_f32(x)
    for m in range(5):
        for g in range(Kg):
            vals = xf[m, 128 * g:min(128 * g + 128, K)]
            sc, codes = _exact_group(vals)
            assert Fraction(float(xs[m, g])) == sc
            assert list(xq[m, 128 * g:128 * g + len(vals)]) == codes
    if K > 128:                       # the whole groups agree with the aligned prefix
        full = (K // 128) * 128
        q1, s1 = quant.quantize_act_1x128(np.ascontiguousarray(x[:, :full]))
        assert np.array_equal(xq[:, :full], q1) and np.array_equal(xs[:, :full // 128], s1)


@pytest.mark.parametrize("N,K", [(8, 8), (136, 200), (256, 264), (300, 128)])
def test_weight_partial_blocks(N, K):
    # Each block, partial ones included, is quantized over its own elements:
    # the scale from the exact amax, sampled codes by exact rationals and a
    # brute-force nearest-code search; everything outside [0,N) x [0,K) is +0.
    w = _llama_like(N, K, seed=N + 3 * K)
    wq, ws, wq_t = quant.quantize_weight_128x128(w)
    Nb, Kb = -(-N // 128), -(-K // 128)
    assert wq.shape == (128 * Nb, 128 * Kb) and ws.shape == (Nb, Kb) and wq_t.shape == (128 * Kb, 128 * Nb)
    assert np.all(wq[N:, :] == 0) and np.all(wq[:, K:] == 0)
    assert np.array_equal(wq_t, wq.T)
    wf = e4m3.bf16_bits_to_f32(w)
    rng = np.random.default_rng(N * K)
    for i in range(Nb):
        for j in range(Kb):
            blk = wf[128 * i:min(128 * i + 128, N), 128 * j:min(128 * j + 128, K)]
            amax = max(abs(Fraction(float(v))) for v in blk.ravel())
            s = rn_float32(amax / 448)
            assert Fraction(float(ws[i, j])) == s
            for _ in range(40):
                r, c = rng.integers(0, blk.shape[0]), rng.integers(0, blk.shape[1])
                v = Fraction(float(blk[r, c]))
                code = nearest_e4m3_code(rn_float32(v / s))
                if np.signbit(blk[r, c]) and code == 0:
                    code = 0x80
                elif v < 0:
                    code |= 0x80
                assert wq[128 * i + r, 128 * j + c] == code
    # a block has the same amax transposed, partial blocks included
    wq2, ws2, wq2_t = quant.quantize_weight_128x128(np.ascontiguousarray(w.T))
    assert np.array_equal(wq2, wq.T) and np.array_equal(ws2, ws.T) and np.array_equal(wq2_t, wq)


def test_transpose_identity_with_partial_channel_block():
    # 128x1 groups run along the tokens; a channel count that is not a
    # multiple of 128 changes nothing for them
    x = _llama_like(256, 200, seed=13)
    q1, s1 = quant.quantize_act_1x128(np.ascontiguousarray(x.T))
    qt, st = quant.transpose_quantize_128x1(x)
    assert qt.shape == (200, 256)
    assert np.array_equal(q1, qt) and np.array_equal(s1, st)
