"""The C-ABI library without a GPU: it loads, exports every declared symbol,
and rejects invalid arguments with the documented status before any HIP call."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8bsq.h")
LIB = os.path.join(ROOT, "fp8_block_scaled_quantize_amd", "libfp8bsq.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from fp8_block_scaled_quantize_amd.build import build
        build()
    return ctypes.CDLL(LIB)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M)


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) >= {"quantize_act_1x128", "quantize_weight_128x128", "transpose_quantize_128x1",
                          "quantize_dual_1x128_128x1", "rmsnorm_quantize_1x128", "swiglu_quantize_1x128",
                          "fp8_gemm_fwd", "fp8_gemm_fwd_grouped", "fp8_gemm_dgrad_grouped",
                          "fp8_gemm_wgrad_grouped", "fp8_gemm_dgrad", "fp8_gemm_wgrad",
                          "fp8bsq_strerror", "fp8bsq_abi_version", "fp8bsq_cast_f32_e4m3",
                          "fp8_weight_stream_layout", "fp8_gemm_fwd_stream", "quantize_weight_128x128_stream"}
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strerror(lib):
    lib.fp8bsq_abi_version.restype = ctypes.c_int
    assert lib.fp8bsq_abi_version() == 7
    lib.fp8bsq_strerror.restype = ctypes.c_char_p
    lib.fp8bsq_strerror.argtypes = [ctypes.c_int]
    for code in range(5):
        assert lib.fp8bsq_strerror(code)
    assert lib.fp8bsq_strerror(99) == b"unknown status"


P = ctypes.c_void_p
I64 = ctypes.c_int64
FAKE = P(0x10000)        # aligned, never dereferenced: validation fails first or no launch happens
MISALIGNED = P(0x10008)


def test_quantizer_validation(lib):
    q = lib.quantize_act_1x128
    q.argtypes = [P, I64, I64, P, P, P]
    assert q(FAKE, 4, 100, FAKE, FAKE, None) == 2          # K not a multiple of 8
    assert q(None, 4, 200, FAKE, FAKE, None) == 1          # a partial channel group passes the shape check
    assert q(FAKE, -1, 128, FAKE, FAKE, None) == 2         # negative
    assert q(FAKE, 1 << 31, 128, FAKE, FAKE, None) == 2    # too large
    assert q(None, 4, 128, FAKE, FAKE, None) == 1          # null
    assert q(FAKE, 4, 128, MISALIGNED, FAKE, None) == 3    # misaligned
    assert q(None, 0, 128, None, None, None) == 0          # empty: no-op
    w = lib.quantize_weight_128x128
    w.argtypes = [P, I64, I64, P, P, P, P]
    assert w(FAKE, 100, 128, FAKE, FAKE, None, None) == 2
    assert w(FAKE, 136, 200, None, FAKE, None, None) == 1  # partial blocks pass the shape check
    assert w(FAKE, 128, 128, None, FAKE, None, None) == 1
    assert w(FAKE, 128, 128, FAKE, FAKE, MISALIGNED, None) == 3
    t = lib.transpose_quantize_128x1
    t.argtypes = [P, I64, I64, P, P, P]
    assert t(FAKE, 64, 60, FAKE, FAKE, None) == 2          # C a multiple of 8 (any M)
    assert t(None, 64, 64, FAKE, FAKE, None) == 1          # C = 64 passes the shape check
    assert t(FAKE, (1 << 31) - 100, 128, FAKE, FAKE, None) == 2   # M rounded up to 128 is too large
    assert t(None, 64, 128, FAKE, FAKE, None) == 1         # a ragged M passes the shape check
    assert t(FAKE, 128, 128, FAKE, None, None) == 1
    c = lib.fp8bsq_cast_f32_e4m3
    c.argtypes = [P, P, I64, P]
    assert c(FAKE, FAKE, 6, None) == 2
    assert c(None, FAKE, 8, None) == 1


def test_dual_quantizer_validation(lib):
    d = lib.quantize_dual_1x128_128x1
    d.argtypes = [P, I64, I64, P, P, P, P, P]
    d.restype = ctypes.c_int
    assert d(None, 64, 128, FAKE, FAKE, FAKE, FAKE, None) == 1        # a ragged M passes the shape check
    assert d(FAKE, 128, 100, FAKE, FAKE, FAKE, FAKE, None) == 2       # channels a multiple of 8
    assert d(None, 128, 96, FAKE, FAKE, FAKE, FAKE, None) == 1        # 96 channels pass the shape check
    assert d(FAKE, -128, 128, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert d(FAKE, 128, 128, FAKE, FAKE, None, FAKE, None) == 1       # every output is required
    assert d(FAKE, 128, 128, FAKE, FAKE, FAKE, MISALIGNED, None) == 3
    assert d(None, 0, 128, None, None, None, None, None) == 0         # empty: no-op


def test_fused_producer_validation(lib):
    r = lib.rmsnorm_quantize_1x128
    r.argtypes = [P, P, ctypes.c_float, I64, I64, P, P, P, P, P, P, P]
    r.restype = ctypes.c_int
    assert r(FAKE, FAKE, 1e-6, 3, 100, FAKE, None, FAKE, FAKE, None, None, None) == 2   # K % 8
    assert r(None, FAKE, 1e-6, 3, 96, FAKE, None, FAKE, FAKE, None, None, None) == 1    # K = 96 passes
    assert r(None, FAKE, 1e-6, 3, 128, FAKE, None, FAKE, FAKE, FAKE, FAKE, None) == 1   # ragged M with transposed outputs
    assert r(FAKE, FAKE, -1.0, 3, 128, FAKE, None, FAKE, FAKE, None, None, None) == 5   # eps < 0
    assert r(FAKE, FAKE, float("nan"), 3, 128, FAKE, None, FAKE, FAKE, None, None, None) == 5
    assert r(FAKE, FAKE, float("inf"), 3, 128, FAKE, None, FAKE, FAKE, None, None, None) == 5
    assert r(FAKE, FAKE, 1e-6, 3, 128, None, None, FAKE, FAKE, None, None, None) == 1   # rstd required
    assert r(FAKE, FAKE, 1e-6, 128, 128, FAKE, None, FAKE, FAKE, FAKE, None, None) == 1 # half of the transposed pair
    assert r(FAKE, MISALIGNED, 1e-6, 3, 128, FAKE, None, FAKE, FAKE, None, None, None) == 3
    assert r(None, None, 1e-6, 0, 128, None, None, None, None, None, None, None) == 0    # empty
    w = lib.swiglu_quantize_1x128
    w.argtypes = [P, P, I64, I64, P, P, P, P, P, P]
    w.restype = ctypes.c_int
    assert w(FAKE, FAKE, 5, 100, None, FAKE, FAKE, None, None, None) == 2
    assert w(FAKE, None, 5, 128, None, FAKE, FAKE, FAKE, FAKE, None) == 1     # ragged M with transposed outputs
    assert w(FAKE, None, 5, 128, None, FAKE, FAKE, None, None, None) == 1
    assert w(FAKE, FAKE, 5, 128, MISALIGNED, FAKE, FAKE, None, None, None) == 3
    assert w(None, None, 0, 128, None, None, None, None, None, None) == 0
    lib.fp8bsq_strerror.restype = ctypes.c_char_p
    lib.fp8bsq_strerror.argtypes = [ctypes.c_int]
    assert b"out of range" in lib.fp8bsq_strerror(5)


def test_gemm_validation(lib):
    for name in ("fp8_gemm_fwd", "fp8_gemm_dgrad", "fp8_gemm_wgrad"):
        f = getattr(lib, name)
        f.argtypes = [P, P, P, P, P, I64, I64, I64, P]
        f.restype = ctypes.c_int
        assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 128, 100, 128, None) == 2, name
        assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 128, 128, 100, None) == 2, name
        assert f(FAKE, FAKE, None, FAKE, FAKE, 128, 136, 200, None) == 1, name  # partial groups pass
        assert f(FAKE, FAKE, None, FAKE, FAKE, 128, 128, 128, None) == 1, name
        assert f(FAKE, FAKE, FAKE, FAKE, MISALIGNED, 128, 128, 128, None) == 3, name
    f = lib.fp8_gemm_wgrad
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 128, 128, None) == 2   # token dim grouped by 128
    f = lib.fp8_gemm_fwd
    assert f(None, None, None, None, None, 0, 128, 128, None) == 0    # M == 0: no-op
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 128, 0, None) == 2      # empty contraction
    # contraction length below 2^24 (checked before the pointers)
    big = 1 << 24
    assert f(None, FAKE, FAKE, FAKE, FAKE, 1, 128, big - 128, None) == 1
    assert f(None, FAKE, FAKE, FAKE, FAKE, 1, 128, big, None) == 2
    assert lib.fp8_gemm_dgrad(None, FAKE, FAKE, FAKE, FAKE, 1, big - 128, 128, None) == 1
    assert lib.fp8_gemm_dgrad(None, FAKE, FAKE, FAKE, FAKE, 1, big, 128, None) == 2
    assert lib.fp8_gemm_wgrad(None, FAKE, FAKE, FAKE, FAKE, big - 128, 128, 128, None) == 1
    assert lib.fp8_gemm_wgrad(None, FAKE, FAKE, FAKE, FAKE, big, 128, 128, None) == 2


def test_grouped_gemm_validation(lib):
    import fp8_block_scaled_quantize_amd as fq
    lib2 = fq.load_library()
    arr = (fq.GemmProblem * 3)()
    good = (0x10000, 0x10000, 0x10000, 0x10000, 0x10000)
    arr[1] = fq.GemmProblem(*good, 128, 128, 100)           # bad K: the whole call fails
    arr[2] = fq.GemmProblem(*good, 128, 128, 128)
    for name, empty in (("fp8_gemm_fwd_grouped", (0, 128, 128)), ("fp8_gemm_dgrad_grouped", (0, 128, 128)),
                        ("fp8_gemm_wgrad_grouped", (128, 0, 128))):
        arr[0] = fq.GemmProblem(*good, *empty)              # empty output: skipped
        f = getattr(lib2, name)
        assert f(arr, 3, None) == 2, name                   # checked before any launch
        assert f(arr, 1, None) == 0, name                   # only empty problems: no-op
        assert f(None, 2, None) == 1, name
        assert f(arr, -1, None) == 2, name
        assert f(None, 0, None) == 0, name
    arr[1] = fq.GemmProblem(0x10000, 0x10000, None, 0x10000, 0x10000, 128, 128, 128)
    assert lib2.fp8_gemm_wgrad_grouped(arr, 3, None) == 1   # a null operand in the second problem
    arr[1] = fq.GemmProblem(0x10000, 0x10000, 0x10008, 0x10000, 0x10000, 128, 128, 128)
    assert lib2.fp8_gemm_fwd_grouped(arr, 2, None) == 3


def test_binding_has_no_cpu_fallback():
    """The product package never imports the oracle and has no CPU compute path."""
    pkg = os.path.join(ROOT, "fp8_block_scaled_quantize_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, fn)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle|import_module\(.oracle|oracle\.", text, re.M), fn


def test_stream_layout_validation(lib):
    q = lib.quantize_weight_128x128_stream
    q.argtypes = [P, I64, I64, P, P, P]
    q.restype = ctypes.c_int
    assert q(FAKE, 100, 128, FAKE, FAKE, None) == 2           # N a multiple of 8
    assert q(None, 136, 200, FAKE, FAKE, None) == 1           # partial blocks pass the shape check
    assert q(FAKE, 128, 128, FAKE, None, None) == 1
    assert q(FAKE, 128, 128, MISALIGNED, FAKE, None) == 3
    assert q(None, 0, 128, None, None, None) == 0             # empty: no-op
    s = lib.fp8_weight_stream_layout
    s.argtypes = [P, I64, I64, P, P]
    s.restype = ctypes.c_int
    assert s(FAKE, 128, 100, FAKE, None) == 2
    assert s(FAKE, 128, 128, None, None) == 1
    assert s(MISALIGNED, 128, 128, FAKE, None) == 3
    assert s(None, 128, 0, None, None) == 0
    f = lib.fp8_gemm_fwd_stream
    f.argtypes = [P, P, P, P, P, I64, I64, I64, P]
    f.restype = ctypes.c_int
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 65, 128, 128, None) == 2    # at most 64 token rows
    assert f(None, FAKE, FAKE, FAKE, FAKE, 64, 128, 128, None) == 1    # 64 rows pass the shape check
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 100, 128, None) == 2
    assert f(FAKE, FAKE, FAKE, FAKE, MISALIGNED, 1, 128, 128, None) == 3
    assert f(None, None, None, None, None, 0, 128, 128, None) == 0     # M == 0: no-op
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 128, 0, None) == 2       # empty contraction
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1 << 28, 128, None) == 2  # weight rows < 2^28 (launch size)
    assert f(None, FAKE, FAKE, FAKE, FAKE, 1, (1 << 28) - 8, 128, None) == 1
