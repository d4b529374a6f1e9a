"""MI355X (gfx950) FP8 block-scaled linear-layer library: Python binding.

A thin ctypes layer over the C ABI of ``libfp8bsq.so`` (declared in
``include/fp8bsq.h``). It only marshals arguments: it takes torch tensors that
live in HIP device memory, checks dtype/shape/contiguity, allocates outputs
with ``torch.empty`` when the caller does not pass them, and hands raw device
pointers plus the current HIP stream to the library. Every step of the
computation runs in the library's HIP kernels; there is no fallback. If the
library is missing, every call raises.

Entry points (same names as the C ABI; Kp, Np, Mp are K, N, M rounded up to
a multiple of 128, Kg = Kp/128; channel counts are any multiple of 8):
    quantize_act_1x128(x)             -> (xq [M,Kp] uint8, xs [M,Kg] float32)
    quantize_weight_128x128(w, transposed=True)
                                      -> (wq [Np,Kp], ws [Ng,Kg], wq_t [Kp,Np] or None)
    transpose_quantize_128x1(x)       -> (xq_t [C,Mp], xs_t [C,Mp/128])
    quantize_dual_1x128_128x1(x)      -> (xq, xs, xq_t, xs_t): both of the above, one read of x
    rmsnorm_quantize_1x128(x, gamma, eps, transposed=False, write_y=False)
                                      -> (xq, xs, xq_t, xs_t, rstd, y): RMSNorm, its output quantized
    swiglu_quantize_1x128(gate, up, transposed=False, write_h=False)
                                      -> (hq, hs, hq_t, hs_t, h): silu(gate)*up, quantized
    fp8_gemm_fwd(xq, xs, wq, ws, n=None)      -> y  [M,N] bf16   (Y = X W^T; N defaults to Np)
    fp8_gemm_dgrad(dyq, dys, wq_t, ws, k=None) -> dx [M,K] bf16  (dX = dY W; K defaults to Kp)
    fp8_gemm_wgrad(dyq_t, dys_t, xq_t, xs_t)  -> dw [N,K] bf16   (dW = dY^T X)
    quantize_weight_128x128_stream(w) -> (wq_s, ws): the weight codes in the streaming layout
    weight_stream_layout(wq)          -> wq_s: row-major codes rearranged for streaming
    fp8_gemm_fwd_stream(xq, xs, wq_s, ws, n=None) -> y [M,N] bf16 (M <= 64; equals fp8_gemm_fwd)
    fp8_gemm_{fwd,dgrad,wgrad}_grouped(problems, outs=None)
                                      -> list of outputs; each problem is the tuple of
                                         tensors the plain call takes (fwd / dgrad: plus,
                                         optionally, n / k), all in one launch
    cast_f32_e4m3(v)                  -> E4M3 bytes of fp32 values
E4M3 codes are returned as uint8 tensors (OCP E4M3 bytes); view them as
``torch.float8_e4m3fn`` if needed. Every function accepts preallocated
outputs through keyword arguments (``out=...``) and never synchronizes.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8bsq.so")

_lib = None


class GemmProblem(ctypes.Structure):
    """One problem of a grouped GEMM call (the C ABI's fp8bsq_gemm_problem)."""
    _fields_ = [("a", ctypes.c_void_p), ("as_", ctypes.c_void_p), ("b", ctypes.c_void_p),
                ("bs", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64)]


class Fp8bsqError(RuntimeError):
    """A C-ABI call returned a non-zero status."""

    def __init__(self, fn, status, message):
        super().__init__(f"{fn}: status {status}: {message}")
        self.status = status


def library_path():
    return LIB_PATH


def load_library():
    """Load libfp8bsq.so (after torch, so its HIP runtime is the one in use)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  -- loads torch's libamdhip64 first; the library binds to it by soname

    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m fp8_block_scaled_quantize_amd.build` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    sigs = {
        "fp8bsq_strerror": ([i32], ctypes.c_char_p),
        "fp8bsq_abi_version": ([], i32),
        "quantize_act_1x128": ([vp, i64, i64, vp, vp, vp], i32),
        "quantize_weight_128x128": ([vp, i64, i64, vp, vp, vp, vp], i32),
        "transpose_quantize_128x1": ([vp, i64, i64, vp, vp, vp], i32),
        "quantize_dual_1x128_128x1": ([vp, i64, i64, vp, vp, vp, vp, vp], i32),
        "rmsnorm_quantize_1x128": ([vp, vp, ctypes.c_float, i64, i64, vp, vp, vp, vp, vp, vp, vp], i32),
        "swiglu_quantize_1x128": ([vp, vp, i64, i64, vp, vp, vp, vp, vp, vp], i32),
        "fp8_gemm_fwd": ([vp, vp, vp, vp, vp, i64, i64, i64, vp], i32),
        "fp8_gemm_dgrad": ([vp, vp, vp, vp, vp, i64, i64, i64, vp], i32),
        "fp8_gemm_wgrad": ([vp, vp, vp, vp, vp, i64, i64, i64, vp], i32),
        "fp8bsq_cast_f32_e4m3": ([vp, vp, i64, vp], i32),
        "quantize_weight_128x128_stream": ([vp, i64, i64, vp, vp, vp], i32),
        "fp8_weight_stream_layout": ([vp, i64, i64, vp, vp], i32),
        "fp8_gemm_fwd_stream": ([vp, vp, vp, vp, vp, i64, i64, i64, vp], i32),
        "fp8_gemm_fwd_grouped": ([ctypes.POINTER(GemmProblem), i32, vp], i32),
        "fp8_gemm_dgrad_grouped": ([ctypes.POINTER(GemmProblem), i32, vp], i32),
        "fp8_gemm_wgrad_grouped": ([ctypes.POINTER(GemmProblem), i32, vp], i32),
    }
    for name, (args, res) in sigs.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def strerror(status):
    return load_library().fp8bsq_strerror(int(status)).decode()


def _check(fn, status):
    if status != 0:
        raise Fp8bsqError(fn, status, strerror(status))


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _need(t, name, dtype, shape):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be in GPU memory, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _out(t, name, dtype, shape, like):
    import torch
    if t is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    return _need(t, name, dtype, shape)


def padded(n):
    """A length rounded up to whole 128-element groups: the grouped dimension of
    the code tensors (and the token length of the 128x1 outputs)."""
    return (n + 127) // 128 * 128


def quantize_act_1x128(x, xq=None, xs=None):
    import torch
    M, K = x.shape
    Kp = padded(K)
    _need(x, "x", torch.bfloat16, (M, K))
    xq = _out(xq, "xq", torch.uint8, (M, Kp), x)
    xs = _out(xs, "xs", torch.float32, (M, Kp // 128), x)
    _check("quantize_act_1x128", load_library().quantize_act_1x128(
        _ptr(x), M, K, _ptr(xq), _ptr(xs), _stream(x)))
    return xq, xs


def quantize_weight_128x128(w, transposed=True, wq=None, ws=None, wq_t=None):
    import torch
    N, K = w.shape
    Np, Kp = padded(N), padded(K)
    _need(w, "w", torch.bfloat16, (N, K))
    wq = _out(wq, "wq", torch.uint8, (Np, Kp), w)
    ws = _out(ws, "ws", torch.float32, (Np // 128, Kp // 128), w)
    if transposed:
        wq_t = _out(wq_t, "wq_t", torch.uint8, (Kp, Np), w)
    else:
        wq_t = None
    _check("quantize_weight_128x128", load_library().quantize_weight_128x128(
        _ptr(w), N, K, _ptr(wq), _ptr(ws), _ptr(wq_t), _stream(w)))
    return wq, ws, wq_t


def padded_tokens(M):
    """Token length of the 128x1 (transposed) outputs: M rounded up to 128."""
    return padded(M)


def transpose_quantize_128x1(x, xq_t=None, xs_t=None):
    import torch
    M, C = x.shape
    Mp = padded_tokens(M)
    _need(x, "x", torch.bfloat16, (M, C))
    xq_t = _out(xq_t, "xq_t", torch.uint8, (C, Mp), x)
    xs_t = _out(xs_t, "xs_t", torch.float32, (C, Mp // 128), x)
    _check("transpose_quantize_128x1", load_library().transpose_quantize_128x1(
        _ptr(x), M, C, _ptr(xq_t), _ptr(xs_t), _stream(x)))
    return xq_t, xs_t


def quantize_dual_1x128_128x1(x, xq=None, xs=None, xq_t=None, xs_t=None):
    import torch
    M, K = x.shape
    Kp = padded(K)
    _need(x, "x", torch.bfloat16, (M, K))
    xq = _out(xq, "xq", torch.uint8, (M, Kp), x)
    xs = _out(xs, "xs", torch.float32, (M, Kp // 128), x)
    Mp = padded_tokens(M)
    xq_t = _out(xq_t, "xq_t", torch.uint8, (K, Mp), x)
    xs_t = _out(xs_t, "xs_t", torch.float32, (K, Mp // 128), x)
    _check("quantize_dual_1x128_128x1", load_library().quantize_dual_1x128_128x1(
        _ptr(x), M, K, _ptr(xq), _ptr(xs), _ptr(xq_t), _ptr(xs_t), _stream(x)))
    return xq, xs, xq_t, xs_t


def rmsnorm_quantize_1x128(x, gamma, eps=1e-6, transposed=False, write_y=False,
                           xq=None, xs=None, xq_t=None, xs_t=None, rstd=None, y=None):
    import torch
    M, K = x.shape
    _need(x, "x", torch.bfloat16, (M, K))
    _need(gamma, "gamma", torch.bfloat16, (K,))
    xq = _out(xq, "xq", torch.uint8, (M, padded(K)), x)
    xs = _out(xs, "xs", torch.float32, (M, padded(K) // 128), x)
    rstd = _out(rstd, "rstd", torch.float32, (M,), x)
    if transposed:
        xq_t = _out(xq_t, "xq_t", torch.uint8, (K, padded_tokens(M)), x)
        xs_t = _out(xs_t, "xs_t", torch.float32, (K, padded_tokens(M) // 128), x)
    else:
        xq_t = xs_t = None
    y = _out(y, "y", torch.bfloat16, (M, K), x) if write_y else None
    _check("rmsnorm_quantize_1x128", load_library().rmsnorm_quantize_1x128(
        _ptr(x), _ptr(gamma), float(eps), M, K, _ptr(rstd), _ptr(y), _ptr(xq), _ptr(xs),
        _ptr(xq_t), _ptr(xs_t), _stream(x)))
    return xq, xs, xq_t, xs_t, rstd, y


def swiglu_quantize_1x128(gate, up, transposed=False, write_h=False,
                          hq=None, hs=None, hq_t=None, hs_t=None, h=None):
    import torch
    M, N = gate.shape
    _need(gate, "gate", torch.bfloat16, (M, N))
    _need(up, "up", torch.bfloat16, (M, N))
    hq = _out(hq, "hq", torch.uint8, (M, padded(N)), gate)
    hs = _out(hs, "hs", torch.float32, (M, padded(N) // 128), gate)
    if transposed:
        hq_t = _out(hq_t, "hq_t", torch.uint8, (N, padded_tokens(M)), gate)
        hs_t = _out(hs_t, "hs_t", torch.float32, (N, padded_tokens(M) // 128), gate)
    else:
        hq_t = hs_t = None
    h = _out(h, "h", torch.bfloat16, (M, N), gate) if write_h else None
    _check("swiglu_quantize_1x128", load_library().swiglu_quantize_1x128(
        _ptr(gate), _ptr(up), M, N, _ptr(h), _ptr(hq), _ptr(hs), _ptr(hq_t), _ptr(hs_t), _stream(gate)))
    return hq, hs, hq_t, hs_t, h


def _cols(n, npad, name):
    """Logical column count of a GEMM output whose code tensors are padded to npad."""
    n = npad if n is None else int(n)
    if padded(n) != npad:
        raise ValueError(f"{name}={n} does not round up to the padded length {npad} of the codes")
    return n


def fp8_gemm_fwd(xq, xs, wq, ws, out=None, n=None):
    """Y [M, N] = Xq Wq^T; n is the weight's logical row count N (default: wq's rows)."""
    import torch
    M, Kp = xq.shape
    Np = wq.shape[0]
    N = _cols(n, Np, "n")
    _need(xq, "xq", torch.uint8, (M, Kp))
    _need(xs, "xs", torch.float32, (M, Kp // 128))
    _need(wq, "wq", torch.uint8, (Np, Kp))
    _need(ws, "ws", torch.float32, (Np // 128, Kp // 128))
    y = _out(out, "out", torch.bfloat16, (M, N), xq)
    _check("fp8_gemm_fwd", load_library().fp8_gemm_fwd(
        _ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), _ptr(y), M, N, Kp, _stream(xq)))
    return y


def fp8_gemm_dgrad(dyq, dys, wq_t, ws, out=None, k=None):
    """dX [M, K] = dYq Wq; k is the weight's logical column count K (default: wq_t's rows)."""
    import torch
    M, Np = dyq.shape
    Kp = wq_t.shape[0]
    K = _cols(k, Kp, "k")
    _need(dyq, "dyq", torch.uint8, (M, Np))
    _need(dys, "dys", torch.float32, (M, Np // 128))
    _need(wq_t, "wq_t", torch.uint8, (Kp, Np))
    _need(ws, "ws", torch.float32, (Np // 128, Kp // 128))
    dx = _out(out, "out", torch.bfloat16, (M, K), dyq)
    _check("fp8_gemm_dgrad", load_library().fp8_gemm_dgrad(
        _ptr(dyq), _ptr(dys), _ptr(wq_t), _ptr(ws), _ptr(dx), M, Np, K, _stream(dyq)))
    return dx


def fp8_gemm_wgrad(dyq_t, dys_t, xq_t, xs_t, out=None):
    import torch
    N, M = dyq_t.shape
    K = xq_t.shape[0]
    _need(dyq_t, "dyq_t", torch.uint8, (N, M))
    _need(dys_t, "dys_t", torch.float32, (N, M // 128))
    _need(xq_t, "xq_t", torch.uint8, (K, M))
    _need(xs_t, "xs_t", torch.float32, (K, M // 128))
    dw = _out(out, "out", torch.bfloat16, (N, K), dyq_t)
    _check("fp8_gemm_wgrad", load_library().fp8_gemm_wgrad(
        _ptr(dyq_t), _ptr(dys_t), _ptr(xq_t), _ptr(xs_t), _ptr(dw), M, N, K, _stream(dyq_t)))
    return dw


def _grouped(role, problems, outs):
    """Shared marshalling of the grouped GEMMs: validate like the plain calls,
    allocate outputs, pass one array of problems."""
    import torch
    arr = (GemmProblem * max(1, len(problems)))()
    results = []
    for g, prob in enumerate(problems):
        a, as_, b, bs = prob[:4]
        cols = prob[4] if len(prob) > 4 else None
        if role == "fwd":
            M, K = a.shape
            Np = b.shape[0]
            N = _cols(cols, Np, "n")
            _need(a, "xq", torch.uint8, (M, K)); _need(as_, "xs", torch.float32, (M, K // 128))
            _need(b, "wq", torch.uint8, (Np, K)); _need(bs, "ws", torch.float32, (Np // 128, K // 128))
            shape = (M, N)
        elif role == "dgrad":
            M, N = a.shape
            Kp = b.shape[0]
            K = _cols(cols, Kp, "k")
            _need(a, "dyq", torch.uint8, (M, N)); _need(as_, "dys", torch.float32, (M, N // 128))
            _need(b, "wq_t", torch.uint8, (Kp, N)); _need(bs, "ws", torch.float32, (N // 128, Kp // 128))
            shape = (M, K)
        else:
            N, M = a.shape
            K = b.shape[0]
            _need(a, "dyq_t", torch.uint8, (N, M)); _need(as_, "dys_t", torch.float32, (N, M // 128))
            _need(b, "xq_t", torch.uint8, (K, M)); _need(bs, "xs_t", torch.float32, (K, M // 128))
            shape = (N, K)
        out = _out(None if outs is None else outs[g], "out", torch.bfloat16, shape, a)
        results.append(out)
        arr[g] = GemmProblem(a.data_ptr(), as_.data_ptr(), b.data_ptr(), bs.data_ptr(), out.data_ptr(), M, N, K)
    if not problems:
        return results
    fn = getattr(load_library(), f"fp8_gemm_{role}_grouped")
    _check(f"fp8_gemm_{role}_grouped", fn(arr, len(problems), _stream(problems[0][0])))
    return results


def fp8_gemm_fwd_grouped(problems, outs=None):
    """problems: [(xq, xs, wq, ws), ...] -> [y, ...] in one launch."""
    return _grouped("fwd", problems, outs)


def fp8_gemm_dgrad_grouped(problems, outs=None):
    """problems: [(dyq, dys, wq_t, ws), ...] -> [dx, ...] in one launch."""
    return _grouped("dgrad", problems, outs)


def fp8_gemm_wgrad_grouped(problems, outs=None):
    """problems: [(dyq_t, dys_t, xq_t, xs_t), ...] -> [dw, ...] in one launch."""
    return _grouped("wgrad", problems, outs)


def quantize_weight_128x128_stream(w, wq_s=None, ws=None):
    """W [N, K] bf16 -> (wq_s [Np, Kp] u8 codes in the weight-streaming layout,
    ws [Ng, Kg] f32), for fp8_gemm_fwd_stream."""
    import torch
    N, K = w.shape
    _need(w, "w", torch.bfloat16, (N, K))
    wq_s = _out(wq_s, "wq_s", torch.uint8, (padded(N), padded(K)), w)
    ws = _out(ws, "ws", torch.float32, (padded(N) // 128, padded(K) // 128), w)
    _check("quantize_weight_128x128_stream", load_library().quantize_weight_128x128_stream(
        _ptr(w), N, K, _ptr(wq_s), _ptr(ws), _stream(w)))
    return wq_s, ws


def weight_stream_layout(wq, out=None):
    """wq [Np, Kp] codes -> the same codes in the weight-streaming layout
    (a uint8 tensor of the same shape; its bytes are arranged as
    include/fp8bsq.h describes, not row-major)."""
    import torch
    Np, Kp = wq.shape
    _need(wq, "wq", torch.uint8, (Np, Kp))
    o = _out(out, "out", torch.uint8, (Np, Kp), wq)
    _check("fp8_weight_stream_layout", load_library().fp8_weight_stream_layout(
        _ptr(wq), Np, Kp, _ptr(o), _stream(wq)))
    return o


def fp8_gemm_fwd_stream(xq, xs, wq_s, ws, out=None, n=None):
    """Y [M, N] = Xq Wq^T for M <= 64 tokens, the weight in its stream layout
    (bit-identical to fp8_gemm_fwd on wq)."""
    import torch
    M, Kp = xq.shape
    Np = wq_s.shape[0]
    N = _cols(n, Np, "n")
    _need(xq, "xq", torch.uint8, (M, Kp))
    _need(xs, "xs", torch.float32, (M, Kp // 128))
    _need(wq_s, "wq_s", torch.uint8, (Np, Kp))
    _need(ws, "ws", torch.float32, (Np // 128, Kp // 128))
    y = _out(out, "out", torch.bfloat16, (M, N), xq)
    _check("fp8_gemm_fwd_stream", load_library().fp8_gemm_fwd_stream(
        _ptr(xq), _ptr(xs), _ptr(wq_s), _ptr(ws), _ptr(y), M, N, Kp, _stream(xq)))
    return y


def cast_f32_e4m3(v, out=None):
    import torch
    (n,) = v.shape
    _need(v, "v", torch.float32, (n,))
    o = _out(out, "out", torch.uint8, (n,), v)
    _check("fp8bsq_cast_f32_e4m3", load_library().fp8bsq_cast_f32_e4m3(
        _ptr(v), _ptr(o), n, _stream(v)))
    return o
