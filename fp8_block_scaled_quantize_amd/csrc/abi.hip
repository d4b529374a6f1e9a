// The C ABI of the library: argument validation, then the kernel launches.
//
// Every check runs before any HIP runtime call, so an invalid call returns its
// status without touching the device or the stream.
#include <math.h>
#include "../../include/fp8bsq.h"

#include <hip/hip_runtime.h>

#include "launch.h"

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;   // every dimension < 2^31
constexpr int64_t kMaxElems = (int64_t)1 << 40;  // every tensor < 2^40 elements
constexpr int64_t kMaxContraction = (int64_t)1 << 24;  // GEMM contraction length < 2^24
constexpr int64_t kStreamMaxTokens = 64;                // token rows of fp8_gemm_fwd_stream at most
// Weight rows of fp8_gemm_fwd_stream below this: its launch runs at most 256
// threads per 16-row fragment (one fragment per workgroup with three staging
// wavefronts), so the grid stays under 2^32 threads.
constexpr int64_t kStreamMaxRows = (int64_t)1 << 28;

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

bool dims_ok(int64_t a, int64_t b) {
  if (a < 0 || b < 0 || a >= kMaxDim || b >= kMaxDim) return false;
  return a == 0 || b < kMaxElems / a;
}

// A length rounded up to whole 128-element groups: the token length of the
// transposed (128x1) outputs and the padded channel length of the code tensors.
int64_t round128(int64_t m) { return (m + 127) / 128 * 128; }

// Channel dimensions: any multiple of 8 (bf16 rows stay 16-byte aligned).
bool channels_ok(int64_t c) { return c % 8 == 0; }

enum class Role { Fwd, Dgrad, Wgrad };
constexpr int kLaunch = -1;   // check_problem: valid and not empty

// The checks of one GEMM call (the same for a plain and a grouped call):
// an error status, FP8BSQ_OK for an empty output (nothing to do), or kLaunch.
int check_problem(Role role, const fp8bsq_gemm_problem& p) {
  const int64_t M = p.M, N = p.N, K = p.K;
  // contraction length and the two output dimensions of each role
  const int64_t Np = round128(N), Kp = round128(K);
  const int64_t red = role == Role::Fwd ? Kp : role == Role::Dgrad ? Np : M;
  const int64_t o1 = role == Role::Wgrad ? N : M;
  const int64_t o2 = role == Role::Fwd ? N : K;
  if (!dims_ok(M, N) || !dims_ok(M, K) || !dims_ok(N, K) || !dims_ok(M, Np) || !dims_ok(M, Kp) ||
      !dims_ok(Np, Kp) || !channels_ok(N) || !channels_ok(K) || (role == Role::Wgrad && M % 128) ||
      red >= kMaxContraction)
    return FP8BSQ_ERR_SHAPE;
  if (o1 == 0 || o2 == 0) return FP8BSQ_OK;
  if (red == 0) return FP8BSQ_ERR_SHAPE;  // an empty contraction would leave the output unwritten
  if (!p.a || !p.as || !p.b || !p.bs || !p.out) return FP8BSQ_ERR_NULL;
  if (!aligned16(p.a) || !aligned16(p.as) || !aligned16(p.b) || !aligned16(p.bs) || !aligned16(p.out))
    return FP8BSQ_ERR_ALIGN;
  return kLaunch;
}

int hip_status(hipError_t e) { return e == hipSuccess ? FP8BSQ_OK : FP8BSQ_ERR_HIP; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

const char* fp8bsq_strerror(int status) {
  switch (status) {
    case FP8BSQ_OK: return "ok";
    case FP8BSQ_ERR_NULL: return "a required pointer is NULL";
    case FP8BSQ_ERR_SHAPE: return "unsupported shape (negative, too large, or not a multiple of 8 / 128 where required)";
    case FP8BSQ_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case FP8BSQ_ERR_HIP: return "the HIP runtime reported an error at launch";
    case FP8BSQ_ERR_VALUE: return "a scalar argument is out of range";
    default: return "unknown status";
  }
}

int fp8bsq_abi_version(void) { return FP8BSQ_ABI_VERSION; }

int quantize_act_1x128(const void* x, int64_t M, int64_t K, uint8_t* xq, float* xs, void* stream) {
  if (!dims_ok(M, K) || !dims_ok(M, round128(K)) || !channels_ok(K)) return FP8BSQ_ERR_SHAPE;
  if (M == 0 || K == 0) return FP8BSQ_OK;
  if (!x || !xq || !xs) return FP8BSQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(xq) || !aligned16(xs)) return FP8BSQ_ERR_ALIGN;
  return hip_status(fp8bsq::launch_quant_act_1x128(x, M, K, xq, xs, as_stream(stream)));
}

int quantize_weight_128x128(const void* w, int64_t N, int64_t K, uint8_t* wq, float* ws,
                            uint8_t* wq_t, void* stream) {
  if (!dims_ok(N, K) || !dims_ok(round128(N), round128(K)) || !channels_ok(N) || !channels_ok(K))
    return FP8BSQ_ERR_SHAPE;
  if (N == 0 || K == 0) return FP8BSQ_OK;
  if (!w || !wq || !ws) return FP8BSQ_ERR_NULL;
  if (!aligned16(w) || !aligned16(wq) || !aligned16(ws) || (wq_t && !aligned16(wq_t)))
    return FP8BSQ_ERR_ALIGN;
  return hip_status(fp8bsq::launch_quant_weight_128x128(w, N, K, wq, ws, wq_t, as_stream(stream)));
}

int transpose_quantize_128x1(const void* x, int64_t M, int64_t C, uint8_t* xq_t, float* xs_t,
                             void* stream) {
  if (!dims_ok(M, C) || !dims_ok(round128(M), C) || !channels_ok(C)) return FP8BSQ_ERR_SHAPE;
  if (M == 0 || C == 0) return FP8BSQ_OK;
  if (!x || !xq_t || !xs_t) return FP8BSQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(xq_t) || !aligned16(xs_t)) return FP8BSQ_ERR_ALIGN;
  return hip_status(fp8bsq::launch_transpose_quant_128x1(x, M, C, xq_t, xs_t, as_stream(stream)));
}

int quantize_dual_1x128_128x1(const void* x, int64_t M, int64_t K, uint8_t* xq, float* xs,
                              uint8_t* xq_t, float* xs_t, void* stream) {
  if (!dims_ok(M, K) || !dims_ok(round128(M), K) || !dims_ok(M, round128(K)) || !channels_ok(K))
    return FP8BSQ_ERR_SHAPE;
  if (M == 0 || K == 0) return FP8BSQ_OK;
  if (!x || !xq || !xs || !xq_t || !xs_t) return FP8BSQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(xq) || !aligned16(xs) || !aligned16(xq_t) || !aligned16(xs_t))
    return FP8BSQ_ERR_ALIGN;
  return hip_status(fp8bsq::launch_quant_dual(x, M, K, xq, xs, xq_t, xs_t, as_stream(stream)));
}

int rmsnorm_quantize_1x128(const void* x, const void* gamma, float eps, int64_t M, int64_t K,
                           float* rstd, void* y, uint8_t* xq, float* xs, uint8_t* xq_t, float* xs_t,
                           void* stream) {
  const bool tr = xq_t != nullptr || xs_t != nullptr;
  if (!dims_ok(M, K) || !dims_ok(round128(M), K) || !dims_ok(M, round128(K)) || !channels_ok(K))
    return FP8BSQ_ERR_SHAPE;
  if (!(eps >= 0.0f) || eps == INFINITY) return FP8BSQ_ERR_VALUE;
  if (M == 0 || K == 0) return FP8BSQ_OK;
  if (!x || !gamma || !rstd || !xq || !xs || (tr && (!xq_t || !xs_t))) return FP8BSQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(gamma) || !aligned16(xq) || !aligned16(xs) || (y && !aligned16(y)) ||
      (tr && (!aligned16(xq_t) || !aligned16(xs_t))))
    return FP8BSQ_ERR_ALIGN;
  return hip_status(fp8bsq::launch_rmsnorm_quant(x, gamma, eps, M, K, rstd, y, xq, xs, xq_t, xs_t,
                                                 as_stream(stream)));
}

int swiglu_quantize_1x128(const void* gate, const void* up, int64_t M, int64_t N, void* h,
                          uint8_t* hq, float* hs, uint8_t* hq_t, float* hs_t, void* stream) {
  const bool tr = hq_t != nullptr || hs_t != nullptr;
  if (!dims_ok(M, N) || !dims_ok(round128(M), N) || !dims_ok(M, round128(N)) || !channels_ok(N))
    return FP8BSQ_ERR_SHAPE;
  if (M == 0 || N == 0) return FP8BSQ_OK;
  if (!gate || !up || !hq || !hs || (tr && (!hq_t || !hs_t))) return FP8BSQ_ERR_NULL;
  if (!aligned16(gate) || !aligned16(up) || !aligned16(hq) || !aligned16(hs) || (h && !aligned16(h)) ||
      (tr && (!aligned16(hq_t) || !aligned16(hs_t))))
    return FP8BSQ_ERR_ALIGN;
  return hip_status(fp8bsq::launch_swiglu_quant(gate, up, M, N, h, hq, hs, hq_t, hs_t, as_stream(stream)));
}

int fp8_gemm_fwd(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws, void* y,
                 int64_t M, int64_t N, int64_t K, void* stream) {
  const fp8bsq_gemm_problem pr{xq, xs, wq, ws, y, M, N, K};
  const int st = check_problem(Role::Fwd, pr);
  if (st != kLaunch) return st;
  return hip_status(fp8bsq::launch_gemm_fwd(xq, xs, wq, ws, y, M, N, K, as_stream(stream)));
}

int fp8_gemm_dgrad(const uint8_t* dyq, const float* dys, const uint8_t* wq_t, const float* ws,
                   void* dx, int64_t M, int64_t N, int64_t K, void* stream) {
  const fp8bsq_gemm_problem pr{dyq, dys, wq_t, ws, dx, M, N, K};
  const int st = check_problem(Role::Dgrad, pr);
  if (st != kLaunch) return st;
  return hip_status(fp8bsq::launch_gemm_dgrad(dyq, dys, wq_t, ws, dx, M, N, K, as_stream(stream)));
}

int fp8_gemm_wgrad(const uint8_t* dyq_t, const float* dys_t, const uint8_t* xq_t, const float* xs_t,
                   void* dw, int64_t M, int64_t N, int64_t K, void* stream) {
  const fp8bsq_gemm_problem pr{dyq_t, dys_t, xq_t, xs_t, dw, M, N, K};
  const int st = check_problem(Role::Wgrad, pr);
  if (st != kLaunch) return st;
  return hip_status(fp8bsq::launch_gemm_wgrad(dyq_t, dys_t, xq_t, xs_t, dw, M, N, K, as_stream(stream)));
}

static int gemm_grouped(Role role, const fp8bsq_gemm_problem* problems, int count, void* stream) {
  if (count < 0) return FP8BSQ_ERR_SHAPE;
  if (count == 0) return FP8BSQ_OK;
  if (!problems) return FP8BSQ_ERR_NULL;
  int live = 0;
  for (int g = 0; g < count; ++g) {         // every problem is checked before any launch
    const int st = check_problem(role, problems[g]);
    if (st == kLaunch) ++live;
    else if (st != FP8BSQ_OK) return st;
  }
  if (live == 0) return FP8BSQ_OK;
  fp8bsq::GemmProblem buf[64];
  const fp8bsq::GemmRole r = role == Role::Fwd ? fp8bsq::GemmRole::Fwd
                             : role == Role::Dgrad ? fp8bsq::GemmRole::Dgrad : fp8bsq::GemmRole::Wgrad;
  int n = 0;
  for (int g = 0; g < count; ++g) {
    const fp8bsq_gemm_problem& p = problems[g];
    if (check_problem(role, p) != kLaunch) continue;
    buf[n++] = fp8bsq::GemmProblem{p.a, p.as, p.b, p.bs, p.out, p.M, p.N, p.K};
    if (n == 64) {
      const int st = hip_status(fp8bsq::launch_gemm_grouped(r, buf, n, as_stream(stream)));
      if (st != FP8BSQ_OK) return st;
      n = 0;
    }
  }
  return n ? hip_status(fp8bsq::launch_gemm_grouped(r, buf, n, as_stream(stream))) : FP8BSQ_OK;
}

int fp8_gemm_fwd_grouped(const fp8bsq_gemm_problem* problems, int count, void* stream) {
  return gemm_grouped(Role::Fwd, problems, count, stream);
}

int fp8_gemm_dgrad_grouped(const fp8bsq_gemm_problem* problems, int count, void* stream) {
  return gemm_grouped(Role::Dgrad, problems, count, stream);
}

int fp8_gemm_wgrad_grouped(const fp8bsq_gemm_problem* problems, int count, void* stream) {
  return gemm_grouped(Role::Wgrad, problems, count, stream);
}

int quantize_weight_128x128_stream(const void* w, int64_t N, int64_t K, uint8_t* wq_s, float* ws, void* stream) {
  if (!dims_ok(N, K) || !dims_ok(round128(N), round128(K)) || !channels_ok(N) || !channels_ok(K))
    return FP8BSQ_ERR_SHAPE;
  if (N == 0 || K == 0) return FP8BSQ_OK;
  if (!w || !wq_s || !ws) return FP8BSQ_ERR_NULL;
  if (!aligned16(w) || !aligned16(wq_s) || !aligned16(ws)) return FP8BSQ_ERR_ALIGN;
  return hip_status(fp8bsq::launch_quant_weight_stream(w, N, K, wq_s, ws, as_stream(stream)));
}

int fp8_weight_stream_layout(const uint8_t* wq, int64_t N, int64_t K, uint8_t* wq_s, void* stream) {
  if (!dims_ok(N, K) || !dims_ok(round128(N), round128(K)) || !channels_ok(N) || !channels_ok(K))
    return FP8BSQ_ERR_SHAPE;
  if (N == 0 || K == 0) return FP8BSQ_OK;
  if (!wq || !wq_s) return FP8BSQ_ERR_NULL;
  if (!aligned16(wq) || !aligned16(wq_s)) return FP8BSQ_ERR_ALIGN;
  return hip_status(fp8bsq::launch_weight_stream_layout(wq, round128(N), round128(K), wq_s, as_stream(stream)));
}

int fp8_gemm_fwd_stream(const uint8_t* xq, const float* xs, const uint8_t* wq_s, const float* ws, void* y,
                        int64_t M, int64_t N, int64_t K, void* stream) {
  const fp8bsq_gemm_problem pr{xq, xs, wq_s, ws, y, M, N, K};
  if (M > kStreamMaxTokens || N >= kStreamMaxRows) return FP8BSQ_ERR_SHAPE;
  const int st = check_problem(Role::Fwd, pr);
  if (st != kLaunch) return st;
  return hip_status(fp8bsq::launch_gemm_fwd_stream(xq, xs, wq_s, ws, y, M, N, K, as_stream(stream)));
}

int fp8bsq_cast_f32_e4m3(const float* in, uint8_t* out, int64_t n, void* stream) {
  if (n < 0 || n >= kMaxElems || n % 4) return FP8BSQ_ERR_SHAPE;
  if (n == 0) return FP8BSQ_OK;
  if (!in || !out) return FP8BSQ_ERR_NULL;
  if (!aligned16(in) || !aligned16(out)) return FP8BSQ_ERR_ALIGN;
  return hip_status(fp8bsq::launch_cast_f32_e4m3(in, out, n, as_stream(stream)));
}

}  // extern "C"
