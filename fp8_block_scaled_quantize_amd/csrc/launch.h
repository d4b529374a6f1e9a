// Kernel launchers of the library (internal). Each enqueues on `stream` and
// returns hipGetLastError(); shapes and pointers are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bsq {

hipError_t launch_quant_act_1x128(const void* x, int64_t M, int64_t K, uint8_t* xq, float* xs,
                                  hipStream_t stream);
hipError_t launch_quant_weight_128x128(const void* w, int64_t N, int64_t K, uint8_t* wq, float* ws,
                                       uint8_t* wq_t, hipStream_t stream);
hipError_t launch_transpose_quant_128x1(const void* x, int64_t M, int64_t C, uint8_t* xq_t,
                                        float* xs_t, hipStream_t stream);
hipError_t launch_quant_dual(const void* x, int64_t M, int64_t C, uint8_t* xq, float* xs,
                             uint8_t* xq_t, float* xs_t, hipStream_t stream);
hipError_t launch_rmsnorm_quant(const void* x, const void* gamma, float eps, int64_t M, int64_t K,
                                float* rstd, void* y, uint8_t* xq, float* xs, uint8_t* xq_t,
                                float* xs_t, hipStream_t stream);
hipError_t launch_swiglu_quant(const void* gate, const void* up, int64_t M, int64_t N, void* h,
                               uint8_t* hq, float* hs, uint8_t* hq_t, float* hs_t, hipStream_t stream);
hipError_t launch_cast_f32_e4m3(const float* in, uint8_t* out, int64_t n, hipStream_t stream);

// One GEMM problem in the C ABI's terms (see include/fp8bsq.h): a/as the
// token-major operand and its scales, b/bs the weight-side operand.
struct GemmProblem {
  const uint8_t* a;
  const float* as;
  const uint8_t* b;
  const float* bs;
  void* out;
  int64_t M, N, K;
};
enum class GemmRole { Fwd, Dgrad, Wgrad };
// Several problems of one role in as few launches as possible (16 per launch).
hipError_t launch_gemm_grouped(GemmRole role, const GemmProblem* problems, int count, hipStream_t stream);

// GEMM roles. All three run the same NT kernel family: D[i][j] = sum_k P[i,k] Q[j,k]
// written to out[j][i]; they differ in operands and in how the P scale is indexed.
hipError_t launch_gemm_fwd(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                           void* y, int64_t M, int64_t N, int64_t K, hipStream_t stream);
hipError_t launch_gemm_dgrad(const uint8_t* dyq, const float* dys, const uint8_t* wq_t,
                             const float* ws, void* dx, int64_t M, int64_t N, int64_t K,
                             hipStream_t stream);
hipError_t launch_gemm_wgrad(const uint8_t* dyq_t, const float* dys_t, const uint8_t* xq_t,
                             const float* xs_t, void* dw, int64_t M, int64_t N, int64_t K,
                             hipStream_t stream);

// The 128x128 weight quantizer writing its codes in the weight-streaming
// layout (quantize.hip), that layout made from row-major codes, and the
// forward for at most 64 token rows that reads it (stream.hip).
hipError_t launch_quant_weight_stream(const void* w, int64_t N, int64_t K, uint8_t* wq_s, float* ws,
                                      hipStream_t stream);
hipError_t launch_weight_stream_layout(const uint8_t* wq, int64_t Np, int64_t Kp, uint8_t* wq_s,
                                       hipStream_t stream);
hipError_t launch_gemm_fwd_stream(const uint8_t* xq, const float* xs, const uint8_t* wq_s, const float* ws,
                                  void* y, int64_t M, int64_t N, int64_t K, hipStream_t stream);

}  // namespace fp8bsq
