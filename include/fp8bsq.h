/*
 * fp8bsq.h -- C ABI of the MI355X (gfx950) FP8 block-scaled linear-layer library.
 *
 * What it computes (Resumen Técnico: Jet-RL, gist.science, section "Esquema de
 * Cuantización"; and "Arquitectura Central" for the shared forward/rollout flow):
 * the linear layers run as FP8 GEMMs; activations are quantized in 1x128
 * per-token groups and weights in 128x128 blocks; DGrad and WGrad also run in
 * FP8, WGrad on operands grouped 1x128 / 128x1 along the token dimension;
 * gradients entering and leaving the GEMMs are bf16; master weights are bf16.
 *
 * Numeric format (fixed by this library; the pages only say "FP8"):
 *   - FP8 codes are OCP E4M3 ("E4M3FN": bias 7, max finite 448, NaN 0x7F/0xFF,
 *     signed zero, subnormals k*2^-9), one byte per element;
 *   - one fp32 scale per group: s = fl32(amax / 448), or 1.0 for an all-zero
 *     group; each element is stored as E4M3_RNE(fl32(x / s)) -- one IEEE fp32
 *     division, then round-to-nearest-even to E4M3, with gradual underflow;
 *   - GEMMs multiply E4M3 codes exactly, accumulate in fp32, apply the two
 *     operand scales once per 128-long block of the contraction dimension,
 *     and round the result to bf16 (nearest even).
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers (HIP device memory) owned by the
 *     caller. Tensors are dense and row-major. bf16 tensors are passed as
 *     void* (16-bit elements). The library allocates nothing and keeps no
 *     pointer after returning.
 *   - Every pointer must be 16-byte aligned.
 *   - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *     Calls only enqueue work on that stream and return; outputs are valid
 *     once the stream has reached that point. The library never synchronizes.
 *   - Outputs must not overlap inputs. Outputs are fully overwritten.
 *   - Results are deterministic: the same inputs, shape and library build give
 *     identical bytes.
 *   - Return value: FP8BSQ_OK (0), or an error code below. Arguments are
 *     validated before any HIP runtime call, so an invalid call touches
 *     neither the device nor the stream. No C++ exception crosses the ABI.
 *   - Sizes are int64_t; every dimension must be >= 0 and < 2^31, and every
 *     tensor must hold fewer than 2^40 elements. The contraction length of a
 *     GEMM must be below 2^24 (the kernels address a tile's rows with 32-bit
 *     offsets). A call with a zero-sized output is a valid no-op.
 *   - Thread-safe and reentrant (no mutable global state).
 *   - Channel dimensions (K, N, C) may be any multiple of 8 (so that bf16 rows
 *     stay 16-byte aligned). Write Kp, Np for K, N rounded up to a multiple of
 *     128, Kg = Kp/128, Ng = Np/128. When a dimension is not a multiple of 128,
 *     its last group is partial: the group's amax (and so its scale) covers
 *     the valid elements only, and the FP8 code tensors are padded along that
 *     dimension to whole groups with code 0x00 (+0), which a GEMM contraction
 *     reads as zero products. bf16 tensors keep their logical shape. (The
 *     pages fix no layout for a partial group; for multiples of 128 nothing
 *     changes.)
 */
#ifndef FP8BSQ_H
#define FP8BSQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8BSQ_ABI_VERSION 7

/* Status codes. */
#define FP8BSQ_OK 0
#define FP8BSQ_ERR_NULL 1      /* a required pointer is NULL                          */
#define FP8BSQ_ERR_SHAPE 2     /* a dimension is negative, too large, or not a multiple of 8 / 128 where required */
#define FP8BSQ_ERR_ALIGN 3     /* a pointer is not 16-byte aligned                    */
#define FP8BSQ_ERR_HIP 4       /* the HIP runtime reported an error at launch         */
#define FP8BSQ_ERR_VALUE 5     /* a scalar argument is out of range (eps must be finite and >= 0) */

/* Returns a static, human-readable description of a status code. */
const char* fp8bsq_strerror(int status);

/* Returns FP8BSQ_ABI_VERSION of the built library. */
int fp8bsq_abi_version(void);

/*
 * quantize_act_1x128 -- 1x128 per-token group quantization.
 * Source: "Esquema de Cuantización", activations bullet (1x128 groups); also
 * applied to dY before DGrad (backward GEMMs run in FP8, gradients arrive bf16).
 *
 *   x   in : bf16 [M, K]
 *   xq  out: E4M3 [M, Kp]          xq[m, k] = E4M3_RNE(fl32(x[m, k] / xs[m, k/128])),
 *                                  0x00 for k >= K
 *   xs  out: fp32 [M, Kg]          xs[m, g] = scale of x[m, 128g : min(128g+128, K)]
 * Shape: K % 8 == 0; M >= 0 (any).
 */
int quantize_act_1x128(const void* x, int64_t M, int64_t K,
                       uint8_t* xq, float* xs, void* stream);

/*
 * quantize_weight_128x128 -- 128x128 per-block weight quantization.
 * Source: "Esquema de Cuantización", weights bullet (128x128 blocks);
 * "Arquitectura Central": the bf16 master weights are what gets quantized.
 *
 *   w    in : bf16 [N, K]
 *   wq   out: E4M3 [Np, Kp]        0x00 outside [0, N) x [0, K)
 *   ws   out: fp32 [Ng, Kg]        ws[i, j] = scale of block w[128i : min(128i+128, N),
 *                                                             128j : min(128j+128, K)]
 *   wq_t out: E4M3 [Kp, Np] or NULL  the byte transpose of wq (the DGrad operand;
 *                                   a block's amax is transpose-invariant)
 * Shape: N % 8 == 0, K % 8 == 0.
 */
int quantize_weight_128x128(const void* w, int64_t N, int64_t K,
                            uint8_t* wq, float* ws, uint8_t* wq_t, void* stream);

/*
 * transpose_quantize_128x1 -- 128x1 token-group quantization, written transposed.
 * Source: "Esquema de Cuantización", backward bullets: WGrad runs in FP8 with
 * 1x128 / 128x1 operand groups; activations saved for backward are FP8.
 *
 *   x    in : bf16 [M, C]
 *   xq_t out: E4M3 [C, Mp]         xq_t[c, m] = code of x[m, c]; Mp = M rounded up to 128
 *   xs_t out: fp32 [C, Mp/128]     xs_t[c, b] = scale of x[128b : min(128b+128, M), c]
 * For M % 128 == 0 (Mp = M), bit-identical to quantize_act_1x128 applied to
 * the transpose of x. A ragged M: the last group holds the remaining tokens
 * (its amax is theirs) and xq_t[c, m] = 0x00 (+0) for M <= m < Mp, so WGrad
 * can contract over Mp tokens. (The pages fix no layout for a ragged tail.)
 * C is not grouped here: xq_t has exactly C rows.
 * Shape: C % 8 == 0; M any.
 */
int transpose_quantize_128x1(const void* x, int64_t M, int64_t C,
                             uint8_t* xq_t, float* xs_t, void* stream);

/*
 * quantize_dual_1x128_128x1 -- both groupings of one activation tensor from a
 * single read: the 1x128 row groups of quantize_act_1x128 (the forward or
 * DGrad operand) and the 128x1 token groups of transpose_quantize_128x1 (the
 * WGrad operand, which the forward also keeps as the saved FP8 activation).
 * Source: "Esquema de Cuantización": activations in 1x128 groups for the
 * forward, 1x128 / 128x1 groupings for WGrad, activations stored in FP8
 * between forward and backward.
 *
 *   x    in : bf16 [M, K]
 *   xq   out: E4M3 [M, Kp],   xs   out: fp32 [M, Kg]      (as quantize_act_1x128)
 *   xq_t out: E4M3 [K, Mp],   xs_t out: fp32 [K, Mp/128]  (as transpose_quantize_128x1;
 *                                                          Mp = M rounded up to 128)
 * Every output is bit-identical to the corresponding single-output call.
 * Shape: K % 8 == 0; M any.
 */
int quantize_dual_1x128_128x1(const void* x, int64_t M, int64_t K, uint8_t* xq, float* xs,
                              uint8_t* xq_t, float* xs_t, void* stream);

/*
 * rmsnorm_quantize_1x128 -- RMSNorm with the quantization of its output fused in.
 * Source: "Esquema de Cuantización": the FP8 copy of an activation is made by
 * the operator that produces it; "Implementación": quantization kernels fused
 * with the RMSNorm operator.
 *
 *   x     in : bf16 [M, K]   (the residual stream)
 *   gamma in : bf16 [K]
 *   eps   in : float, finite, >= 0
 *   rstd  out: fp32 [M]      rstd[m] = 1 / sqrt(fl32(sum_k x[m,k]^2 / K) + eps), the
 *                            per-row statistic a backward pass needs (required)
 *   y     out: bf16 [M, K] or NULL   y[m,k] = bf16(fl32(fl32(x[m,k] * rstd[m]) * gamma[k]))
 *   xq, xs    out: quantize_act_1x128(y)
 *   xq_t, xs_t out: transpose_quantize_128x1(y), or both NULL
 * The codes are those of the bf16 values y, bit for bit, whether or not y is
 * written. The sum of squares is accumulated in fp32 (per lane in order, then
 * a fixed butterfly over the wavefront), so rstd is deterministic; y may
 * differ from an exact evaluation by one bf16 unit in the last place.
 * Shape: K % 8 == 0; M any (xq is [M, Kp] and xs [M, Kg] as quantize_act_1x128;
 * the transposed outputs are [K, Mp] and [K, Mp/128], Mp = M rounded up to
 * 128, as transpose_quantize_128x1). Two kernel launches (the row statistics,
 * then the quantizing pass); rstd doubles as the buffer between them.
 */
int rmsnorm_quantize_1x128(const void* x, const void* gamma, float eps, int64_t M, int64_t K,
                           float* rstd, void* y, uint8_t* xq, float* xs, uint8_t* xq_t, float* xs_t,
                           void* stream);

/*
 * swiglu_quantize_1x128 -- the gated activation with the quantization of its
 * output fused in (the down projection's input).
 * Source: "Esquema de Cuantización" (FP8 copy made by the producing operator);
 * "Implementación": quantization kernels fused with the activation operator.
 *
 *   gate, up in : bf16 [M, N]
 *   h        out: bf16 [M, N] or NULL   h = bf16(fl32(silu(gate) * up)), with
 *                 silu(g) = g * sigmoid(g) evaluated in fp32 from the hardware
 *                 exp2 and reciprocal (relative error about 2^-21)
 *   hq, hs     out: quantize_act_1x128(h)
 *   hq_t, hs_t out: transpose_quantize_128x1(h), or both NULL
 * The codes are those of the bf16 values h, bit for bit, whether or not h is
 * written; h may differ from an exact evaluation by one bf16 unit in the last
 * place.
 * Shape: N % 8 == 0; M any (hq is [M, Np] and hs [M, Ng] as quantize_act_1x128;
 * the transposed outputs are [N, Mp] and [N, Mp/128], Mp = M rounded up to
 * 128, as transpose_quantize_128x1).
 */
int swiglu_quantize_1x128(const void* gate, const void* up, int64_t M, int64_t N, void* h,
                          uint8_t* hq, float* hs, uint8_t* hq_t, float* hs_t, void* stream);

/*
 * fp8_gemm_fwd -- forward / rollout GEMM, Y = Xq . Wq^T.
 * Source: "Esquema de Cuantización" (linear layers as FP8 GEMMs on 1x128
 * activations and 128x128 weights); "Arquitectura Central" (rollout and
 * training forward share this one flow).
 *
 *   xq in : E4M3 [M, Kp], xs in: fp32 [M, Kg]         (from quantize_act_1x128)
 *   wq in : E4M3 [Np, Kp], ws in: fp32 [Ng, Kg]       (from quantize_weight_128x128)
 *   y  out: bf16 [M, N]
 *   y[m, n] = bf16( sum_kb xs[m,kb] * ws[n/128,kb] * sum_{k in kb} xq[m,k]*wq[n,k] )
 * M, N, K are the logical sizes. Shape: N % 8 == 0, K % 8 == 0, M >= 0 (any),
 * Kp < 2^24.
 */
int fp8_gemm_fwd(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                 void* y, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * fp8_gemm_dgrad -- DGrad, dX = dYq . Wq (contraction over N).
 * Source: "Esquema de Cuantización", backward bullets (DGrad in FP8; bf16
 * gradients between operators).
 *
 *   dyq  in : E4M3 [M, Np], dys in: fp32 [M, Ng]      (quantize_act_1x128 of dY)
 *   wq_t in : E4M3 [Kp, Np]                            (wq_t of quantize_weight_128x128)
 *   ws   in : fp32 [Ng, Kg]                            (the same forward block scales)
 *   dx   out: bf16 [M, K]
 *   dx[m, k] = bf16( sum_nb dys[m,nb] * ws[nb,k/128] * sum_{n in nb} dyq[m,n]*wq_t[k,n] )
 * M, N, K are the logical sizes. Shape: N % 8 == 0, K % 8 == 0, M >= 0 (any),
 * Np < 2^24.
 */
int fp8_gemm_dgrad(const uint8_t* dyq, const float* dys, const uint8_t* wq_t, const float* ws,
                   void* dx, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * fp8_gemm_wgrad -- WGrad, dW = dYq^T . Xq (contraction over the M tokens).
 * Source: "Esquema de Cuantización", backward bullets (WGrad in FP8 with
 * 1x128 and 128x1 groupings: both operands grouped along the tokens).
 *
 *   dyq_t in : E4M3 [N, M], dys_t in: fp32 [N, M/128]  (transpose_quantize_128x1 of dY)
 *   xq_t  in : E4M3 [K, M], xs_t  in: fp32 [K, M/128]  (transpose_quantize_128x1 of X)
 *   dw    out: bf16 [N, K]
 *   dw[n, k] = bf16( sum_mb dys_t[n,mb] * xs_t[k,mb] * sum_{m in mb} dyq_t[n,m]*xq_t[k,m] )
 * Shape: M % 128 == 0, N % 8 == 0, K % 8 == 0, M < 2^24. For a ragged
 * token count pass the padded Mp of the 128x1 quantizers' outputs (their
 * padded codes are +0 and contribute nothing).
 */
int fp8_gemm_wgrad(const uint8_t* dyq_t, const float* dys_t, const uint8_t* xq_t, const float* xs_t,
                   void* dw, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * Grouped GEMMs -- several problems of one role in as few launches as the
 * hardware allows (one launch per 16 problems).
 * Source: the same passages as the single calls above; grouping is a launch
 * choice, not part of the method.
 *
 * Every problem is the argument list of the plain call, in this order:
 *   fwd:   a = xq,    as = xs,    b = wq,   bs = ws,   out = y  [M, N]
 *   dgrad: a = dyq,   as = dys,   b = wq_t, bs = ws,   out = dx [M, K]
 *   wgrad: a = dyq_t, as = dys_t, b = xq_t, bs = xs_t, out = dw [N, K]
 * Each problem is validated exactly as the plain call (all of them before any
 * launch; the first error is returned); problems with an empty output are
 * skipped. Every output is bit-identical to the plain call's. Outputs of
 * different problems must not overlap.
 * For grouped callers (several linears of a layer, the experts of a MoE
 * layer): one launch lets the tiles of small problems fill the compute units
 * that a single small problem would leave idle.
 */
typedef struct fp8bsq_gemm_problem {
  const uint8_t* a;
  const float* as;
  const uint8_t* b;
  const float* bs;
  void* out;
  int64_t M, N, K;
} fp8bsq_gemm_problem;

int fp8_gemm_fwd_grouped(const fp8bsq_gemm_problem* problems, int count, void* stream);
int fp8_gemm_dgrad_grouped(const fp8bsq_gemm_problem* problems, int count, void* stream);
int fp8_gemm_wgrad_grouped(const fp8bsq_gemm_problem* problems, int count, void* stream);

/*
 * quantize_weight_128x128_stream -- quantize_weight_128x128 with its codes
 * written in the weight-streaming layout (see fp8_weight_stream_layout)
 * instead of row-major, for weights that only feed fp8_gemm_fwd_stream.
 * Source: as quantize_weight_128x128.
 *
 *   w    in : bf16 [N, K] row-major
 *   wq_s out: E4M3, Np * Kp bytes, byte-identical to
 *             fp8_weight_stream_layout(wq) of quantize_weight_128x128's wq
 *   ws   out: fp32 [Ng, Kg], as quantize_weight_128x128
 * Shape: N % 8 == 0, K % 8 == 0. No transposed copy.
 */
int quantize_weight_128x128_stream(const void* w, int64_t N, int64_t K, uint8_t* wq_s, float* ws, void* stream);

/*
 * fp8_weight_stream_layout -- the weight codes rearranged for streaming.
 * Source: "Arquitectura Central" (rollout runs the training forward's FP8
 * flow on the same 128x128-block weight codes, refreshed once per optimizer
 * update) and "Esquema de Cuantización" (the 128x128 weight quantization).
 * The same codes in another order, made once per weight version, for
 * fp8_gemm_fwd_stream: no arithmetic, no rounding.
 *
 *   wq   in : E4M3 [Np, Kp]      (wq of quantize_weight_128x128)
 *   wq_s out: E4M3, Np * Kp bytes: with Kb = Kp/128, for 16-row fragment f,
 *             K block kb, half h (0/1), lane l = 16 g + r (g < 4, r < 16) and
 *             byte b < 16:
 *               wq_s[((f*Kb + kb)*2 + h)*1024 + 16*l + b] = wq[(16f + r)*Kp + 128kb + 32g + 16h + b]
 *             i.e. each 16-row x 128-byte block of wq as 2 KB of contiguous
 *             bytes, blocks of one 16-row band in K order.
 * N, K are the weight's logical sizes. Shape: N % 8 == 0, K % 8 == 0.
 */
int fp8_weight_stream_layout(const uint8_t* wq, int64_t N, int64_t K, uint8_t* wq_s, void* stream);

/*
 * fp8_gemm_fwd_stream -- the forward / rollout GEMM of fp8_gemm_fwd for at most
 * 64 token rows (decode), reading the weight in its stream layout.
 * Source: the same passages as fp8_gemm_fwd.
 *
 *   xq in : E4M3 [M, Kp], xs in: fp32 [M, Kg]         (from quantize_act_1x128)
 *   wq_s in: fp8_weight_stream_layout of wq [Np, Kp], ws in: fp32 [Ng, Kg]
 *   y  out: bf16 [M, N], bit-identical to fp8_gemm_fwd(xq, xs, wq, ws, y, M, N, K)
 * For decode the GEMM is bound by reading the weight once; the stream layout
 * lets each wavefront read its weight rows as one sequential stream.
 * Shape: 1 <= M <= 64 (M = 0 is a no-op), N % 8 == 0, N < 2^28, K % 8 == 0,
 * Kp < 2^24.
 */
int fp8_gemm_fwd_stream(const uint8_t* xq, const float* xs, const uint8_t* wq_s, const float* ws, void* y,
                        int64_t M, int64_t N, int64_t K, void* stream);

/*
 * fp8bsq_cast_f32_e4m3 -- the library's E4M3 encoder on its own.
 * Rounds each fp32 value to E4M3, nearest, ties to even, sign kept; the same
 * device routine every quantizer uses after its division. Inputs must be
 * finite with |v| <= 464 (the largest magnitude with a finite nearest code);
 * other inputs give unspecified bytes.
 *
 *   in  in : fp32 [n];  out out: E4M3 [n].  n >= 0 and n % 4 == 0.
 */
int fp8bsq_cast_f32_e4m3(const float* in, uint8_t* out, int64_t n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8BSQ_H */
