"""FP8Linear: the unified FP8 flow of one linear layer as a torch autograd op.

Source: Resumen Técnico: Jet-RL (gist.science). "Arquitectura Central": the
bf16 master weights are quantized for use, and rollout (inference) and the
training forward run one and the same quantization flow, so the inference
graph is a subgraph of the training forward graph. "Esquema de
Cuantización": the linear layers are FP8 GEMMs on 1x128 activation groups and
128x128 weight blocks; DGrad and WGrad run in FP8 (WGrad on 1x128 / 128x1
groupings); the activations kept for the backward pass are stored in FP8.

Every step runs in the library's HIP kernels through the C ABI:
    forward   quantize_weight_128x128(W)         once per weight version (cached)
              quantize_dual_1x128_128x1(X)        training: X codes for the GEMM and
                                                  the transposed codes saved for WGrad
              quantize_act_1x128(X)               inference (gradients off or not needed)
              fp8_gemm_fwd                        Y = Xq Wq^T
              fp8_gemm_fwd_stream                 inference with at most 64 tokens (decode),
                                                  on the weight codes in their streaming
                                                  layout (made once per weight version);
                                                  the same bits as fp8_gemm_fwd
    backward  quantize_dual_1x128_128x1(dY)
              fp8_gemm_dgrad                      dX = dYq Wq
              fp8_gemm_wgrad                      dW = dYq^T Xq
Both paths quantize X with the same 1x128 rule and run the same GEMM
arithmetic (the streaming forward gives fp8_gemm_fwd's bits), so a row of Y
does not depend on whether gradients are tracked, on the other rows of the
batch, or on the batch size. Feature counts that are not a multiple of
128 end in partial groups; the FP8 codes are then padded to whole groups with
+0 codes and the GEMMs return the logical feature counts.
"""

import torch

from . import (fp8_gemm_dgrad, fp8_gemm_fwd, fp8_gemm_fwd_stream, fp8_gemm_wgrad, quantize_act_1x128,
               quantize_dual_1x128_128x1, quantize_weight_128x128, weight_stream_layout)

# Token counts up to which inference runs the weight-streaming forward.
STREAM_MAX_TOKENS = 64


class _WeightCodes:
    """FP8 codes of a bf16 weight, refreshed when the weight changes in place.

    The streaming-layout copy (the same codes rearranged, N x K more bytes) is
    made from the row-major codes on the first decode-sized inference call of
    a weight version.
    """

    def __init__(self):
        self.key = None
        self.wq = self.ws = self.wq_t = None
        self.wq_s = None

    def get(self, w):
        key = (w.data_ptr(), w._version, tuple(w.shape))
        if key != self.key:
            self.wq, self.ws, self.wq_t = quantize_weight_128x128(w.detach(), transposed=True)
            self.wq_s = None
            self.key = key
        return self.wq, self.ws, self.wq_t

    def get_stream(self, w):
        self.get(w)
        if self.wq_s is None:
            self.wq_s = weight_stream_layout(self.wq)
        return self.wq_s, self.ws


class FP8LinearFunction(torch.autograd.Function):
    """Y = X W^T with FP8 block-scaled operands; X [M, K] and W [N, K] in bf16."""

    @staticmethod
    def forward(ctx, x, w, codes):
        # any token count: the 128x1 copies are padded to whole 128-token blocks
        # with +0 codes, and WGrad contracts over the padded length
        wq, ws, wq_t = codes.get(w)
        xq, xs, xq_t, xs_t = quantize_dual_1x128_128x1(x)
        y = fp8_gemm_fwd(xq, xs, wq, ws, n=w.shape[0])
        ctx.save_for_backward(xq_t, xs_t, wq_t, ws)
        ctx.in_features = w.shape[1]
        return y

    @staticmethod
    def backward(ctx, dy):
        xq_t, xs_t, wq_t, ws = ctx.saved_tensors
        dy = dy.contiguous()
        need_dx, need_dw = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        if need_dw:
            dyq, dys, dyq_t, dys_t = quantize_dual_1x128_128x1(dy)
        else:
            dyq, dys = quantize_act_1x128(dy)
        dx = fp8_gemm_dgrad(dyq, dys, wq_t, ws, k=ctx.in_features) if need_dx else None
        dw = fp8_gemm_wgrad(dyq_t, dys_t, xq_t, xs_t) if need_dw else None
        return dx, dw, None


def fp8_linear_inference(x, w, codes):
    """The rollout path: Y = Xq Wq^T with no state kept for a backward pass
    (the weight-streaming forward for at most STREAM_MAX_TOKENS tokens)."""
    xq, xs = quantize_act_1x128(x)
    if x.shape[0] <= STREAM_MAX_TOKENS:
        wq_s, ws = codes.get_stream(w)
        return fp8_gemm_fwd_stream(xq, xs, wq_s, ws, n=w.shape[0])
    wq, ws, _ = codes.get(w)
    return fp8_gemm_fwd(xq, xs, wq, ws, n=w.shape[0])


class FP8Linear(torch.nn.Module):
    """A bias-free linear layer (in_features -> out_features) on the FP8 flow.

    The weight is a bf16 parameter [out_features, in_features]; both feature
    counts must be multiples of 8. Inputs are bf16 [..., in_features] on the
    GPU; leading dimensions are flattened into tokens.
    """

    def __init__(self, in_features, out_features, device="cuda", weight=None):
        super().__init__()
        if in_features % 8 or out_features % 8 or in_features <= 0 or out_features <= 0:
            raise ValueError("in_features and out_features must be positive multiples of 8")
        if weight is None:
            weight = torch.empty((out_features, in_features), dtype=torch.bfloat16, device=device)
            torch.nn.init.normal_(weight, std=0.02)
        self.weight = torch.nn.Parameter(weight)
        self._codes = _WeightCodes()

    def forward(self, x):
        lead = x.shape[:-1]
        x2 = x.reshape(-1, x.shape[-1]).contiguous()
        if torch.is_grad_enabled() and (self.weight.requires_grad or x2.requires_grad):
            y = FP8LinearFunction.apply(x2, self.weight, self._codes)
        else:
            y = fp8_linear_inference(x2, self.weight, self._codes)
        return y.reshape(*lead, y.shape[-1])
