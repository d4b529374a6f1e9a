"""CPU oracle for the FP8 block-scaled linear-layer flow (test infrastructure).

This package is the slow, plainly written reference that the HIP kernels are
checked against. It is test infrastructure, not part of the product: only the
test suite, the smoke check in ``__graft_entry__`` and the CPU-baseline leg of
``bench.py`` may import it. The product path (the C-ABI library and its Python
binding) never imports, links or calls anything here, and this package shares
no code with it: the only thing both sides use is the seeded input generator,
which holds none of the method's arithmetic.

What it follows (the Jet-RL pages; see each function for the exact passage):

* Resumen Técnico: Jet-RL (gist.science), section "Esquema de Cuantización":
  linear layers run as FP8 GEMMs; activations are grouped 1x128, weights
  128x128; DGrad and WGrad also run in FP8, WGrad with 1x128 / 128x1 operand
  groups; gradients between operators stay bf16; saved activations are FP8.
* Same page, "Arquitectura Central": master weights are bf16, and rollout and
  training forward share one quantization flow.
* Same page, "Esquema de Cuantización" (saved activations in FP8, fused with
  the producing operator) and "Implementación" (quantization fused with the
  activation and RMSNorm kernels): the RMSNorm and SwiGLU producers.

Numeric choices the pages leave open (format OCP E4M3, fp32 scale amax/448,
round-to-nearest-even, bf16 GEMM output, the parity tolerance) are the ones the
project fixes up front; every such reading is listed in the design notes.

Modules:
    e4m3   -- the OCP E4M3 codec (decode table, RNE encoder), bf16 helpers
    quant  -- the three group quantizers (1x128, 128x128, 128x1 transposed)
    gemm   -- fp64 GEMMs over dequantized operands, bf16 RNE, tolerance check
    fused  -- RMSNorm and SwiGLU (fp64, rounded once to bf16), whose outputs
              the fused kernels quantize

Every function is pinned by ``tests/test_oracle_*.py`` against something other
than itself: brute-force searches, exact rational arithmetic, closed forms,
invariants and an independent library (torch's float8_e4m3fn cast).
"""

from . import e4m3, quant, gemm, fused  # noqa: F401
