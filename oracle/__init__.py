"""Plain, slow CPU oracle for the fused grouped scaled-activation + block-quantize + grouped GEMM path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its Python binding) may
import or call this package; only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` do.  It shares no code, tables or constants with the GPU side.

Everything is numpy in float64.  Where the method prescribes an FP32 operation sequence, each step is
evaluated in float64 (exact or correctly rounded for +, -, *, /) and rounded to float32 with numpy's
round-to-nearest-even, which equals the correctly rounded FP32 result (53 >= 2*24 + 2, so the double
rounding is innocuous for these operations).

Sources (the web pages this method is taken from):
  [P1] "[PyTorch] Enable fused activation recompute for ScaledTanhSReLU" (TransformerEngine PR 3473)
  [P2] "Activation + GroupedLinear Fusion for MOE" (TransformerEngine PR 3238)
  [P3] "[PyTorch] Preserve FP8 recompute state for inner autocast" (TransformerEngine PR 3284)
The MXFP8 scale rule and the E4M3 / E2M1 / E8M0 element formats are those of the OCP Microscaling
(MX) v1.0 specification; the FP4 recipe with E4M3 scales per 16 and a per-tensor FP32 scale is the
published NVFP4 recipe that [P1] runs (Description, second paragraph).

Parity status of each function is stated in its module header; "parity unpinned" marks a step whose
exact arithmetic the pages do not fix and no closed form or invariant fully determines.
"""

from . import codecs, activations, quant, gemm, mlp  # noqa: F401
