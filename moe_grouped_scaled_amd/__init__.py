"""MI355X (gfx950) fused MoE expert-MLP hot path: per-row scaled activation + grouped MXFP8 / NVFP4
block quantization + grouped MX GEMM, behind the C ABI of include/mgs.h.

``_native`` is the ctypes binding (same names as the C entry points); ``expert_mlp`` drives one
expert-MLP training step (FC1 -> scaled activation -> FC2, recompute, delayed wgrad, bias) through it.
Importing the package loads libmgs.so and raises if it is missing: there is no fallback path.
"""

from . import _native  # noqa: F401
from ._native import (  # noqa: F401
    MgsError,
    QTensor,
    act_bwd_workspace_bytes,
    act_params,
    grouped_col_sum,
    grouped_gemm_mx,
    grouped_mx_quantize,
    grouped_scaled_act_bwd,
    grouped_scaled_act_fwd,
    qtensor_nbytes,
    quantize_workspace_bytes,
)
