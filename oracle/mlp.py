"""One expert-MLP training step (FC1 -> per-row scaled activation -> FC2, forward and backward).

Test infrastructure only (see the package header).

Sources:
  * [P2] Sequence diagram: forward = scaled activation + grouped quantize, then the FC2 grouped GEMM,
    saving (input_, scales) for backward; backward = FC2 backward giving dL/d(act_out * scales), then
    the activation backward giving (grouped_dy, dense_dy, grad_scales), then FC1's backward.
  * [P1] Description: the step runs with bias, with all experts' weights in one tensor and with
    delayed weight-gradient computation; turning recompute on alters only the tensors kept between
    forward and backward.

Step, in order (each GEMM as in oracle.gemm, each quantization as in oracle.quant):
  forward : X1 -> q(row, col); W1 -> q(row) and q(col); Y1 = bf16(X1 W1_g^T + b1_g)
            A = act(Y1) * p -> q(row, col);  W2 -> q(row), q(col);  Y2 = bf16(A W2_g^T + b2_g)
  backward: dY2 -> q(row, col); dA = bf16(dY2 W2_g);  (dY1, dp) = act_bwd(Y1, dA, p)
            dY1 -> bf16 dense, q(row, col); dX1 = bf16(dY1 W1_g)
  wgrad   : dW2_g = dY2_g^T A_g ; dW1_g = dY1_g^T X1_g (both from the columnwise copies, FP32)
            db2_g = sum over the group's rows of dY2 ; db1_g = sum of the dense BF16 dY1.
With act_input="bf16" (default) the recompute variant computes the same values (recompute only
changes what is kept between forward and backward); the memory drop is a closed form, see
``recompute_memory_drop``.  With act_input="fp32" the forward activates the FP32 FC1 output
f32(X1 W1_g^T + b1_g) instead of its BF16 rounding ([P1] Description and review discussion: the fused
forward reads the FP32 accumulator, the backward the saved BF16 output); the backward still reads
Y1 = bf16(...), and with recompute FC2's columnwise input is regenerated from Y1 (NVFP4: under the
forward's group amax), so FC2's weight gradient alone differs between the recompute twins.

Parity: composed from the pinned pieces; end-to-end values are compared with relative-RMS bounds.
"""

import numpy as np

from . import activations as act_mod
from .codecs import bf16_bits_to_f64, f32, f32_to_bf16_bits
from .gemm import (
    dequant_col_grouped,
    dgrad_weight,
    dequant_row_grouped,
    gemm_grouped_k,
    gemm_grouped_m,
)
from .quant import MXFP8, NVFP4, col_offsets, group_offsets, quantize_grouped


def _bf16(x64):
    """float64 -> FP32 -> BF16 value (float64), as a GEMM with FP32 accumulation and BF16 output."""
    return bf16_bits_to_f64(f32_to_bf16_bits(f32(x64).astype(np.float32)))


def _q(x, splits, fmt, width, row=True, col=True, rht=None):
    q = quantize_grouped(x, splits, fmt, rowwise=row, colwise=col, rht=rht)
    gs = q.get("group_scale")
    out = {"raw": q}
    if row:
        out["row"] = dequant_row_grouped(fmt, q["row_data"], q["row_scales"], splits, width, gs)
    if col:
        out["col"] = dequant_col_grouped(fmt, q["col_data"], q["col_scales"], splits, width,
                                         q.get("col_group_scale", gs))
    return out


def mlp_step(kind, fmt, splits, x1, w1, b1, w2, b2, p, dy2, act_params=None, act_input="bf16",
             recompute=False, rht=None):
    """All inputs are float64 arrays holding BF16 (x1, w1, b1, w2, b2, dy2) or FP32 (p) values.

    Shapes: x1 [M, H]; w1 [E, F_in, H]; b1 [E, F_in]; w2 [E, H, F]; b2 [E, H]; p [M]; dy2 [M, H].
    `rht` (NVFP4 only, a 16-bit sign mask): Hadamard-transform the columnwise copies of the four
    weight-gradient operands (X1, A, dY2, dY1) with the same signs.
    Returns a dict of float64 results.
    """
    act_params = act_params or {}
    e = len(splits)
    m, h = x1.shape
    f_in = w1.shape[1]
    f = w2.shape[2]
    wsplit_1 = [f_in] * e
    wsplit_2 = [h] * e

    qx1 = _q(x1, splits, fmt, h, rht=rht)
    qw1 = _q(w1.reshape(e * f_in, h), wsplit_1, fmt, h)
    w1_row = qw1["row"].reshape(e, f_in, h)
    w1_col = dgrad_weight(qw1["col"], f_in)  # per expert [H x F_in]
    y1_acc = gemm_grouped_m(qx1["row"], list(w1_row), splits, bias=b1)
    y1 = _bf16(y1_acc)

    if act_input == "fp32":
        a32 = act_mod.scaled_act_fwd(kind, f32(y1_acc), p, **act_params)
    else:
        assert act_input == "bf16", act_input
        a32 = act_mod.scaled_act_fwd(kind, y1, p, **act_params)
    qa = _q(a32, splits, fmt, f, rht=rht)
    if recompute and act_input == "fp32":
        # FC2's columnwise input regenerated from the saved BF16 Y1 (the forward's only rowwise)
        a_rec = act_mod.scaled_act_fwd(kind, y1, p, **act_params)
        amax = qa["raw"].get("group_amax")
        q_rec = quantize_grouped(a_rec, splits, fmt, rowwise=False, colwise=True, group_amax=amax, rht=rht)
        qa["col"] = dequant_col_grouped(fmt, q_rec["col_data"], q_rec["col_scales"], splits, f,
                                        q_rec.get("col_group_scale", q_rec.get("group_scale")))
    qw2 = _q(w2.reshape(e * h, f), wsplit_2, fmt, f)
    w2_row = qw2["row"].reshape(e, h, f)
    w2_col = dgrad_weight(qw2["col"], h)     # per expert [F x H]
    y2 = _bf16(gemm_grouped_m(qa["row"], list(w2_row), splits, bias=b2))

    qdy2 = _q(dy2, splits, fmt, h, rht=rht)
    da = _bf16(gemm_grouped_m(qdy2["row"], w2_col, splits))
    dy1_32, dp = act_mod.scaled_act_bwd(kind, y1, da, p, **act_params)
    dy1_bf16 = _bf16(dy1_32)
    qdy1 = _q(dy1_32, splits, fmt, f_in, rht=rht)
    dx1 = _bf16(gemm_grouped_m(qdy1["row"], w1_col, splits))

    dw2 = gemm_grouped_k(qdy2["col"], qa["col"])    # [E, H, F]
    dw1 = gemm_grouped_k(qdy1["col"], qx1["col"])   # [E, F_in, H]
    off = group_offsets(splits)
    db2 = np.stack([dy2[off[g]:off[g + 1]].sum(axis=0) for g in range(e)])
    db1 = np.stack([dy1_bf16[off[g]:off[g + 1]].sum(axis=0) for g in range(e)])
    return {
        "y1": y1, "a32": a32, "y2": y2, "da": da, "dy1": dy1_32, "dp": dp, "dx1": dx1,
        "dw1": dw1, "dw2": dw2, "db1": db1, "db2": db2,
        # the quantized operands of the six GEMMs (layouts of oracle.quant.quantize_grouped)
        "q_x1": qx1["raw"], "q_w1": qw1["raw"], "q_a": qa["raw"], "q_w2": qw2["raw"],
        "q_dy2": qdy2["raw"], "q_dy1": qdy1["raw"],
    }


def recompute_memory_drop(fmt, splits, width_out):
    """Bytes not kept between forward and backward when recompute is on: the columnwise copy of the
    activation output (data + scales), i.e. what the forward no longer writes.  [P1] Description,
    first list, last bullet: memory must drop, measured between forward and backward.
    """
    rows = int(col_offsets(splits)[-1])
    if fmt == MXFP8:
        return rows * width_out + rows * width_out // 32
    return rows * width_out // 2 + rows * width_out // 16
