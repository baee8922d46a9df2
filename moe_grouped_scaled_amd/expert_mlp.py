"""One MoE expert-MLP training step (FC1 -> per-row scaled activation -> FC2) driven through the C ABI.

Sources:
  * page "Activation + GroupedLinear Fusion for MOE", sequence diagram: forward = fused scaled
    activation + grouped quantize, then the FC2 grouped GEMM, saving (input_, scales); backward = FC2
    backward giving dL/d(act_out * scales), then the fused activation backward giving (grouped_dy,
    dense_dy, grad_scales), then FC1's backward.
  * same page, review finding on the fused backward: with FC1's weights frozen while the per-row
    scales (and the module input) still need gradients, the fused backward must run without FC1's
    weight-gradient state.  Here every gradient is requested separately (`grad_x1`, `grad_probs`,
    `grad_fc1`, `grad_fc2`); an unrequested one is a NULL output of the fused launches, and the
    quantized copies only it would consume are neither made nor kept.
  * same page ("[PyTorch] Enable fused activation recompute ...", Description and review discussion):
    the fused forward activates FC1's FP32 accumulator, the backward and the recompute its saved BF16
    rounding.  `fc1_fp32_act=True` does the same here: FC1 writes FP32, one fused launch activates and
    quantizes it and writes the BF16 copy the backward keeps; the regenerated FC2 input then differs
    from the forward's by the BF16 rounding, and so does FC2's weight gradient with recompute on.
    With the default (False) both passes activate the BF16 FC1 output and the twins are bitwise equal.
  * same page, Description and review discussion: the fused forward runs the activation in FC1's
    GEMM epilogue.  `fuse_fc1_act=True` does that here for MXFP8 and unary activations when the
    forward writes no columnwise copy (recompute on, or no FC2 weight gradient): FC1's epilogue stores
    the BF16 FC1 output and FC2's quantized input in one launch, bit for bit what the separate pass
    writes from the same values (its FP32 value with `fc1_fp32_act`, else its BF16 rounding).
    `fuse_fc1_act="auto"` takes the epilogue only where it is the faster of the two (EPILOGUE_ACTS).
  * same page, deviation table: its NVFP4 rows were measured with a recipe it names NVFP4_RHT.
    `rht_signs` (NVFP4; a 16-bit sign mask) applies the random Hadamard transform to the columnwise
    copies of the four weight-gradient operands (X1, A, dY2, dY1), all with the same signs, so both
    weight-gradient GEMMs multiply transformed operands whose product is unchanged.
  * page "[PyTorch] Enable fused activation recompute for ScaledTanhSReLU", Description: with
    activation recompute the forward keeps only the BF16 FC1 output and the backward regenerates FC2's
    input from it; forward, dgrad, dprobs and FC1 wgrad are unchanged; memory drops between forward and
    backward; bias and delayed weight-gradient computation change what wgrad consumes, and the
    regenerated tensor must live until the delayed wgrad runs.

Every arithmetic step runs in the library's HIP kernels; this module only allocates torch buffers,
orders the calls and decides what is kept between forward and backward.  Tensor shapes:
  x1 [M, H] BF16, probs [M] FP32, w1 [E, F_in, H], b1 [E, F_in], w2 [E, H, F], b2 [E, H] (BF16),
  with F_in = F for unary activations and 2 F for gated ones ([gate | up]).
"""

import torch

from . import _native as N

GATED = ("swiglu", "clamped_swiglu", "glu")
# Activations whose epilogue form is faster than the separate fused pass.  Measured at 16 experts x
# 2048 tokens with hidden = ffn = 4096: FC1's epilogue adds ~81 us for SReLU and sigmoid, against an
# ~87 us separate pass, but ~220 us for TanhSReLU and ~376 us for GeLU, against 134 and 193 us.  In
# the epilogue the activation math runs with the matrix cores idle; the separate pass overlaps it
# with its own memory traffic.
EPILOGUE_ACTS = ("srelu", "sigmoid")


def use_fc1_epilogue(fuse_fc1_act, kind, fmt, writes_col):
    """Whether the forward runs the activation in FC1's GEMM epilogue.  `fuse_fc1_act` is True,
    False or "auto" (the epilogue for the activations in EPILOGUE_ACTS).  The epilogue exists for
    MXFP8 and unary activations, and only when the forward writes no columnwise copy of FC2's input."""
    if fuse_fc1_act not in (True, False, "auto"):
        raise ValueError("fuse_fc1_act must be True, False or 'auto', not %r" % (fuse_fc1_act,))
    if fmt != "mxfp8" or kind in GATED or writes_col:
        return False
    return fuse_fc1_act is True or (fuse_fc1_act == "auto" and kind in EPILOGUE_ACTS)


class ExpertMLP:
    def __init__(self, kind, fmt, w1, w2, b1=None, b2=None, recompute=False, delay_wgrad=False,
                 s=2.0, limit=7.0, alpha=1.0, beta=0.0, grad_x1=True, grad_probs=True, grad_fc1=True,
                 grad_fc2=True, fc1_fp32_act=False, fuse_fc1_act=False, rht_signs=None):
        self.kind, self.fmt = kind, fmt
        self.w1, self.w2, self.b1, self.b2 = w1, w2, b1, b2
        self.e, self.f_in, self.h = w1.shape
        self.f = w2.shape[2]
        assert w2.shape == (self.e, self.h, self.f)
        assert self.f_in == (2 * self.f if kind in GATED else self.f)
        self.recompute, self.delay_wgrad = recompute, delay_wgrad
        self.fc1_fp32_act = fc1_fp32_act
        self.fuse_fc1_act = fuse_fc1_act
        assert rht_signs is None or fmt == "nvfp4", "the Hadamard transform is an NVFP4 recipe"
        self.rht = rht_signs
        self.fused_fc1_calls = 0  # forwards whose FC1 GEMM ran the activation in its epilogue
        # which gradients the backward produces (parameters of FC1 / FC2 = weight and bias)
        self.grad_x1, self.grad_probs = grad_x1, grad_probs
        self.grad_fc1, self.grad_fc2 = grad_fc1, grad_fc2
        # anything below FC2's output needs FC2's dgrad and the activation backward
        self.grad_below_fc2 = grad_x1 or grad_probs or grad_fc1
        self.act = N.act_params(kind, s=s, limit=limit, alpha=alpha, beta=beta)
        self.ctx = None
        self.pending_wgrad = None
        # which fused outputs each pass requested (the recompute path writes FC2's columnwise input
        # in the backward launch instead of the forward one)
        self.trace = {"fwd_act_col": 0, "bwd_act_col": 0}

    # ------------------------------------------------------------------ helpers
    def _quant(self, x, splits, width, row=True, col=True, rht=None):
        qr = N.QTensor(self.fmt, False, splits, width) if row else None
        qc = N.QTensor(self.fmt, True, splits, width, rht=rht) if col else None
        N.grouped_mx_quantize(self.fmt, splits, width, x, qr, qc, self._amax_buf(len(splits), col and rht is not None))
        return qr, qc

    def _amax_buf(self, n, rht=False):
        """NVFP4 per-group amax: E entries, 2E when a columnwise copy is Hadamard-transformed."""
        return torch.empty(2 * n if rht else n, dtype=torch.float32, device="cuda") if self.fmt == "nvfp4" else None

    # ------------------------------------------------------------------ forward
    def forward(self, x1, probs, splits):
        """`splits`: host split sizes, or an N.DeviceGroups (device-resident split sizes): then
        x1 and probs have the capacity's rows, only the first sum(splits) of which are used, and the
        step enqueues the offsets computation first, so that a captured graph of the step follows the
        split sizes held in the device tensor at each replay."""
        e, h, f, f_in = self.e, self.h, self.f, self.f_in
        if isinstance(splits, N.DeviceGroups):
            if x1.shape[0] != splits.max_rows or probs.shape[0] != splits.max_rows:
                raise ValueError("with device-resident split sizes x1 and probs have the capacity's %d rows "
                                 "(got %d and %d)" % (splits.max_rows, x1.shape[0], probs.shape[0]))
            splits.update()
        m = x1.shape[0]
        fmt = self.fmt
        wsplit1, wsplit2 = [f_in] * e, [h] * e
        x1_row, x1_col = self._quant(x1, splits, h, col=self.grad_fc1, rht=self.rht)  # FC1 fprop / wgrad
        w1_row, w1_col = self._quant(self.w1.view(e * f_in, h), wsplit1, h,  # fprop / dgrad copies
                                     col=self.grad_x1)
        y1 = torch.empty((m, f_in), dtype=torch.bfloat16, device="cuda")
        a_row = N.QTensor(fmt, False, splits, f)
        a_col = None if (self.recompute or not self.grad_fc2) else N.QTensor(fmt, True, splits, f, rht=self.rht)
        a_amax = self._amax_buf(e, a_col is not None and self.rht is not None)
        if use_fc1_epilogue(self.fuse_fc1_act, self.kind, fmt, a_col is not None):
            N.grouped_gemm_mx_fprop_act(splits, m, f_in, h, x1_row, w1_row, y1, self.act, probs, a_row,
                                        bias=self.b1, act_input="fp32" if self.fc1_fp32_act else "bf16")
            del x1_row, w1_row
            self.fused_fc1_calls += 1
        elif self.fc1_fp32_act:
            y1_f32 = torch.empty((m, f_in), dtype=torch.float32, device="cuda")
            N.grouped_gemm_mx("fprop", fmt, splits, m, f_in, h, x1_row, w1_row, y1_f32, bias=self.b1)
            del x1_row, w1_row
            N.grouped_scaled_act_fwd_f32(self.act, fmt, splits, f_in, y1_f32, probs, a_row, a_col, a_amax,
                                         x_bf16_out=y1)
            del y1_f32
        else:
            N.grouped_gemm_mx("fprop", fmt, splits, m, f_in, h, x1_row, w1_row, y1, bias=self.b1)
            del x1_row, w1_row
            N.grouped_scaled_act_fwd(self.act, fmt, splits, f_in, y1, probs, a_row, a_col, a_amax)
        self.trace["fwd_act_col"] += a_col is not None
        w2_row, w2_col = self._quant(self.w2.view(e * h, f), wsplit2, f, col=self.grad_below_fc2)
        y2 = torch.empty((m, h), dtype=torch.bfloat16, device="cuda")
        N.grouped_gemm_mx("fprop", fmt, splits, m, h, f, a_row, w2_row, y2, bias=self.b2)
        del a_row, w2_row
        self.ctx = dict(splits=splits if isinstance(splits, N.DeviceGroups) else list(map(int, splits)), m=m, y1=y1,
                        probs=probs, a_col=a_col,
                        a_amax=a_amax, x1_col=x1_col, w1_col=w1_col, w2_col=w2_col)
        return y2

    # ------------------------------------------------------------------ backward
    def _workspace(self, nbytes):
        """Partial sums of the backward launches (dprobs, bias gradients): one buffer shared by the
        calls of a step, which run in order on one stream; kept between steps, grown on demand."""
        ws = getattr(self, "_ws", None)
        if ws is None or ws.numel() < nbytes:
            ws = self._ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
        return ws

    def backward(self, dy2):
        c = self.ctx
        splits, m, fmt = c["splits"], c["m"], self.fmt
        e, h, f, f_in = self.e, self.h, self.f, self.f_in
        g1, g2, below = self.grad_fc1, self.grad_fc2, self.grad_below_fc2
        # dY2 quantized for FC2's dgrad and wgrad; FC2's bias gradient (its column sums) in the same pass
        dy2_row = N.QTensor(fmt, False, splits, h) if below else None
        dy2_col = N.QTensor(fmt, True, splits, h, rht=self.rht) if g2 else None
        db2 = torch.empty((e, h), dtype=torch.float32, device="cuda") if (g2 and self.b2 is not None) else None
        if below or g2:
            N.grouped_mx_quantize(fmt, splits, h, dy2, dy2_row, dy2_col,
                                  self._amax_buf(e, g2 and self.rht is not None), col_sum=db2,
                                  workspace=self._workspace(N.quantize_workspace_bytes(splits, h)))
        a_col = c["a_col"]
        grads = {}
        dy1_col = db1 = None
        if below:
            da = torch.empty((m, f), dtype=torch.bfloat16, device="cuda")
            N.grouped_gemm_mx("dgrad", fmt, splits, m, f, h, dy2_row, c["w2_col"], da)
            del dy2_row
            # FC1's bias gradient: column sums of the dense BF16 dY1, taken inside the activation backward
            db1 = torch.empty((e, f_in), dtype=torch.float32, device="cuda") if (g1 and self.b1 is not None) else None
            dy1_row = N.QTensor(fmt, False, splits, f_in) if self.grad_x1 else None
            dy1_col = N.QTensor(fmt, True, splits, f_in, rht=self.rht) if g1 else None
            dprobs = torch.empty(m, dtype=torch.float32, device="cuda") if self.grad_probs else None
            if self.recompute and g2:
                a_col = N.QTensor(fmt, True, splits, f, rht=self.rht)
                self.trace["bwd_act_col"] += 1
            N.grouped_scaled_act_bwd(self.act, fmt, splits, f_in, c["y1"], da, c["probs"],
                                     dx_row=dy1_row, dx_col=dy1_col,
                                     dx_group_amax=self._amax_buf(e, g1 and self.rht is not None)
                                     if (dy1_row is not None or dy1_col is not None) else None,
                                     dprobs=dprobs, dx_col_sum=db1,
                                     act_col=a_col if (self.recompute and g2) else None,
                                     saved_group_amax=c["a_amax"],
                                     workspace=self._workspace(N.act_bwd_workspace_bytes(self.act, splits, f_in)))
            del da
            if self.grad_x1:
                dx1 = torch.empty((m, h), dtype=torch.bfloat16, device="cuda")
                N.grouped_gemm_mx("dgrad", fmt, splits, m, h, f_in, dy1_row, c["w1_col"], dx1)
                del dy1_row
                grads["dx1"] = dx1
            if self.grad_probs:
                grads["dprobs"] = dprobs
        elif self.recompute and g2:
            # nothing below FC2 needs a gradient: FC2's columnwise input is regenerated from the saved
            # BF16 FC1 output by a forward launch that requests only that output (the same bits)
            a_col = N.QTensor(fmt, True, splits, f, rht=self.rht)
            self.trace["bwd_act_col"] += 1
            N.grouped_scaled_act_fwd(self.act, fmt, splits, f_in, c["y1"], c["probs"], None, a_col,
                                     self._amax_buf(e, self.rht is not None))
        # what the weight gradients consume stays alive until backward_dw (possibly delayed)
        self.pending_wgrad = dict(splits=splits, m=m, dy2_col=dy2_col, a_col=a_col if g2 else None,
                                  dy1_col=dy1_col, x1_col=c["x1_col"] if g1 else None, db1=db1, db2=db2)
        self.ctx = None
        if not self.delay_wgrad:
            grads.update(self.backward_dw())
        return grads

    def backward_dw(self, dw1=None, dw2=None, accumulate=False):
        """Weight (and bias) gradients from the kept columnwise copies; FP32 results."""
        p = self.pending_wgrad
        assert p is not None, "backward_dw() without a pending backward"
        splits, m, fmt = p["splits"], p["m"], self.fmt
        e, h, f, f_in = self.e, self.h, self.f, self.f_in
        out = {}
        if self.grad_fc2:
            if dw2 is None:
                dw2 = torch.empty((e, h, f), dtype=torch.float32, device="cuda")
            N.grouped_gemm_mx("wgrad", fmt, splits, h, f, m, p["dy2_col"], p["a_col"], dw2, accumulate=accumulate)
            out["dw2"] = dw2
        if self.grad_fc1:
            if dw1 is None:
                dw1 = torch.empty((e, f_in, h), dtype=torch.float32, device="cuda")
            N.grouped_gemm_mx("wgrad", fmt, splits, f_in, h, m, p["dy1_col"], p["x1_col"], dw1, accumulate=accumulate)
            out["dw1"] = dw1
        # the bias gradients were taken in the backward's quantize / activation passes
        if p["db2"] is not None:
            out["db2"] = p["db2"]
        if p["db1"] is not None:
            out["db1"] = p["db1"]
        self.pending_wgrad = None
        return out


def gemm_flops(m, h, f, f_in):
    """FLOPs of the six grouped GEMMs of one step (fprop, dgrad and wgrad of FC1 and FC2)."""
    return 2 * m * (h * f_in + f * h) * 3
