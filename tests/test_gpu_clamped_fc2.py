"""The clamped-SwiGLU + FC2 workload at its full shape on the GPU: 32 experts (one GPU's share of an
expert-parallel layer), 65,536 tokens in a Zipf(1.2) split with four empty experts (the largest holds
21,757), FC1 output 2 x 2048, clamp 7, FC2 to hidden 7168.

The GPU runs each kernel over the whole workload, in the launches a training step makes; the oracle
recomputes sampled pieces one by one, where every value is local:
  * rowwise blocks lie inside a token row, so sampled rows fix their rowwise codes and scales, dense
    dL/dx and dprobs;
  * columnwise blocks are 32 tokens of one expert in one column, so a 128-token block of an expert
    fixes that block's columnwise codes and scales in every column;
  * an FPROP or DGRAD output row needs the row's operand and the expert's weight; an output row of
    the weight gradient needs one column of dY2 over the expert's tokens and the other operand.
Checked experts: the largest, one under 500 tokens, one of 2,000-4,000 tokens (these two in full)
and an empty one.  Criteria: clamped-SwiGLU codes differ in at most 0.1 % of the elements, each by at
most one step; GEMM outputs within 1e-3 relative to RMS in FP32, on operands asserted byte-identical
to the oracle's own quantization of the same inputs.

Pages: "Activation + GroupedLinear Fusion for MOE" (Greptile summary: clamped SwiGLU fused with the
per-row scale and the grouped quantization; sequence diagram: FC2 forward, FC2 backward, activation
backward); "[PyTorch] Enable fused activation recompute for ScaledTanhSReLU" (Description: the
backward regenerates FC2's columnwise input).
"""

import numpy as np
import pytest

import workloads
from oracle import activations as A
from oracle import codecs
from oracle import gemm as G
from oracle import quant as Q
from tests.helpers import bf16_f64, bf16_host, compare_quantized, f32, rel_rms, to_dev, to_dev_bf16, u8

pytestmark = pytest.mark.gpu

E, H, F, W_IN, LIMIT = 32, 7168, 2048, 4096, 7.0
TOL = 1e-3


@pytest.fixture(scope="module")
def N():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from moe_grouped_scaled_amd import _native
    return _native


@pytest.fixture(scope="module")
def wl():
    d = workloads.make("clamped_fc2")
    assert int(d["splits"].sum()) == 65536 and int(np.sum(d["splits"] == 0)) == 4
    return d


def _checked_groups(splits):
    largest = int(np.argmax(splits))
    small = [g for g in range(E) if 0 < splits[g] < 500][0]
    mid = [g for g in range(E) if 2000 <= splits[g] <= 4000][0]
    empty = [g for g in range(E) if splits[g] == 0][0]
    return largest, small, mid, empty


def _mx(codes, scale_codes):
    """(code, block scale per element, dequantized value) of an MXFP8 matrix with plain
    [rows, width / 32] scales."""
    s = np.repeat(codecs.e8m0_decode(scale_codes), 32, axis=1)
    return codes, s, codecs.e4m3_decode(codes) * s


def _gpu_col_block(q, width, coff_g, mp_g, t0):
    """Codes [width x 128] and plain scales [width x 4] of tokens t0 .. t0 + 127 of one expert's MXFP8
    columnwise copy (the expert's [width x mp_g] matrix starts at element width * coff_g)."""
    d = u8(q.data[width * coff_g: width * (coff_g + mp_g)].view(width, mp_g)[:, t0:t0 + 128])
    s_all = u8(q.scales[width * coff_g // 32: width * (coff_g + mp_g) // 32])
    s = Q.mx_scales_from_kstep(s_all, width, mp_g)[:, t0 // 32: t0 // 32 + 4]
    return d, s


def _gpu_rows(q, total_rows, width, rows):
    """Codes [len(rows) x width] and plain scales of rows of an MXFP8 rowwise copy."""
    import torch
    idx = torch.as_tensor(rows, device=q.data.device)
    d = u8(q.data.view(total_rows, width)[idx])
    # K-step grouped scales: byte ((kb / 4) * R + r) * 4 + kb % 4 -> [steps, R, 4]
    steps = -(-width // 128)
    s = u8(q.scales.view(steps, total_rows, 4)[:, idx, :])          # [steps, n, 4]
    s = np.transpose(s, (1, 0, 2)).reshape(len(rows), steps * 4)[:, : width // 32]
    return d, s


def _dense_dx_ok(got_bits, dx32, x, dy, p, wa):
    """Dense BF16 dL/dx: at most 0.1 % of the values differ from the oracle's rounding, each by one
    BF16 step or, near a root of the derivative where its FP32 terms cancel, by 2^-20 of their
    magnitude (as in the small-case backward test)."""
    ref = codecs.f32_to_bf16_bits(dx32.astype(np.float32))
    diff = got_bits != ref
    assert diff.mean() <= 1e-3, diff.mean()
    gv, rv = bf16_f64(got_bits[diff]), bf16_f64(ref[diff])
    xg, xu = np.abs(x[:, :wa]), np.abs(x[:, wa:])
    mag = np.abs(dy) * p[:, None] * (1.0 + xg) * (1.0 + xu)
    mag = np.concatenate([mag, mag], axis=1)
    tol = np.abs(rv) * 2.0 ** -7 * 1.0001 + 2.0 ** -20 * mag[diff] + 1e-30
    assert np.all(np.abs(gv - rv) <= tol)
    return ref


def test_clamped_backward_full_size(N, wl):
    """The fused clamped-SwiGLU backward over all 65,536 tokens, with every output requested (dense,
    rowwise and columnwise dL/dx, dprobs, the FC1 bias gradient and the recomputed FC2 input); the
    recompute output is byte-identical to the forward's columnwise copy."""
    import torch
    d = wl
    splits = d["splits"]
    sp = list(map(int, splits))
    m = int(splits.sum())
    largest, small, mid, empty = _checked_groups(splits)
    print("case: clamped SwiGLU backward, 32 experts x 65536 tokens; experts", largest, small, mid, empty,
          "sizes", sp[largest], sp[small], sp[mid], sp[empty], flush=True)
    act = N.act_params("clamped_swiglu", limit=LIMIT)
    x, dy, p = to_dev_bf16(d["x"]), to_dev_bf16(d["dy"]), to_dev(d["p"])
    dx = torch.empty((m, W_IN), dtype=torch.bfloat16, device="cuda")
    dxr, dxc = N.QTensor("mxfp8", False, sp, W_IN), N.QTensor("mxfp8", True, sp, W_IN)
    ac, fc = N.QTensor("mxfp8", True, sp, F), N.QTensor("mxfp8", True, sp, F)
    dp = torch.empty(m, dtype=torch.float32, device="cuda")
    cs = torch.full((E, W_IN), 7.0, dtype=torch.float32, device="cuda")
    N.grouped_scaled_act_bwd(act, "mxfp8", sp, W_IN, x, dy, p, dx=dx, dx_row=dxr, dx_col=dxc, dprobs=dp,
                             dx_col_sum=cs, act_col=ac)
    N.grouped_scaled_act_fwd(act, "mxfp8", sp, W_IN, x, p, None, fc)
    torch.cuda.synchronize()
    assert torch.equal(ac.data, fc.data) and torch.equal(ac.scales, fc.scales), "recompute != forward"
    off, coff = Q.group_offsets(splits), Q.col_offsets(splits)
    assert coff[empty + 1] == coff[empty]                       # an empty expert has no columns
    assert np.all(f32(cs[empty]) == 0.0)                         # and a zero bias gradient
    got_row, ref_row, got_col, ref_col, got_act, ref_act = [], [], [], [], [], []
    for g in (largest, small, mid):
        mg, r0, c0 = int(splits[g]), int(off[g]), int(coff[g])
        mp = int(coff[g + 1] - coff[g])
        nb = -(-mg // 128)
        whole = g != largest
        blocks = range(nb) if whole else sorted({0, nb // 2, nb - 1})
        dx_bits_all, dx32_all = [], []
        for j in blocks:
            t0 = 128 * j
            nt = min(128, mg - t0)
            rows = np.arange(r0 + t0, r0 + t0 + nt)
            xr, dyr = bf16_f64(d["x"][rows]), bf16_f64(d["dy"][rows])
            pr = d["p"][rows].astype(np.float64)
            dx32, dpr = A.scaled_act_bwd("clamped_swiglu", xr, dyr, pr, limit=LIMIT)
            y = A.scaled_act_fwd("clamped_swiglu", xr, pr, limit=LIMIT)
            # dense dL/dx and dprobs of these rows
            got_dx = bf16_host(dx[r0 + t0: r0 + t0 + nt])
            dx_bits_all.append(_dense_dx_ok(got_dx, dx32, xr, dyr, pr, F))
            dx32_all.append(dx32)
            a = A.act("clamped_swiglu", xr, limit=LIMIT)
            bound = (F + 8) * 2.0 ** -24 * np.sum(np.abs(dyr * a), axis=1) + 1e-30
            assert np.all(np.abs(f32(dp[r0 + t0: r0 + t0 + nt]) - dpr) <= bound)
            # rowwise and columnwise quantized dL/dx, and the recomputed FC2 input, of this block
            qdx = Q.quantize_grouped(dx32, [nt], "mxfp8")
            qy = Q.quantize_grouped(y, [nt], "mxfp8", rowwise=False)
            gd, gs = _gpu_rows(dxr, m, W_IN, rows)
            got_row.append(_mx(gd, gs))
            ref_row.append(_mx(qdx["row_data"].reshape(nt, W_IN), Q.mx_scales_from_kstep(qdx["row_scales"], nt, W_IN)))
            gd, gs = _gpu_col_block(dxc, W_IN, c0, mp, t0)
            got_col.append(_mx(gd, gs))
            ref_col.append(_mx(qdx["col_data"].reshape(W_IN, 128), Q.mx_scales_from_kstep(qdx["col_scales"], W_IN, 128)))
            gd, gs = _gpu_col_block(ac, F, c0, mp, t0)
            got_act.append(_mx(gd, gs))
            ref_act.append(_mx(qy["col_data"].reshape(F, 128), Q.mx_scales_from_kstep(qy["col_scales"], F, 128)))
        if whole:
            # per-expert column sums of the dense BF16 dL/dx (FC1's bias gradient)
            v = bf16_f64(np.concatenate(dx_bits_all))
            mag = np.abs(v).sum(axis=0)
            bound = (mg + 1) * 2.0 ** -24 * mag + 2.0 ** -7 * mag + 1e-30
            assert np.all(np.abs(f32(cs[g]) - v.sum(axis=0)) <= bound), g
    flat = lambda lst: tuple(np.concatenate([t[i].reshape(-1) for t in lst]) for i in range(3))
    for name, got, ref in (("dx rowwise", got_row, ref_row), ("dx columnwise", got_col, ref_col),
                           ("recomputed FC2 input", got_act, ref_act)):
        nd, n = compare_quantized("mxfp8", flat(got), flat(ref))
        print(name, "%d of %d codes differ" % (nd, n), flush=True)


def test_fc2_gemms_full_size_identical_operands(N, wl):
    """FC2's FPROP, DGRAD and WGRAD launches at the workload's full shape (FP32 outputs), each checked
    on sampled output rows of four experts against the oracle GEMM on operands that are byte-identical
    to the GPU's (the identity quantizer is exact on both sides, asserted per checked piece): the
    weight W2 [32 x 7168 x 2048], dY2 [65536 x 7168] and an activation-shaped FC2 input [65536 x 2048]
    (the workload's upstream-gradient draw).  An empty expert's weight gradient is zero."""
    import torch
    d = wl
    splits = d["splits"]
    sp = list(map(int, splits))
    m = int(splits.sum())
    largest, small, mid, empty = _checked_groups(splits)
    print("case: FC2 fprop/dgrad/wgrad, 32 experts x 65536 tokens, 2048 -> 7168; experts",
          largest, small, mid, empty, flush=True)
    rng = np.random.default_rng(17)
    w2r, w2c = N.QTensor("mxfp8", False, [H] * E, F), N.QTensor("mxfp8", True, [H] * E, F)
    N.grouped_mx_quantize("mxfp8", [H] * E, F, to_dev_bf16(d["w2"].reshape(E * H, F)), w2r, w2c)
    y2r, y2c = N.QTensor("mxfp8", False, sp, H), N.QTensor("mxfp8", True, sp, H)
    N.grouped_mx_quantize("mxfp8", sp, H, to_dev_bf16(d["dy2"]), y2r, y2c)
    ar, acl = N.QTensor("mxfp8", False, sp, F), N.QTensor("mxfp8", True, sp, F)
    N.grouped_mx_quantize("mxfp8", sp, F, to_dev_bf16(d["dy"]), ar, acl)
    c_fp = torch.empty((m, H), dtype=torch.float32, device="cuda")
    N.grouped_gemm_mx("fprop", "mxfp8", sp, m, H, F, ar, w2r, c_fp)
    c_dg = torch.empty((m, F), dtype=torch.float32, device="cuda")
    N.grouped_gemm_mx("dgrad", "mxfp8", sp, m, F, H, y2r, w2c, c_dg)
    c_wg = torch.full((E, H, F), 7.0, dtype=torch.float32, device="cuda")
    N.grouped_gemm_mx("wgrad", "mxfp8", sp, H, F, m, y2c, acl, c_wg)
    torch.cuda.synchronize()
    assert bool((c_wg[empty] == 0).all()), "empty expert: weight gradient not zero"
    off, coff = Q.group_offsets(splits), Q.col_offsets(splits)
    for g in (largest, small, mid):
        mg, r0, c0 = int(splits[g]), int(off[g]), int(coff[g])
        mp = int(coff[g + 1] - coff[g])
        # the expert's weight, both copies, byte-identical to the oracle's
        qw = Q.quantize_grouped(bf16_f64(d["w2"][g]), [H], "mxfp8")
        gwd, gws = _gpu_rows(w2r, E * H, F, np.arange(g * H, (g + 1) * H))
        assert np.array_equal(gwd, qw["row_data"].reshape(H, F))
        assert np.array_equal(gws, Q.mx_scales_from_kstep(qw["row_scales"], H, F))
        wc0 = g * H                               # padded offset of expert g in [H] * E (H % 128 == 0)
        assert np.array_equal(u8(w2c.data[F * wc0: F * (wc0 + H)]), qw["col_data"])
        assert np.array_equal(u8(w2c.scales[F * wc0 // 32: F * (wc0 + H) // 32]), qw["col_scales"])
        w_row = G.dequant_rows("mxfp8", qw["row_data"], qw["row_scales"], H, F)          # [H x F]
        w_col = G.dequant_rows("mxfp8", qw["col_data"], qw["col_scales"], F, H)          # [F x H]
        rows = np.sort(rng.choice(np.arange(r0, r0 + mg), size=min(16, mg), replace=False))
        # FPROP rows: A rows (identity quantization of the activation-shaped input) . W2_g^T
        qa = Q.quantize_grouped(bf16_f64(d["dy"][rows]), [len(rows)], "mxfp8", colwise=False)
        gad, gas = _gpu_rows(ar, m, F, rows)
        assert np.array_equal(gad, qa["row_data"].reshape(len(rows), F))
        assert np.array_equal(gas, Q.mx_scales_from_kstep(qa["row_scales"], len(rows), F))
        ref = G.dequant_rows("mxfp8", qa["row_data"], qa["row_scales"], len(rows), F) @ w_row.T
        err = rel_rms(f32(c_fp[torch.as_tensor(rows, device="cuda")]), ref)
        assert err <= TOL, ("fprop", g, err)
        # DGRAD rows: dY2 rows . W2_g (its columnwise copy)
        qd = Q.quantize_grouped(bf16_f64(d["dy2"][rows]), [len(rows)], "mxfp8", colwise=False)
        gdd, gds = _gpu_rows(y2r, m, H, rows)
        assert np.array_equal(gdd, qd["row_data"].reshape(len(rows), H))
        assert np.array_equal(gds, Q.mx_scales_from_kstep(qd["row_scales"], len(rows), H))
        ref = G.dequant_rows("mxfp8", qd["row_data"], qd["row_scales"], len(rows), H) @ w_col.T
        err_d = rel_rms(f32(c_dg[torch.as_tensor(rows, device="cuda")]), ref)
        assert err_d <= TOL, ("dgrad", g, err_d)
        # WGRAD output rows S: columns S of dY2 over the expert's tokens . the FC2 input's columnwise copy
        S = np.sort(rng.choice(H, size=64, replace=False))
        qs = Q.quantize_grouped(bf16_f64(d["dy2"][r0:r0 + mg][:, S]), [mg], "mxfp8", rowwise=False)
        ys = u8(y2c.data[H * c0: H * (c0 + mp)].view(H, mp)[torch.as_tensor(S, device="cuda")])
        assert np.array_equal(ys.reshape(-1), qs["col_data"])
        ys_s = Q.mx_scales_from_kstep(u8(y2c.scales[H * c0 // 32: H * (c0 + mp) // 32]), H, mp)[S]
        assert np.array_equal(ys_s, Q.mx_scales_from_kstep(qs["col_scales"], len(S), mp))
        qb = Q.quantize_grouped(bf16_f64(d["dy"][r0:r0 + mg]), [mg], "mxfp8", rowwise=False)
        assert np.array_equal(u8(acl.data[F * c0: F * (c0 + mp)]), qb["col_data"])
        assert np.array_equal(u8(acl.scales[F * c0 // 32: F * (c0 + mp) // 32]), qb["col_scales"])
        ref = (G.dequant_rows("mxfp8", qs["col_data"], qs["col_scales"], len(S), mp)
               @ G.dequant_rows("mxfp8", qb["col_data"], qb["col_scales"], F, mp).T)
        err_w = rel_rms(f32(c_wg[g][torch.as_tensor(S, device="cuda")]), ref)
        assert err_w <= TOL, ("wgrad", g, err_w)
        print("expert %d (%d tokens): rel-RMS fprop %.2e dgrad %.2e wgrad %.2e" % (g, mg, err, err_d, err_w),
              flush=True)


def test_fc2_fprop_chained_after_the_fused_forward(N, wl):
    """FC2 FPROP (BF16 output) on the fused clamped-SwiGLU forward's rowwise output, as the forward
    step chains them: the forward's codes on sampled rows satisfy the agreement criterion against the
    oracle (<= 0.1 % of codes, each <= 1 step), and the GEMM rows agree with the oracle's product of
    its own quantized rows (rounded to BF16) within 1e-3."""
    import torch
    d = wl
    splits = d["splits"]
    sp = list(map(int, splits))
    m = int(splits.sum())
    largest, small, mid, _ = _checked_groups(splits)
    rng = np.random.default_rng(9)
    act = N.act_params("clamped_swiglu", limit=LIMIT)
    qa = N.QTensor("mxfp8", False, sp, F)
    N.grouped_scaled_act_fwd(act, "mxfp8", sp, W_IN, to_dev_bf16(d["x"]), to_dev(d["p"]), qa, None)
    qw = N.QTensor("mxfp8", False, [H] * E, F)
    N.grouped_mx_quantize("mxfp8", [H] * E, F, to_dev_bf16(d["w2"].reshape(E * H, F)), qw, None)
    c = torch.empty((m, H), dtype=torch.bfloat16, device="cuda")
    N.grouped_gemm_mx("fprop", "mxfp8", sp, m, H, F, qa, qw, c)
    torch.cuda.synchronize()
    off = Q.group_offsets(splits)
    got_q, ref_q = [], []
    for g in (largest, small, mid):
        rows = np.sort(rng.choice(np.arange(off[g], off[g + 1]), size=min(16, int(splits[g])), replace=False))
        y = A.scaled_act_fwd("clamped_swiglu", bf16_f64(d["x"][rows]), d["p"][rows].astype(np.float64), limit=LIMIT)
        qrow = Q.quantize_grouped(y, [len(rows)], "mxfp8", colwise=False)
        gd, gs = _gpu_rows(qa, m, F, rows)
        got_q.append(_mx(gd, gs))
        ref_q.append(_mx(qrow["row_data"].reshape(len(rows), F), Q.mx_scales_from_kstep(qrow["row_scales"], len(rows), F)))
        qwg = Q.quantize_grouped(bf16_f64(d["w2"][g]), [H], "mxfp8", colwise=False)
        gwd, gws = _gpu_rows(qw, E * H, F, np.arange(g * H, (g + 1) * H))
        assert np.array_equal(gwd, qwg["row_data"].reshape(H, F))
        assert np.array_equal(gws, Q.mx_scales_from_kstep(qwg["row_scales"], H, F))
        ref = (G.dequant_rows("mxfp8", qrow["row_data"], qrow["row_scales"], len(rows), F)
               @ G.dequant_rows("mxfp8", qwg["row_data"], qwg["row_scales"], H, F).T)
        ref_b = bf16_f64(codecs.f32_to_bf16_bits(codecs.f32(ref).astype(np.float32)))
        got_c = bf16_f64(bf16_host(c[torch.as_tensor(rows, device="cuda")]))
        assert rel_rms(got_c, ref_b) <= TOL, (g, rel_rms(got_c, ref_b))
    flat = lambda lst: tuple(np.concatenate([t[i].reshape(-1) for t in lst]) for i in range(3))
    compare_quantized("mxfp8", flat(got_q), flat(ref_q))
