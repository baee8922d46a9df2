"""GPU parity of the grouped MX GEMM (FPROP / DGRAD / WGRAD, MXFP8 and NVFP4) against the oracle.

Operands are quantized by the oracle (bytes copied to the GPU), so the GEMM is checked on its own.
Criterion: ||C - C_ref||_2 / ||C_ref||_2 <= 1e-3 over the tensor and per non-empty group, FP32 output
(BF16 output is compared with the oracle result rounded to BF16); integer special cases are exact.
"""

import numpy as np
import pytest

import workloads
from oracle import codecs
from oracle import gemm as G
from oracle import quant as Q
from tests.helpers import bf16_f64, bf16_host, f32, rel_rms, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu
TOL = 1e-3


@pytest.fixture(scope="module")
def N():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from moe_grouped_scaled_amd import _native
    return _native


def dev_q(N, fmt, colwise, splits, width, q):
    import torch
    t = N.QTensor(fmt, colwise, splits, width)
    pre = "col" if colwise else "row"
    t.data.copy_(torch.from_numpy(np.ascontiguousarray(q[pre + "_data"])))
    t.scales.copy_(torch.from_numpy(np.ascontiguousarray(q[pre + "_scales"])))
    if fmt == "nvfp4":
        t.group_scale.copy_(torch.from_numpy(q["group_scale"].astype(np.float32)))
    return t


def _f32_values(rng, shape, std=1.0):
    return bf16_f64(workloads.normal_bf16(rng, shape, std))


def check_groups(got, ref, splits, axis_rows=True):
    assert rel_rms(got, ref) <= TOL, rel_rms(got, ref)
    if axis_rows:
        off = Q.group_offsets(splits)
        for g in range(len(splits)):
            if splits[g]:
                assert rel_rms(got[off[g]:off[g + 1]], ref[off[g]:off[g + 1]]) <= TOL, g


def test_integer_codes_unit_scales_exact(N):
    """All scale codes 127 (1.0) and small-integer E4M3 codes: the result is the integer matmul."""
    import torch
    rng = np.random.default_rng(0)
    splits = [3, 0, 130, 61]
    m, n, k = sum(splits), 160, 288
    enc = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48}
    a_int = rng.integers(-4, 5, (m, k))
    b_int = rng.integers(-4, 5, (len(splits), n, k))

    def codes(v):
        c = np.vectorize(lambda t: enc[abs(int(t))])(v).astype(np.uint8)
        return c | np.where(v < 0, 0x80, 0).astype(np.uint8)

    unit = lambda r: Q.mx_scales_to_kstep(np.full((r, k // 32), 127, np.uint8))
    qa = {"row_data": codes(a_int).reshape(-1), "row_scales": unit(m)}
    qb = {"row_data": codes(b_int).reshape(-1), "row_scales": unit(len(splits) * n)}
    A = dev_q(N, "mxfp8", False, splits, k, qa)
    B = dev_q(N, "mxfp8", False, [n] * len(splits), k, qb)
    c = torch.empty((m, n), dtype=torch.float32, device="cuda")
    N.grouped_gemm_mx("fprop", "mxfp8", splits, m, n, k, A, B, c)
    torch.cuda.synchronize()
    got = f32(c)
    off = Q.group_offsets(splits)
    for g in range(len(splits)):
        want = (a_int[off[g]:off[g + 1]] @ b_int[g].T).astype(np.float64)
        assert np.array_equal(got[off[g]:off[g + 1]], want)


@pytest.mark.parametrize("fmt", ["mxfp8", "nvfp4"])
@pytest.mark.parametrize("k", [32, 128, 160, 256, 384, 640])
def test_integer_products_exact_for_every_step_count(N, fmt, k):
    """Small-integer codes with unit scales give the integer matmul exactly for one to five K steps of
    128, whole or with a partial last step: the K loop ends on different paths for odd and even step
    counts and for a partial step, and the accumulators must be complete on each."""
    import torch
    rng = np.random.default_rng(k)
    splits = [3, 0, 130, 61]
    e, m, n = len(splits), sum(splits), 160
    if fmt == "mxfp8":
        vals = np.array([0, 1, 2, 3, 4])
        enc = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48}           # E4M3 codes of 0..4
    else:
        vals = np.array([0, 1, 2, 3, 4, 6])
        enc = {0: 0, 1: 2, 2: 4, 3: 5, 4: 6, 6: 7}                     # E2M1 codes of 0..6
    sign = 0x80 if fmt == "mxfp8" else 0x8
    a_int = rng.choice(vals, (m, k)) * rng.choice([-1, 1], (m, k))
    b_int = rng.choice(vals, (e, n, k)) * rng.choice([-1, 1], (e, n, k))

    def codes(v):
        c = np.vectorize(lambda t: enc[abs(int(t))])(v).astype(np.uint8)
        c = c | np.where(v < 0, sign, 0).astype(np.uint8)
        return c if fmt == "mxfp8" else codecs.pack_e2m1(c)

    def unit(rows, groups):
        if fmt == "mxfp8":
            return {"row_scales": Q.mx_scales_to_kstep(np.full((rows, k // 32), 127, np.uint8))}
        return {"row_scales": np.full(rows * (k // 16), 0x38, np.uint8), "group_scale": np.ones(groups, np.float32)}

    A = dev_q(N, fmt, False, splits, k, {"row_data": codes(a_int).reshape(-1), **unit(m, e)})
    B = dev_q(N, fmt, False, [n] * e, k, {"row_data": codes(b_int).reshape(e * n, k).reshape(-1) if fmt == "mxfp8"
                                          else codes(b_int.reshape(e * n, k)).reshape(-1), **unit(e * n, e)})
    c = torch.empty((m, n), dtype=torch.float32, device="cuda")
    N.grouped_gemm_mx("fprop", fmt, splits, m, n, k, A, B, c)
    torch.cuda.synchronize()
    got = f32(c)
    off = Q.group_offsets(splits)
    for g in range(e):
        want = (a_int[off[g]:off[g + 1]] @ b_int[g].T).astype(np.float64)
        assert np.array_equal(got[off[g]:off[g + 1]], want), (fmt, k, g)


@pytest.mark.parametrize("fmt", ["mxfp8", "nvfp4"])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_fprop_dgrad(N, fmt, out_dtype):
    import torch
    rng = np.random.default_rng(1)
    splits = [0, 100, 37, 256]
    e, m, n, k = len(splits), sum(splits), 160, 544      # M, N and K tails
    x = _f32_values(rng, (m, k))
    w = _f32_values(rng, (e, n, k), 0.02)
    bias_bits = workloads.normal_bf16(rng, (e, n), 0.02)
    qx = Q.quantize_grouped(x, splits, fmt, colwise=False)
    qw = Q.quantize_grouped(w.reshape(e * n, k), [n] * e, fmt)
    A = dev_q(N, fmt, False, splits, k, qx)
    B = dev_q(N, fmt, False, [n] * e, k, qw)
    a_ref = G.dequant_row_grouped(fmt, qx["row_data"], qx["row_scales"], splits, k, qx.get("group_scale"))
    w_ref = G.dequant_row_grouped(fmt, qw["row_data"], qw["row_scales"], [n] * e, k, qw.get("group_scale"))
    ref = G.gemm_grouped_m(a_ref, list(w_ref.reshape(e, n, k)), splits, bias=bf16_f64(bias_bits))
    dt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    c = torch.empty((m, n), dtype=dt, device="cuda")
    N.grouped_gemm_mx("fprop", fmt, splits, m, n, k, A, B, c, bias=to_dev_bf16(bias_bits))
    torch.cuda.synchronize()
    if out_dtype == "f32":
        check_groups(f32(c), ref, splits)
    else:
        ref_b = bf16_f64(codecs.f32_to_bf16_bits(codecs.f32(ref).astype(np.float32)))
        check_groups(bf16_f64(bf16_host(c)), ref_b, splits)
    # DGRAD: dX = dY . W_g with W quantized along N (its columnwise copy)
    dy = _f32_values(rng, (m, n))
    qdy = Q.quantize_grouped(dy, splits, fmt, colwise=False)
    Ad = dev_q(N, fmt, False, splits, n, qdy)
    Bd = dev_q(N, fmt, True, [n] * e, k, qw)            # per group [k x n]
    dy_ref = G.dequant_row_grouped(fmt, qdy["row_data"], qdy["row_scales"], splits, n, qdy.get("group_scale"))
    w_col = G.dgrad_weight(G.dequant_col_grouped(fmt, qw["col_data"], qw["col_scales"], [n] * e, k,
                                                 qw.get("group_scale")), n)
    ref_d = G.gemm_grouped_m(dy_ref, w_col, splits)
    cd = torch.empty((m, k), dtype=torch.float32, device="cuda")
    N.grouped_gemm_mx("dgrad", fmt, splits, m, k, n, Ad, Bd, cd)
    torch.cuda.synchronize()
    check_groups(f32(cd), ref_d, splits)


@pytest.mark.parametrize("fmt", ["mxfp8", "nvfp4"])
def test_wgrad_and_accumulate(N, fmt):
    import torch
    rng = np.random.default_rng(2)
    splits = [45, 0, 200, 31, 64]
    e, m_tok, h, f = len(splits), sum(splits), 96, 160
    dy = _f32_values(rng, (m_tok, h))
    a = _f32_values(rng, (m_tok, f))
    qdy = Q.quantize_grouped(dy, splits, fmt, rowwise=False)
    qa = Q.quantize_grouped(a, splits, fmt, rowwise=False)
    A = dev_q(N, fmt, True, splits, h, qdy)
    B = dev_q(N, fmt, True, splits, f, qa)
    ref = G.gemm_grouped_k(G.dequant_col_grouped(fmt, qdy["col_data"], qdy["col_scales"], splits, h, qdy.get("group_scale")),
                           G.dequant_col_grouped(fmt, qa["col_data"], qa["col_scales"], splits, f, qa.get("group_scale")))
    c = torch.full((e, h, f), 7.0, dtype=torch.float32, device="cuda")
    N.grouped_gemm_mx("wgrad", fmt, splits, h, f, m_tok, A, B, c)
    torch.cuda.synchronize()
    got = f32(c)
    assert np.all(got[1] == 0.0)                       # empty group -> zero weight gradient
    assert rel_rms(got, ref) <= TOL
    for g in range(e):
        if splits[g]:
            assert rel_rms(got[g], ref[g]) <= TOL
    # accumulate: C += A_g B_g^T (delayed weight-gradient accumulation)
    init = rng.standard_normal((e, h, f)).astype(np.float32)
    c2 = to_dev(init)
    N.grouped_gemm_mx("wgrad", fmt, splits, h, f, m_tok, A, B, c2, accumulate=True)
    torch.cuda.synchronize()
    assert rel_rms(f32(c2), init + ref) <= TOL
    assert np.array_equal(f32(c2)[1], init[1].astype(np.float64))   # empty group left unchanged


@pytest.mark.parametrize("fmt", ["mxfp8", "nvfp4"])
def test_wgrad_bf16_output(N, fmt):
    """WGRAD into a BF16 weight gradient: the oracle's product rounded to BF16, per group, and zeros
    for an empty group; a K length per group that is not a multiple of the 128-token K step."""
    import torch
    rng = np.random.default_rng(4)
    splits = [0, 300, 17, 129]
    e, m_tok, h, f = len(splits), sum(splits), 128, 224
    dy = _f32_values(rng, (m_tok, h))
    a = _f32_values(rng, (m_tok, f))
    qdy = Q.quantize_grouped(dy, splits, fmt, rowwise=False)
    qa = Q.quantize_grouped(a, splits, fmt, rowwise=False)
    A = dev_q(N, fmt, True, splits, h, qdy)
    B = dev_q(N, fmt, True, splits, f, qa)
    ref = G.gemm_grouped_k(G.dequant_col_grouped(fmt, qdy["col_data"], qdy["col_scales"], splits, h, qdy.get("group_scale")),
                           G.dequant_col_grouped(fmt, qa["col_data"], qa["col_scales"], splits, f, qa.get("group_scale")))
    c = torch.full((e, h, f), 7.0, dtype=torch.bfloat16, device="cuda")
    N.grouped_gemm_mx("wgrad", fmt, splits, h, f, m_tok, A, B, c)
    torch.cuda.synchronize()
    got = bf16_f64(bf16_host(c))
    ref_b = bf16_f64(codecs.f32_to_bf16_bits(codecs.f32(ref).astype(np.float32)))
    assert np.all(got[0] == 0.0)                       # empty group -> zero weight gradient
    for g in range(1, e):
        assert rel_rms(got[g], ref_b[g]) <= TOL, g


FPROP_ACT_CASES = [(k, a) for k in ("srelu", "tanh_srelu", "gelu", "sigmoid", "identity") for a in ("bf16", "fp32")]


@pytest.mark.parametrize("kind,act_input", FPROP_ACT_CASES)
def test_fprop_act_epilogue_equals_separate_forward(N, kind, act_input):
    """FC1 FPROP with the activation + MXFP8 rowwise quantization in its epilogue, against the two
    launches it replaces on the same operands: the plain FPROP (BF16 output, or FP32 output for
    act_input fp32) followed by the fused forward (BF16 input, or FP32 input writing the BF16 copy).
    C and the quantized y must agree bit for bit.  Ragged groups (empty, 1, 31, 33 rows), n = 416
    (the second tile column's second wave holds one 32-column block) and a partial K step."""
    import torch
    rng = np.random.default_rng(7)
    splits = [0, 1, 31, 33, 300, 64]
    e, m, n, k = len(splits), sum(splits), 416, 288
    a = _f32_values(rng, (m, k))
    w = _f32_values(rng, (e * n, k), 0.05)
    qa_o = Q.quantize_grouped(a, splits, "mxfp8", colwise=False)
    qw_o = Q.quantize_grouped(w, [n] * e, "mxfp8", colwise=False)
    qa = dev_q(N, "mxfp8", False, splits, k, qa_o)
    qw = dev_q(N, "mxfp8", False, [n] * e, k, qw_o)
    bias_bits = workloads.normal_bf16(rng, (e, n), 0.5)
    bias = to_dev_bf16(bias_bits)
    p_host = workloads.uniform_f32(rng, m)
    probs = to_dev(p_host) if kind != "identity" else None
    act = N.act_params(kind, s=2.0)
    c = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    qy = N.QTensor("mxfp8", False, splits, n)
    N.grouped_gemm_mx_fprop_act(splits, m, n, k, qa, qw, c, act, probs, qy, bias=bias, act_input=act_input)
    ref_row = N.QTensor("mxfp8", False, splits, n)
    if act_input == "bf16":
        c_ref = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        N.grouped_gemm_mx("fprop", "mxfp8", splits, m, n, k, qa, qw, c_ref, bias=bias)
        N.grouped_scaled_act_fwd(act, "mxfp8", splits, n, c_ref, probs, ref_row)
    else:
        c32 = torch.empty((m, n), dtype=torch.float32, device="cuda")
        N.grouped_gemm_mx("fprop", "mxfp8", splits, m, n, k, qa, qw, c32, bias=bias)
        c_ref = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        N.grouped_scaled_act_fwd_f32(act, "mxfp8", splits, n, c32, probs, ref_row, x_bf16_out=c_ref)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_host(c), bf16_host(c_ref)), "C differs"
    assert np.array_equal(qy.scales.cpu().numpy(), ref_row.scales.cpu().numpy()), "scales differ"
    assert np.array_equal(qy.data.cpu().numpy(), ref_row.data.cpu().numpy()), "codes differ"
    # and against the oracle on its own product of the same operands: C (BF16) within the GEMM
    # criterion, and y = act(C) * p quantized, with C the FP32 accumulator value (act_input fp32, the
    # value the page's fused forward activates) or its BF16 rounding, within the agreement criterion:
    # <= 0.1 % of the codes differ, each by <= 1 step plus the activation's response to the bounded
    # difference of the two C's.  The scaled MFMA reduces its 128 products with less than FP32
    # precision (relative RMS ~1.4e-5 against the exact product on identical operands, where the FP16
    # MFMA gives ~3e-8), which near C = 0 exceeds the finest E4M3 step of a block; per element the
    # difference is taken as at most 2^-12 of the sum of the absolute terms (and, for BF16 input, one
    # BF16 rounding step more).
    from oracle import activations as A
    from tests.helpers import compare_quantized, mx_elementwise
    a_deq = G.dequant_row_grouped("mxfp8", qa_o["row_data"], qa_o["row_scales"], splits, k)
    w_deq = G.dequant_row_grouped("mxfp8", qw_o["row_data"], qw_o["row_scales"], [n] * e, k)
    c64 = G.gemm_grouped_m(a_deq, list(w_deq.reshape(e, n, k)), splits, bias=bf16_f64(bias_bits))
    c32_ref = codecs.f32(c64)
    c_bf = bf16_f64(codecs.f32_to_bf16_bits(c32_ref.astype(np.float32)))
    check_groups(bf16_f64(bf16_host(c)), c_bf, splits)
    x_act = c32_ref if act_input == "fp32" else c_bf
    pp = p_host.astype(np.float64) if probs is not None else np.ones(m)
    y = A.scaled_act_fwd(kind, x_act, pp, s=2.0)
    ref = Q.quantize_grouped(y, splits, "mxfp8", colwise=False)
    absum = G.gemm_grouped_m(np.abs(a_deq), list(np.abs(w_deq).reshape(e, n, k)), splits,
                             bias=np.abs(bf16_f64(bias_bits)))
    d_c = 2.0 ** -12 * absum + (2.0 ** -8 * np.abs(c32_ref) if act_input == "bf16" else 0.0)
    # the largest slope of the activation within d_c of x, by sampling the interval's ends and middle
    slope = np.max([np.abs(A.act_grad(kind, x_act + t * d_c, s=2.0)) for t in (-1.0, 0.0, 1.0)], axis=0)
    extra = 2.0 * slope * pp[:, None] * d_c
    nd, ntot = compare_quantized("mxfp8", mx_elementwise(qy.data.cpu().numpy(), qy.scales.cpu().numpy(), m, n),
                                 mx_elementwise(ref["row_data"], ref["row_scales"], m, n), extra=extra)
    print(kind, act_input, "%d of %d codes differ from the oracle's" % (nd, ntot))
