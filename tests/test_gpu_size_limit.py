"""Parity at the largest tensors the quantizing calls accept.

A columnwise copy is addressed with 32-bit offsets inside one group, so the C ABI rejects a group
whose padded columnwise matrix reaches 2^31 elements.  Here one expert holds 524,155 tokens of width
4096: padded to 524,160 tokens, its columnwise matrix has 2^31 - 2^19 elements and its BF16 input is
4.3 GB; the last 32-token panel is partial (27 real rows).  Inputs are drawn on the device from a
seeded generator (only the rows checked are copied back).  Rowwise and columnwise quantization are
local to a row and to a 32-token block of one column, so the oracle on the first and last rows (and
the first and last 128-token blocks) fixes exactly those outputs; ScaledSReLU is bit-exact.  The FC2
FPROP at that M (N = 256, K = 4096) is checked on the same rows by the GEMM criterion.
"""

import numpy as np
import pytest

from oracle import activations as A
from oracle import gemm as G
from oracle import quant as Q
from tests.helpers import bf16_f64, bf16_host, f32, rel_rms

pytestmark = pytest.mark.gpu

M_TOK, W = 524155, 4096
MP = 524160                       # roundup(M_TOK, 128): MP * W = 2^31 - 2^19


@pytest.fixture(scope="module")
def big():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert MP * W < 2 ** 31 and (MP + 128) * W >= 2 ** 31
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    x = torch.randn((M_TOK, W), generator=g, device="cuda").to(torch.bfloat16)
    dy = torch.randn((M_TOK, W), generator=g, device="cuda").to(torch.bfloat16)
    p = torch.rand(M_TOK, generator=g, device="cuda")
    return x, dy, p


def _rows(t, r0, r1):
    return t[r0:r1].cpu()


def _check_row_slices(qr, x, p, r0, r1):
    """Rowwise MXFP8 codes and K-step-grouped scales of rows r0..r1 against the oracle."""
    xs, ps = bf16_f64(bf16_host(_rows(x, r0, r1))), f32(_rows(p, r0, r1))
    ref = Q.quantize_grouped(A.scaled_act_fwd("srelu", xs, ps), [r1 - r0], "mxfp8", colwise=False)
    got = qr.data.view(M_TOK, W)[r0:r1].cpu().numpy().reshape(-1)
    assert np.array_equal(got, ref["row_data"])
    # scales: byte (row r, block kb) at ((kb // 4) * M + r) * 4 + kb % 4
    sc = qr.scales.view(W // 128, M_TOK, 4)[:, r0:r1, :].cpu().numpy()
    ref_sc = ref["row_scales"].reshape(W // 128, r1 - r0, 4)
    assert np.array_equal(sc, ref_sc)


def _check_col_block(qc, x, p, t0):
    """Columnwise MXFP8 copy of tokens t0..t0+127 (zero padding past the group) against the oracle."""
    t1 = min(t0 + 128, M_TOK)
    xs, ps = bf16_f64(bf16_host(_rows(x, t0, t1))), f32(_rows(p, t0, t1))
    y = np.zeros((128, W))
    y[:t1 - t0] = A.scaled_act_fwd("srelu", xs, ps)
    ref = Q.quantize_grouped(y, [128], "mxfp8", rowwise=False)       # one [W x 128] block
    data = qc.data.view(W, MP)[:, t0:t0 + 128].cpu().numpy()
    assert np.array_equal(data.reshape(-1), ref["col_data"])
    # scales K-step grouped over [W x MP]: the block's 4 scales of column c at ((t0 / 128) * W + c) * 4
    sc = qc.scales.view(MP // 128, W, 4)[t0 // 128].cpu().numpy()
    assert np.array_equal(sc.reshape(-1), ref["col_scales"])


def test_act_fwd_at_the_size_limit(big):
    import torch
    from moe_grouped_scaled_amd import _native as N
    x, _, p = big
    qr, qc = N.QTensor("mxfp8", False, [M_TOK], W), N.QTensor("mxfp8", True, [M_TOK], W)
    N.grouped_scaled_act_fwd(N.act_params("srelu"), "mxfp8", [M_TOK], W, x, p, qr, qc)
    torch.cuda.synchronize()
    for r0, r1 in ((0, 64), (M_TOK - 96, M_TOK)):
        _check_row_slices(qr, x, p, r0, r1)
    for t0 in (0, MP - 128):
        _check_col_block(qc, x, p, t0)


def test_act_bwd_at_the_size_limit(big):
    """Backward at the limit: rowwise and columnwise dL/dx, dprobs and the recomputed FC2 input, on
    the last 128-token block (its columnwise dx and recompute) and the last rows."""
    import torch
    from moe_grouped_scaled_amd import _native as N
    x, dy, p = big
    act = N.act_params("srelu")
    dxr, dxc = N.QTensor("mxfp8", False, [M_TOK], W), N.QTensor("mxfp8", True, [M_TOK], W)
    ac = N.QTensor("mxfp8", True, [M_TOK], W)
    dp = torch.empty(M_TOK, dtype=torch.float32, device="cuda")
    N.grouped_scaled_act_bwd(act, "mxfp8", [M_TOK], W, x, dy, p, dx_row=dxr, dx_col=dxc, dprobs=dp, act_col=ac)
    torch.cuda.synchronize()
    t0 = MP - 128
    xs, ds, ps = bf16_f64(bf16_host(_rows(x, t0, M_TOK))), bf16_f64(bf16_host(_rows(dy, t0, M_TOK))), f32(_rows(p, t0, M_TOK))
    n = M_TOK - t0
    dx32, dpr = A.scaled_act_bwd("srelu", xs, ds, ps)
    ref_r = Q.quantize_grouped(dx32, [n], "mxfp8", colwise=False)
    assert np.array_equal(dxr.data.view(M_TOK, W)[t0:].cpu().numpy().reshape(-1), ref_r["row_data"])
    pad = np.zeros((128, W))
    pad[:n] = dx32
    ref_c = Q.quantize_grouped(pad, [128], "mxfp8", rowwise=False)
    assert np.array_equal(dxc.data.view(W, MP)[:, t0:].cpu().numpy().reshape(-1), ref_c["col_data"])
    assert np.array_equal(dxc.scales.view(MP // 128, W, 4)[t0 // 128].cpu().numpy().reshape(-1), ref_c["col_scales"])
    _check_col_block(ac, x, p, t0)                     # recompute = the forward's columnwise copy
    got_dp = f32(dp[t0:].cpu())
    bound = (W + 8) * 2.0 ** -24 * np.sum(np.abs(ds * A.act("srelu", xs)), axis=1)
    assert np.all(np.abs(got_dp - dpr) <= bound)


def test_fprop_at_the_size_limit(big):
    """FC2 FPROP with M = 524,155 tokens (A is 2^31 - 2^19 - 20,480 bytes of codes), N = 256:
    the first and last rows against the oracle on the same quantized operands."""
    import torch
    from moe_grouped_scaled_amd import _native as N
    x, _, p = big
    n = 256
    qa = N.QTensor("mxfp8", False, [M_TOK], W)
    N.grouped_scaled_act_fwd(N.act_params("srelu"), "mxfp8", [M_TOK], W, x, p, qa, None)
    g = torch.Generator(device="cuda")
    g.manual_seed(8)
    w = (torch.randn((n, W), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    qw = N.QTensor("mxfp8", False, [n], W)
    N.grouped_mx_quantize("mxfp8", [n], W, w, qw)
    c = torch.empty((M_TOK, n), dtype=torch.float32, device="cuda")
    N.grouped_gemm_mx("fprop", "mxfp8", [M_TOK], M_TOK, n, W, qa, qw, c)
    torch.cuda.synchronize()
    wd = G.dequant_rows("mxfp8", qw.data.cpu().numpy(), qw.scales.cpu().numpy(), n, W)
    for r0, r1 in ((0, 256), (M_TOK - 300, M_TOK)):
        codes = qa.data.view(M_TOK, W)[r0:r1].cpu().numpy().reshape(-1)
        # the rows' scales, sliced out of the K-step grouped array, are that sub-matrix's own layout
        sc = qa.scales.view(W // 128, M_TOK, 4)[:, r0:r1, :].cpu().numpy().reshape(-1)
        ad = G.dequant_rows("mxfp8", codes, sc, r1 - r0, W)
        ref = ad @ wd.T
        assert rel_rms(f32(c[r0:r1].cpu()), ref) <= 1e-3
