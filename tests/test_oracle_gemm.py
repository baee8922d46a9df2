"""Pins of the oracle's grouped GEMM: exact integer special cases, grouping, transposed operands."""

import numpy as np

from oracle import codecs, quant
from oracle.gemm import (
    dequant_col_grouped,
    dgrad_weight,
    dequant_row_grouped,
    dequant_rows,
    gemm_grouped_k,
    gemm_grouped_m,
    rel_rms_error,
)
from oracle.mlp import mlp_step

E4M3_INT = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48}


def _e4m3_int_codes(v):
    c = np.vectorize(lambda a: E4M3_INT[abs(int(a))])(v).astype(np.uint8)
    return c | (np.where(v < 0, 0x80, 0)).astype(np.uint8)


def test_unit_scale_integer_gemm_is_exact_int_matmul():
    rng = np.random.default_rng(0)
    splits = [3, 0, 40, 21]
    m, n, k = sum(splits), 48, 96
    a_int = rng.integers(-4, 5, (m, k))
    b_int = rng.integers(-4, 5, (len(splits), n, k))
    unit = lambda r: quant.mx_scales_to_kstep(np.full((r, k // 32), 127, np.uint8))
    a = dequant_rows(quant.MXFP8, _e4m3_int_codes(a_int), unit(m), m, k)
    bs = [dequant_rows(quant.MXFP8, _e4m3_int_codes(b_int[g]), unit(n), n, k)
          for g in range(len(splits))]
    c = gemm_grouped_m(a, bs, splits)
    off = quant.group_offsets(splits)
    for g in range(len(splits)):
        want = a_int[off[g]:off[g + 1]] @ b_int[g].T
        assert np.array_equal(c[off[g]:off[g + 1]], want.astype(np.float64))


def test_nvfp4_unit_scale_integer_gemm_is_exact():
    rng = np.random.default_rng(1)
    vals = np.array([0, 1, 2, 3, 4, 6])
    code_of = {0: 0, 1: 2, 2: 4, 3: 5, 4: 6, 6: 7}
    a_int = rng.choice(vals, (8, 32)) * rng.choice([-1, 1], (8, 32))
    b_int = rng.choice(vals, (5, 32)) * rng.choice([-1, 1], (5, 32))

    def enc(v):
        c = np.vectorize(lambda x: code_of[abs(int(x))])(v).astype(np.uint8)
        return codecs.pack_e2m1(c | (np.where(v < 0, 8, 0)).astype(np.uint8))

    ones = np.full(8 * 2, 0x38, np.uint8)   # E4M3 1.0 block scales
    a = dequant_rows(quant.NVFP4, enc(a_int), ones, 8, 32, 1.0)
    b = dequant_rows(quant.NVFP4, enc(b_int), ones[:10], 5, 32, 1.0)
    assert np.array_equal(a @ b.T, (a_int @ b_int.T).astype(np.float64))


def test_dgrad_and_wgrad_through_transposed_copies_exact_for_representable_values():
    """Small integers in [-4, 4] are exact under any MXFP8 block scale, so the rowwise and columnwise
    copies both dequantize to the same matrix: dgrad via the columnwise weight equals dY @ W, and wgrad
    via the columnwise copies equals dY^T @ X per group, exactly."""
    rng = np.random.default_rng(2)
    splits = [32, 0, 45, 64]
    e, m, n, k = len(splits), sum(splits), 64, 96
    w_int = rng.integers(-4, 5, (e, n, k)).astype(np.float64)
    dy_int = rng.integers(-4, 5, (m, n)).astype(np.float64)
    x_int = rng.integers(-4, 5, (m, k)).astype(np.float64)
    qw = quant.quantize_grouped(w_int.reshape(e * n, k), [n] * e, quant.MXFP8)
    w_col = dequant_col_grouped(quant.MXFP8, qw["col_data"], qw["col_scales"], [n] * e, k)  # [K x NP]
    assert w_col[0].shape == (k, 128) and np.all(w_col[0][:, n:] == 0)
    w_col = dgrad_weight(w_col, n)
    qdy = quant.quantize_grouped(dy_int, splits, quant.MXFP8)
    dy_row = dequant_row_grouped(quant.MXFP8, qdy["row_data"], qdy["row_scales"], splits, n)
    dx = gemm_grouped_m(dy_row, w_col, splits)
    off = quant.group_offsets(splits)
    for g in range(e):
        assert np.array_equal(dx[off[g]:off[g + 1]], dy_int[off[g]:off[g + 1]] @ w_int[g])
    qx = quant.quantize_grouped(x_int, splits, quant.MXFP8)
    dw = gemm_grouped_k(dequant_col_grouped(quant.MXFP8, qdy["col_data"], qdy["col_scales"], splits, n),
                        dequant_col_grouped(quant.MXFP8, qx["col_data"], qx["col_scales"], splits, k))
    assert dw.shape == (e, n, k)
    for g in range(e):
        assert np.array_equal(dw[g], dy_int[off[g]:off[g + 1]].T @ x_int[off[g]:off[g + 1]])
    assert np.all(dw[1] == 0)   # empty group -> zero weight gradient


def test_bias_added_per_group():
    a = np.ones((5, 32))
    b = [np.ones((4, 32)), np.ones((4, 32))]
    bias = np.array([[1, 2, 3, 4], [10, 20, 30, 40]], dtype=np.float64)
    c = gemm_grouped_m(a, b, [2, 3], bias=bias)
    assert c[0].tolist() == [33, 34, 35, 36] and c[4].tolist() == [42, 52, 62, 72]


def test_rel_rms_error():
    assert rel_rms_error(np.array([1.0, 1.0]), np.array([1.0, 1.0])) == 0.0
    assert abs(rel_rms_error(np.array([1.1, 0.0]), np.array([1.0, 0.0])) - 0.1) < 1e-12


def test_mlp_step_wgrad_close_to_unquantized():
    """The quantized step's weight gradients sit within MXFP8 quantization error of the plain
    float64 step on the same forward values (relative RMS of a few percent)."""
    rng = np.random.default_rng(3)
    splits = [32, 64, 0, 32]
    e, m, h, f = 4, 128, 64, 64
    bf = lambda a: codecs.bf16_bits_to_f64(codecs.f32_to_bf16_bits(a.astype(np.float32)))
    x1 = bf(rng.standard_normal((m, h)))
    w1 = bf(rng.standard_normal((e, f, h)) * 0.1)
    w2 = bf(rng.standard_normal((e, h, f)) * 0.1)
    b1 = bf(rng.standard_normal((e, f)) * 0.1)
    b2 = bf(rng.standard_normal((e, h)) * 0.1)
    p = codecs.f32(rng.random(m))
    dy2 = bf(rng.standard_normal((m, h)))
    r = mlp_step("srelu", quant.MXFP8, splits, x1, w1, b1, w2, b2, p, dy2)
    off = quant.group_offsets(splits)
    for g in range(e):
        sl = slice(off[g], off[g + 1])
        ref_dw2 = dy2[sl].T @ r["a32"][sl]
        if splits[g] == 0:
            assert np.all(r["dw2"][g] == 0)
            continue
        assert rel_rms_error(r["dw2"][g], ref_dw2) < 0.06
        assert np.allclose(r["db2"][g], dy2[sl].sum(axis=0))
    assert r["y2"].shape == (m, h) and r["dx1"].shape == (m, h) and r["dp"].shape == (m,)
