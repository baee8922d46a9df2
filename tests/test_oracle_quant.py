"""Pins of the oracle's grouped MXFP8 / NVFP4 quantizers: closed forms, error bounds, layouts."""

import numpy as np
import pytest

from oracle import codecs, quant
from oracle.gemm import dequant_col_grouped, dequant_row_grouped


def test_e8m0_scale_closed_forms():
    # X = 2^(floor(log2 amax) - 8): amax 1 -> 2^-8 (code 119); 3.5 -> 2^-7 (120, 3.5/2^-7 = 448 exactly)
    amax = np.array([1.0, 3.5, 448.0, 500.0, 0.0, 2.0 ** -130, 2.0 ** 130])
    assert quant.mxfp8_scale_code(amax).tolist() == [119, 120, 127, 127, 0, 0, 249]


def test_mxfp8_block_examples():
    y = np.zeros((1, 64))
    y[0, :32] = np.linspace(-3.5, 3.5, 32)       # amax 3.5 -> scale 2^-7, max maps to 448 exactly
    y[0, 32] = 500.0                              # amax 500 -> scale 1, 500 saturates to 448
    y[0, 33] = 1.0
    q, s = quant.mxfp8_quantize_rows(y)
    assert s.tolist() == [[120, 127]]
    assert q[0, 31] == 0x7E and q[0, 0] == 0xFE   # +-448
    assert q[0, 32] == 0x7E and q[0, 33] == 0x38  # 448 (saturated) and 1.0
    assert np.all(q[0, 34:] == 0)


def _mx_error_ok(deq, y, block_scale):
    """|deq - clip(y)| <= max(2^-4 |y|, 2^-10 X): half an E4M3 step in the normal and subnormal range."""
    lim = 448.0 * block_scale
    yc = np.clip(y, -lim, lim)
    bound = np.maximum(2.0 ** -4 * np.abs(yc), 2.0 ** -10 * block_scale)
    return np.all(np.abs(deq - yc) <= bound * (1 + 1e-12))


@pytest.mark.parametrize("splits", [[64, 128, 32, 32], [0, 1, 31, 33, 64], [5]])
def test_mxfp8_grouped_roundtrip_bound_and_layout(splits):
    rng = np.random.default_rng(0)
    m, w = sum(splits), 96
    y = codecs.f32(rng.standard_normal((m, w)) * np.exp(rng.uniform(-3, 3, (m, 1))))
    q = quant.quantize_grouped(y, splits, quant.MXFP8)
    nd, ns = quant.qtensor_nbytes(quant.MXFP8, False, splits, w)
    assert q["row_data"].size == nd and q["row_scales"].size == ns
    nd, ns = quant.qtensor_nbytes(quant.MXFP8, True, splits, w)
    assert q["col_data"].size == nd and q["col_scales"].size == ns
    # rowwise: each block dequantizes within half an E4M3 step of its values
    deq = dequant_row_grouped(quant.MXFP8, q["row_data"], q["row_scales"], splits, w)
    xs = codecs.e8m0_decode(quant.mx_scales_from_kstep(q["row_scales"], m, w))
    assert _mx_error_ok(deq, y, np.repeat(xs, 32, axis=1))
    # columnwise: element (token r of group g, column j) sits at [j, r] of group g's [w x mp_g] block
    mats = dequant_col_grouped(quant.MXFP8, q["col_data"], q["col_scales"], splits, w)
    off = quant.group_offsets(splits)
    coff = quant.col_offsets(splits)
    for g, mat in enumerate(mats):
        m_g = off[g + 1] - off[g]
        mp = coff[g + 1] - coff[g]
        assert mat.shape == (w, mp)
        assert np.all(mat[:, m_g:] == 0)                         # padding is zero
        yt = y[off[g]:off[g + 1]].T
        s0 = w * coff[g] // 32
        cs_codes = quant.mx_scales_from_kstep(q["col_scales"][s0:s0 + w * mp // 32], w, mp)
        cs = codecs.e8m0_decode(cs_codes)
        assert _mx_error_ok(mat[:, :m_g], yt, np.repeat(cs, 32, axis=1)[:, :m_g])
        # the column scale is the closed-form code of the amax over the block's real rows only
        for b in range(mp // 32):
            blk = np.abs(yt[:, 32 * b:min(32 * b + 32, m_g)])
            want = quant.mxfp8_scale_code(blk.max(axis=1)) if blk.shape[1] else np.zeros(w, np.uint8)
            assert np.array_equal(cs_codes[:, b], want)   # all-padding blocks get code 0


def test_kstep_scale_layout():
    """Scale byte of (row r, block kb) sits at ((kb // 4) * R + r) * 4 + kb % 4; partial steps padded."""
    codes = np.arange(5 * 3, dtype=np.uint8).reshape(5, 3) + 1       # R = 5 rows, K = 96 (3 blocks)
    flat = quant.mx_scales_to_kstep(codes)
    assert flat.size == 4 * 5 * 1
    for r in range(5):
        for kb in range(3):
            assert flat[((kb // 4) * 5 + r) * 4 + kb % 4] == codes[r, kb]
        assert flat[r * 4 + 3] == 0
    assert np.array_equal(quant.mx_scales_from_kstep(flat, 5, 96), codes)
    wide = np.arange(2 * 8, dtype=np.uint8).reshape(2, 8)             # K = 256: two full steps
    f2 = quant.mx_scales_to_kstep(wide)
    assert f2.tolist() == [0, 1, 2, 3, 8, 9, 10, 11, 4, 5, 6, 7, 12, 13, 14, 15]


def test_mxfp8_colwise_is_rowwise_of_transpose():
    rng = np.random.default_rng(1)
    splits = [128, 32]
    y = codecs.f32(rng.standard_normal((160, 64)))
    q = quant.quantize_grouped(y, splits, quant.MXFP8, rowwise=False)
    qt0 = quant.mxfp8_quantize_rows(y[:128].T)        # a full group: no padding tokens
    assert np.array_equal(q["col_data"][:64 * 128], qt0[0].reshape(-1))
    assert np.array_equal(q["col_scales"][:64 * 128 // 32], quant.mx_scales_to_kstep(qt0[1]))


def _brute_e4m3(v):
    mags = codecs.E4M3_MAGS
    d = np.abs(np.abs(v)[..., None] - mags)
    best = d.min(axis=-1, keepdims=True)
    idx = np.argmax(d == best, axis=-1)   # first (smaller) candidate
    tie = np.sum(d == best, axis=-1) > 1
    idx = np.where(tie & (idx % 2 == 1), idx + 1, idx)
    return idx


@pytest.mark.parametrize("splits", [[512, 512, 512, 512], [0, 16, 48, 100]])
def test_nvfp4_invariants(splits):
    rng = np.random.default_rng(2)
    m, w = sum(splits), 64
    y = codecs.f32(rng.standard_normal((m, w)) * 1.5)
    q = quant.quantize_grouped(y, splits, quant.NVFP4)
    off = quant.group_offsets(splits)
    sc = q["row_scales"].reshape(m, w // 16)
    codes = codecs.unpack_e2m1(q["row_data"].reshape(m, w // 2))
    assert np.all(np.abs(codecs.e2m1_decode(codes)) <= 6)
    for g in range(len(splits)):
        if splits[g] == 0:
            continue
        yg = y[off[g]:off[g + 1]]
        a_g = np.abs(yg).max()
        assert q["group_amax"][g] == a_g
        s_enc = float(codecs.f32(2688.0 / a_g))
        assert q["group_scale"][g] == codecs.f32(1.0 / s_enc)
        sg = sc[off[g]:off[g + 1]]
        # the block holding the group maximum gets the largest E4M3 scale, 448
        r, c = np.unravel_index(np.argmax(np.abs(yg)), yg.shape)
        assert sg[r, c // 16] == 0x7E
        # every block scale is the E4M3 value nearest to amax_b / 6 * S_enc (brute-force search)
        amax_b = np.abs(yg.reshape(-1, w // 16, 16)).max(axis=-1)
        want = _brute_e4m3(codecs.f32(codecs.f32(amax_b / 6.0) * s_enc))
        assert np.array_equal(sg, want)
        # every code is the E2M1 value nearest to y * S_enc / s_b, except within a few ulps of a midpoint
        d_b = codecs.e4m3_decode(sg)
        v = yg.reshape(-1, w // 16, 16) * (s_enc / d_b)[..., None]
        near = np.abs(v)[..., None] - codecs.E2M1_MAGS
        nearest = np.argmin(np.abs(near), axis=-1)
        cg = codes[off[g]:off[g + 1]].reshape(-1, w // 16, 16) & 7
        mids = (codecs.E2M1_MAGS[:-1] + codecs.E2M1_MAGS[1:]) / 2
        close = np.min(np.abs(np.abs(v)[..., None] - mids), axis=-1) <= 4 * 2.0 ** -23 * np.abs(v)
        assert np.all((cg == nearest) | close)
        # dequantization error: half an E2M1 step of the block, relative to the value
        deq = codecs.e2m1_decode(cg) * np.sign(yg.reshape(-1, w // 16, 16)) * d_b[..., None] * q["group_scale"][g]
        step = np.where(np.abs(v) < 2, 0.5, np.where(np.abs(v) < 4, 1.0, 2.0))
        bound = (0.5 * step + np.maximum(np.abs(v) - 6, 0)) * d_b[..., None] / s_enc
        assert np.all(np.abs(deq - yg.reshape(-1, w // 16, 16)) <= bound * (1 + 1e-5) + 1e-30)


def test_nvfp4_zero_and_global_edge_cases():
    s_enc, s_dec = quant.nvfp4_global(0.0)
    assert s_enc == 1.0 and s_dec == 1.0
    s_enc, _ = quant.nvfp4_global(1e-45)          # 2688 / 1e-45 overflows FP32
    assert s_enc == quant.FLT_MAX
    y = np.zeros((16, 32))
    q = quant.quantize_grouped(y, [16], quant.NVFP4)
    assert np.all(q["row_data"] == 0) and np.all(q["row_scales"] == 0) and np.all(q["col_data"] == 0)


def test_nvfp4_colwise_reuses_group_amax_and_pads():
    rng = np.random.default_rng(3)
    splits = [20, 40]
    y = codecs.f32(rng.standard_normal((60, 32)))
    q = quant.quantize_grouped(y, splits, quant.NVFP4)
    nd, ns = quant.qtensor_nbytes(quant.NVFP4, True, splits, 32)
    assert q["col_data"].size == nd and q["col_scales"].size == ns
    mats = dequant_col_grouped(quant.NVFP4, q["col_data"], q["col_scales"], splits, 32, q["group_scale"])
    assert mats[0].shape == (32, 128) and np.all(mats[0][:, 20:] == 0)
    assert mats[1].shape == (32, 128) and np.all(mats[1][:, 40:] == 0)
    rel = np.sqrt(np.mean((mats[1][:, :40] - y[20:].T) ** 2) / np.mean(y[20:] ** 2))
    assert rel < 0.2
