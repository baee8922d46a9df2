"""Pins of the oracle's random Hadamard transform for NVFP4 columnwise copies (the recipe the recompute
page names NVFP4_RHT; the definition is the published one: blocks of 16 along the weight-gradient
GEMM's reduction axis, v -> H16 diag(s) v / 4).

What fixes it independently of the oracle's own formula: the Sylvester recursion H_2n = [[H, H],
[H, -H]] from H_1 = [1]; orthogonality (the transform preserves inner products, so a GEMM of two
transformed operands equals the GEMM of the originals); closed forms on one-hot and constant blocks;
and the NVFP4 error bound carried back through the inverse transform.
"""

import numpy as np
import pytest

from oracle import gemm as G
from oracle import quant as Q

MASK = 0x6B35


def _sylvester(n):
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def test_hadamard_is_sylvester_and_orthogonal():
    h = Q.hadamard16()
    assert np.array_equal(h, _sylvester(16))
    assert np.array_equal(h @ h.T, 16 * np.eye(16))


def test_closed_forms():
    s = Q.rht_signs(MASK)
    assert s[0] == -1 and s[1] == 1 and s[2] == -1 and s[15] == 1  # 0x6B35 = 0b0110_1011_0011_0101
    ones = np.ones(16)
    assert np.array_equal(Q.rht16(ones, 0), np.r_[4.0, np.zeros(15)])       # constant block -> DC only
    for n in (0, 5, 15):
        e = np.zeros(16)
        e[n] = 1.0
        assert np.array_equal(Q.rht16(e, MASK), s[n] * _sylvester(16)[:, n] / 4)   # one column of H


def test_inner_products_norms_and_inverse():
    rng = np.random.default_rng(0)
    a, b = rng.standard_normal((3, 64)), rng.standard_normal((5, 64))
    ta, tb = Q.rht16(a, MASK), Q.rht16(b, MASK)
    assert np.allclose(ta @ tb.T, a @ b.T, rtol=1e-13, atol=1e-13)
    assert np.allclose(np.linalg.norm(ta, axis=1), np.linalg.norm(a, axis=1), rtol=1e-14)
    # inverse: D H / 4 per block
    back = (ta.reshape(3, 4, 16) @ _sylvester(16) / 4 * Q.rht_signs(MASK)).reshape(3, 64)
    assert np.allclose(back, a, rtol=0, atol=1e-14)


def test_columnwise_copy_layout_scales_and_error_bound():
    """A partial last block (37 tokens: 2 full blocks + 5 tokens) carries transformed values in its
    padding positions; the transformed copy's group scale comes from its own amax; dequantized and
    transformed back, every block is within the NVFP4 half-step bound (carried through the orthogonal
    inverse as a 2-norm)."""
    rng = np.random.default_rng(1)
    splits, w = [37, 0, 64], 32
    y = Q.f32(rng.standard_normal((sum(splits), w)) * 2.0)
    y[3, 5] = 40.0                                    # an outlier the transform spreads over its block
    q = Q.quantize_grouped(y, splits, "nvfp4", rowwise=False, colwise=True, rht=MASK)
    mats = G.dequant_col_grouped("nvfp4", q["col_data"], q["col_scales"], splits, w, q["col_group_scale"])
    off = Q.group_offsets(splits)
    for g, m_g in enumerate(splits):
        if m_g == 0:
            continue
        mp = Q.roundup(m_g, 128)
        yt = np.zeros((w, mp))
        yt[:, :m_g] = y[off[g]:off[g + 1]].T
        t = Q.f32(Q.rht16(yt, MASK))
        assert q["col_group_amax"][g] == Q.f32(np.max(np.abs(t)))
        if m_g % 16:
            assert np.any(t[:, m_g:Q.roundup(m_g, 16)] != 0)     # padding of the partial block is used
        deq = mats[g]
        # per-element bound in the transformed domain: half an E2M1 step at the element's magnitude
        # (steps 0.5 up to 2, 1 up to 4, 2 above) times the block's decode scale
        err = np.abs(deq - t)
        blocks = t.reshape(w, mp // 16, 16)
        eblocks = err.reshape(w, mp // 16, 16)
        amax_b = np.max(np.abs(blocks), axis=-1, keepdims=True)
        bound = amax_b / 6 * 1.0 * 1.0625          # half of the largest step (2) in units of amax_b/6, + scale rounding
        assert np.all(eblocks <= bound + 1e-12)
        # back in the original domain the per-block error 2-norm is unchanged
        inv = lambda m: (m.reshape(w, mp // 16, 16) @ _sylvester(16) / 4 * Q.rht_signs(MASK)).reshape(w, mp)
        e_orig = (inv(deq) - inv(t)).reshape(w, mp // 16, 16)
        assert np.allclose(np.linalg.norm(e_orig, axis=-1), np.linalg.norm(eblocks, axis=-1), rtol=1e-9, atol=1e-12)


def test_wgrad_of_transformed_operands_matches_plain_product():
    """dW = dY^T X over one expert's tokens from the two RHT columnwise copies: the transform cancels,
    so the dequantized product is within NVFP4 quantization error of the FP64 product, like the plain
    recipe's."""
    rng = np.random.default_rng(2)
    splits, h, f = [200], 64, 96
    dy = Q.f32(rng.standard_normal((200, h)))
    x = Q.f32(rng.standard_normal((200, f)))
    exact = dy.T @ x
    errs = {}
    for rht in (None, MASK):
        qd = Q.quantize_grouped(dy, splits, "nvfp4", rowwise=False, colwise=True, rht=rht)
        qx = Q.quantize_grouped(x, splits, "nvfp4", rowwise=False, colwise=True, rht=rht)
        gs = "col_group_scale" if rht else "group_scale"
        a = G.dequant_col_grouped("nvfp4", qd["col_data"], qd["col_scales"], splits, h, qd[gs])[0]
        b = G.dequant_col_grouped("nvfp4", qx["col_data"], qx["col_scales"], splits, f, qx[gs])[0]
        errs[rht] = np.sqrt(np.mean((a @ b.T - exact) ** 2)) / np.sqrt(np.mean(exact ** 2))
    assert errs[MASK] < 0.25 and errs[None] < 0.25
    assert 0.5 < errs[MASK] / errs[None] < 2.0, errs
