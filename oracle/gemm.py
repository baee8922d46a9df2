"""Grouped GEMM on block-quantized operands, in float64.

Test infrastructure only (see the package header).

Sources:
  * [P2] Greptile summary, second bullet, and the sequence diagram: GroupedLinear consumes the
    pre-quantized grouped tensor; per expert group g it computes out_g = x_g W_g^T (FC2 forward), and
    the backward produces the input gradient and the weight gradient of each group.
  * [P1] Description, second paragraph: options that change what the weight gradient consumes (bias,
    one grouped weight tensor, delayed weight-gradient computation).

Every mode is written as C_g = A_g . B_g^T with both operands stored K-contiguous:
  fprop : A = activation rowwise [m_g x K],      B = W_g rowwise [N x K]        -> C [m_g x N]
  dgrad : A = dY rowwise [m_g x N],              B = W_g columnwise [K x N]     -> C [m_g x K]
  wgrad : A = dY columnwise [N_y x mp_g],        B = X columnwise [N_x x mp_g]  -> dW_g [N_y x N_x]
Operands are dequantized exactly to float64 (MXFP8: e4m3 * 2^(c-127); NVFP4: e2m1 * s_b * S_dec),
the product is taken in float64, the per-group bias is added, and an empty group's wgrad is zero.

Parity: the all-unit-scale, small-integer-code case reduces exactly to an int64 matmul (pinned in
the CPU tests); the general case is the definition above.
"""

import numpy as np

from .codecs import e2m1_decode, e4m3_decode, e8m0_decode, unpack_e2m1
from .quant import MXFP8, NVFP4, col_offsets, group_offsets, mx_scales_from_kstep


def dequant_rows(fmt, data, scales, rows, width, group_scale=None):
    """Dequantize a [rows x width] K-contiguous block-quantized matrix to float64.

    MXFP8 scales are in the K-step grouped layout of that matrix; ``group_scale`` (NVFP4 only) is a
    scalar S_dec applied to the whole matrix.
    """
    if rows == 0:
        return np.zeros((0, width))
    if fmt == MXFP8:
        q = e4m3_decode(np.asarray(data, np.uint8).reshape(rows, width))
        s = e8m0_decode(mx_scales_from_kstep(scales, rows, width))
        return q * np.repeat(s, 32, axis=1)
    codes = unpack_e2m1(np.asarray(data, np.uint8).reshape(rows, width // 2))
    q = e2m1_decode(codes)
    s = e4m3_decode(np.asarray(scales, np.uint8).reshape(rows, width // 16))
    return q * np.repeat(s, 16, axis=1) * float(group_scale)


def dequant_row_grouped(fmt, data, scales, split_sizes, width, group_scale=None):
    """Dequantize a rowwise grouped qtensor [M x width]; NVFP4 applies each group's S_dec.

    MXFP8 scales are K-step grouped over the whole [M x width] matrix."""
    off = group_offsets(split_sizes)
    m = int(off[-1])
    if fmt == MXFP8:
        return dequant_rows(fmt, data, scales, m, width)
    out = np.zeros((m, width))
    bpr_d, bpr_s = width // 2, width // 16
    for g in range(len(split_sizes)):
        r0, r1 = off[g], off[g + 1]
        out[r0:r1] = dequant_rows(fmt, data[r0 * bpr_d:r1 * bpr_d], scales[r0 * bpr_s:r1 * bpr_s],
                                  r1 - r0, width, group_scale[g])
    return out


def dequant_col_grouped(fmt, data, scales, split_sizes, width, group_scale=None):
    """Dequantize a columnwise grouped qtensor into a list of [width x mp_g] matrices."""
    coff = col_offsets(split_sizes)
    mats = []
    db = 1 if fmt == MXFP8 else 2
    sb = 32 if fmt == MXFP8 else 16
    for g in range(len(split_sizes)):
        mp = int(coff[g + 1] - coff[g])
        d0 = int(width * coff[g] // db)
        s0 = int(width * coff[g] // sb)
        d = data[d0:d0 + width * mp // db]
        s = scales[s0:s0 + width * mp // sb]
        gs = None if group_scale is None else group_scale[g]
        mats.append(dequant_rows(fmt, d, s, width, mp, gs))
    return mats


def dgrad_weight(col_mats, k):
    """The columnwise copy of a weight, per group [n x roundup(k, 128)] with zero padding, as the
    [n x k] DGRAD operand (the padding columns meet no input column)."""
    return [np.asarray(w)[:, :k] for w in col_mats]


def gemm_grouped_m(a, b_per_group, split_sizes, bias=None):
    """fprop / dgrad: C[off_g:off_g+m_g] = A[off_g:off_g+m_g] . B_g^T (+ bias_g). float64."""
    off = group_offsets(split_sizes)
    n = b_per_group[0].shape[0]
    c = np.zeros((int(off[-1]), n))
    for g in range(len(split_sizes)):
        r0, r1 = off[g], off[g + 1]
        if r1 > r0:
            c[r0:r1] = a[r0:r1] @ b_per_group[g].T
            if bias is not None:
                c[r0:r1] += np.asarray(bias[g], dtype=np.float64)[None, :]
    return c


def gemm_grouped_k(a_per_group, b_per_group):
    """wgrad: dW_g = A_g . B_g^T with K = the group's padded token count; empty groups give zeros."""
    out = []
    for a, b in zip(a_per_group, b_per_group):
        if a.shape[1] == 0:
            out.append(np.zeros((a.shape[0], b.shape[0])))
        else:
            out.append(a @ b.T)
    return np.stack(out)


def rel_rms_error(got, ref):
    """||got - ref||_2 / ||ref||_2 (the relative-to-RMS criterion)."""
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    den = np.sqrt(np.sum(ref * ref))
    num = np.sqrt(np.sum((got - ref) ** 2))
    return num / den if den > 0 else num
