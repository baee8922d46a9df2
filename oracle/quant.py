"""Grouped block quantization: MXFP8 (E4M3 + E8M0 per 32) and NVFP4 (E2M1 + E4M3 per 16 + FP32 per tensor).

Test infrastructure only (see the package header).

Sources:
  * [P1] Description, second paragraph: both recipes (MXFP8 and NVFP4) run the fused path; the NVFP4
    regeneration returns BF16 that is then requantized.
  * [P2] Greptile summary, first two bullets: the activation output is quantized into a grouped tensor
    that the grouped GEMM consumes as is.
  * [P3] "A behaviour change worth calling out": quantizers carry a rowwise and a columnwise usage; the
    columnwise copy feeds the weight-gradient GEMM.
  * OCP Microscaling Formats v1.0: MXFP8 E4M3 block of 32 with shared scale
    X = 2^(floor(log2(amax)) - emax_elem), emax_elem = 8 for E4M3 (448 = 1.75 * 2^8).
  * The NVFP4 recipe: a per-tensor FP32 encode scale S_enc = (448 * 6) / amax_tensor, a per-16-block
    E4M3 decode scale s_b = E4M3(amax_b / 6 * S_enc), elements E2M1(y * S_enc / s_b); the stored
    per-tensor value is S_dec = 1 / S_enc, and y ~= e2m1 * s_b * S_dec.

Readings (listed in the design notes):
  * MXFP8 scale code c = clamp(floor(log2 amax) - 8 + 127, 0, 254); an all-zero block gets c = 0.
  * Quantization always starts from the FP32 value (never from a BF16-rounded copy).
  * The NVFP4 "per-tensor" scale is per group: each expert's slice is the tensor its GEMM consumes.
  * NVFP4 FP32 sequence: S_enc = f32(2688 / A_g) (1 when A_g = 0, FLT_MAX when it overflows);
    sf = f32(f32(amax_b / 6) * S_enc); s_b = E4M3(sf); d_b = decode(s_b); if d_b == 0 all codes are 0,
    else r_b = f32(S_enc / d_b) and code = E2M1(f32(y * r_b)).  S_dec = f32(1 / S_enc).
  * Columnwise layout: per group, the [m_g x W] slice is transposed to [W x m_g], rows padded with
    zeros to roundup(m_g, 128) for both formats (a whole number of 128-token K steps of the weight-
    gradient GEMM), and quantized along the (token) rows, so blocks never straddle groups and a
    partial last block takes its amax over its real rows only.
  * E2M1 packing: element 2i in the low nibble.

Buffer layouts produced here are the library's documented qtensor layouts:
  rowwise MXFP8 : data u8 [M, W],                         scales: K-step grouped over [M, W]
  rowwise NVFP4 : data u8 [M, W/2],                       scales u8 [M, W/16],  group_scale f32 [E]
  colwise MXFP8 : per group g at data offset W*coff[g]:    data [W, mp_g],
                  scales at W*coff[g]/32:                  K-step grouped over [W, mp_g]
  colwise NVFP4 : per group g at data offset W*coff[g]/2: data [W, mp_g/2],     scales [W, mp_g/16]
  with mp_g = roundup(m_g, 128) and coff[g] = sum_{h<g} mp_h.
  "K-step grouped" (MXFP8 scales of an [R x K] matrix): the four 32-block scales of each 128-wide K
  step are stored together per row, steps outermost -- the byte of (row r, block kb) is at
  ((kb // 4) * R + r) * 4 + kb % 4, 4 * R * ceil(K / 128) bytes in all, unused bytes of a partial
  last step zero.

Random Hadamard transform (the recipe [P1]'s deviation table names "NVFP4_RHT" without defining
it; the reading follows the published NVFP4 training recipe): before NVFP4 columnwise quantization,
every 16-token block v of a column becomes H16 diag(s) v / 4, H16 the Sylvester Hadamard matrix
(H[k, n] = (-1)^popcount(k & n)) and s a fixed sign vector given as a 16-bit mask (bit i set: s_i = -1).
The map is orthogonal, so applied to both operands of a weight-gradient GEMM along their common
(token) axis it leaves the product unchanged while spreading outliers over the block.  The
transformed copy takes its per-group encode scale from its own amax (over the transformed values,
padding positions of a partial block included: they carry transformed values the product needs).

Parity: MXFP8 pinned (closed-form scale codes, exhaustive codec tests, M6 statistics).  The NVFP4
FP32 sequence is a reading; it is pinned only by invariants (the block holding the group maximum gets
s_b = 448, codes within +-6, dequantization error bound), so its exact bits are "parity unpinned".
"""

import numpy as np

from .codecs import (
    E4M3_MAX,
    e2m1_encode,
    e4m3_decode,
    e4m3_encode,
    f32,
    floor_log2,
    pack_e2m1,
)

MXFP8 = "mxfp8"
NVFP4 = "nvfp4"
BLOCK = {MXFP8: 32, NVFP4: 16}
COL_ALIGN = 128
FLT_MAX = float(np.finfo(np.float32).max)


def roundup(n, a):
    return (n + a - 1) // a * a


def group_offsets(split_sizes):
    """Row offsets off[g] = sum_{h<g} m_h (E + 1 entries). [P2] sequence diagram: split_sizes."""
    return np.concatenate([[0], np.cumsum(np.asarray(split_sizes, dtype=np.int64))]).astype(np.int64)


def col_offsets(split_sizes):
    """Padded token offsets of the columnwise layout: coff[g] = sum_{h<g} roundup(m_h, 128)."""
    padded = [roundup(int(m), COL_ALIGN) for m in split_sizes]
    return np.concatenate([[0], np.cumsum(padded)]).astype(np.int64)


# ----------------------------------------------------------------------------- MXFP8

def mxfp8_scale_code(amax):
    """E8M0 code of the shared scale for blocks with maximum magnitude ``amax`` (float64 >= 0)."""
    amax = np.asarray(amax, dtype=np.float64)
    safe = np.where(amax > 0, amax, 1.0)
    c = floor_log2(safe) - 8 + 127
    c = np.clip(c, 0, 254)
    return np.where(amax > 0, c, 0).astype(np.uint8)


def mxfp8_quantize_rows(y32):
    """Quantize float32 values (given as float64) along the last axis in blocks of 32."""
    y = np.asarray(y32, dtype=np.float64)
    rows, w = y.shape
    assert w % 32 == 0
    blocks = y.reshape(rows, w // 32, 32)
    amax = np.max(np.abs(blocks), axis=-1)
    code = mxfp8_scale_code(amax)
    x_scale = np.ldexp(1.0, code.astype(np.int64) - 127)  # 2^(c - 127)
    q = e4m3_encode(blocks / x_scale[..., None])
    return q.reshape(rows, w), code


def mx_scales_to_kstep(scales_rk):
    """Row-major [R, K/32] E8M0 codes -> the K-step grouped byte layout (flat, zero padded)."""
    s = np.asarray(scales_rk, dtype=np.uint8)
    r, nkb = s.shape
    nsteps = (nkb + 3) // 4
    out = np.zeros((nsteps, r, 4), dtype=np.uint8)
    for kb in range(nkb):
        out[kb // 4, :, kb % 4] = s[:, kb]
    return out.reshape(-1)


def mx_scales_from_kstep(flat, r, k):
    """Inverse of mx_scales_to_kstep for an [R, K] matrix: returns [R, K/32] codes."""
    nkb = k // 32
    nsteps = (nkb + 3) // 4
    a = np.asarray(flat, dtype=np.uint8).reshape(nsteps, r, 4)
    out = np.zeros((r, nkb), dtype=np.uint8)
    for kb in range(nkb):
        out[:, kb] = a[kb // 4, :, kb % 4]
    return out


# ----------------------------------------------------------------------------- NVFP4

def nvfp4_global(amax_group):
    """(S_enc, S_dec) for a group maximum magnitude, FP32 sequence as stated in the header."""
    a = float(amax_group)
    if a == 0.0:
        s_enc = 1.0
    else:
        s_enc = float(f32(2688.0 / a))
        if np.isinf(s_enc):
            s_enc = FLT_MAX
    s_dec = float(f32(1.0 / s_enc))
    return s_enc, s_dec


def nvfp4_quantize_rows(y32, s_enc):
    """Quantize along the last axis in blocks of 16 with encode scale ``s_enc``.

    Returns (packed codes [rows, w/2], E4M3 block scales [rows, w/16]).
    """
    y = np.asarray(y32, dtype=np.float64)
    rows, w = y.shape
    assert w % 16 == 0
    blocks = y.reshape(rows, w // 16, 16)
    amax_b = np.max(np.abs(blocks), axis=-1)
    sf = f32(f32(amax_b / 6.0) * s_enc)
    s_code = e4m3_encode(sf)
    d_b = e4m3_decode(s_code)
    nz = d_b != 0
    r_b = f32(s_enc / np.where(nz, d_b, 1.0))
    v = f32(blocks * r_b[..., None])
    codes = e2m1_encode(v)
    codes = np.where(nz[..., None], codes, 0).astype(np.uint8)
    return pack_e2m1(codes.reshape(rows, w)), s_code


# ----------------------------------------------------------------------------- Hadamard

def hadamard16():
    """Sylvester Hadamard matrix of order 16 from its closed form H[k, n] = (-1)^popcount(k & n)."""
    k = np.arange(16)
    parity = np.array([[bin(a & b).count("1") & 1 for b in k] for a in k])
    return np.where(parity == 1, -1.0, 1.0)


def rht_signs(mask):
    """The sign vector s (length 16) of a 16-bit mask: bit i set means s_i = -1."""
    return np.array([-1.0 if (int(mask) >> i) & 1 else 1.0 for i in range(16)])


def rht16(x, mask):
    """H16 diag(s) v / 4 on every block of 16 consecutive values along the last axis (float64)."""
    x = np.asarray(x, dtype=np.float64)
    assert x.shape[-1] % 16 == 0
    blocks = x.reshape(x.shape[:-1] + (x.shape[-1] // 16, 16)) * rht_signs(mask)
    return (blocks @ hadamard16().T / 4.0).reshape(x.shape)


# ----------------------------------------------------------------------------- grouped

def quantize_grouped(y32, split_sizes, fmt, rowwise=True, colwise=True, group_amax=None, rht=None):
    """Grouped quantization of a [M, W] float32 tensor (float64 array of float32 values).

    Returns a dict with (as requested) 'row_data', 'row_scales', 'col_data', 'col_scales' (flat uint8
    buffers in the documented layouts), and for NVFP4 'group_amax' and 'group_scale' (float32 [E]).
    NVFP4 with `group_amax` given takes the per-tensor scales from it instead of from y: the recompute
    requantizes with the amax its forward saved ([P1] Description: recompute regenerates FC2's input
    under the forward's quantization state).  NVFP4 with `rht` (a 16-bit sign mask) transforms the
    columnwise copy (see the module notes) and returns its own 'col_group_amax' / 'col_group_scale'
    (`group_amax` then applies to the rowwise copy only).
    """
    y = np.asarray(y32, dtype=np.float64)
    m_total, w = y.shape
    off = group_offsets(split_sizes)
    coff = col_offsets(split_sizes)
    assert off[-1] == m_total
    e = len(split_sizes)
    out = {}
    s_enc = np.ones(e)
    if fmt == NVFP4:
        amax = np.zeros(e)
        for g in range(e):
            sl = y[off[g]:off[g + 1]]
            amax[g] = np.max(np.abs(sl)) if sl.size else 0.0
        if group_amax is not None:
            amax = np.asarray(group_amax, dtype=np.float64)
        pairs = [nvfp4_global(a) for a in amax]
        s_enc = np.array([p[0] for p in pairs])
        out["group_amax"] = f32(amax)
        out["group_scale"] = np.array([p[1] for p in pairs])
    if rowwise:
        if fmt == MXFP8:
            d, s = mxfp8_quantize_rows(y) if m_total else (np.zeros((0, w), np.uint8), np.zeros((0, w // 32), np.uint8))
        else:
            parts_d, parts_s = [], []
            for g in range(e):
                sl = y[off[g]:off[g + 1]]
                if sl.shape[0] == 0:
                    continue
                d_g, s_g = nvfp4_quantize_rows(sl, s_enc[g])
                parts_d.append(d_g)
                parts_s.append(s_g)
            d = np.concatenate(parts_d) if parts_d else np.zeros((0, w // 2), np.uint8)
            s = np.concatenate(parts_s) if parts_s else np.zeros((0, w // 16), np.uint8)
        out["row_data"] = d.reshape(-1)
        out["row_scales"] = mx_scales_to_kstep(s) if fmt == MXFP8 else s.reshape(-1)
    if colwise:
        assert rht is None or fmt == NVFP4, "the Hadamard transform applies to NVFP4 columnwise copies"
        col_t, col_enc = [], s_enc
        for g in range(e):
            m_g = off[g + 1] - off[g]
            mp = coff[g + 1] - coff[g]
            yt = np.zeros((w, mp))
            yt[:, :m_g] = y[off[g]:off[g + 1]].T
            col_t.append(f32(rht16(yt, rht)) if rht is not None and mp else yt)
        if rht is not None:
            camax = np.array([np.max(np.abs(t)) if t.size else 0.0 for t in col_t])
            pairs = [nvfp4_global(a) for a in camax]
            col_enc = np.array([p[0] for p in pairs])
            out["col_group_amax"] = f32(camax)
            out["col_group_scale"] = np.array([p[1] for p in pairs])
        parts_d, parts_s = [], []
        for g in range(e):
            mp = coff[g + 1] - coff[g]
            if mp == 0:
                continue
            yt = col_t[g]
            if fmt == MXFP8:
                d_g, s_g = mxfp8_quantize_rows(yt)
                s_g = mx_scales_to_kstep(s_g)
            else:
                d_g, s_g = nvfp4_quantize_rows(yt, col_enc[g])
            parts_d.append(d_g.reshape(-1))
            parts_s.append(s_g.reshape(-1))
        out["col_data"] = np.concatenate(parts_d) if parts_d else np.zeros(0, np.uint8)
        out["col_scales"] = np.concatenate(parts_s) if parts_s else np.zeros(0, np.uint8)
    return out


def qtensor_nbytes(fmt, colwise, split_sizes, width):
    """(data bytes, scale bytes) of a grouped qtensor in the documented layout."""
    rows = int(col_offsets(split_sizes)[-1]) if colwise else int(np.sum(split_sizes))
    if fmt == MXFP8:
        if colwise:   # per group [width x mp_g], mp_g a multiple of 128
            return rows * width, rows * width // 32
        return rows * width, 4 * rows * ((width + 127) // 128)
    return rows * width // 2, rows * width // 16
