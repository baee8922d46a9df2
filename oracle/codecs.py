"""Element codecs: BF16, FP32 rounding, E4M3 (OCP E4M3FN), E2M1, E8M0.

Test infrastructure only (see the package header).

Definitions written out from the formats themselves:
  * BF16: the upper 16 bits of an IEEE binary32; encoding rounds to nearest, ties to even.
  * E4M3 (OCP "E4M3FN"): sign, 4 exponent bits (bias 7), 3 mantissa bits; no infinities; the only
    NaN encodings are S.1111.111; largest finite magnitude 448; subnormal step 2^-9.
    Encoding rounds to nearest, ties to the even code, saturates magnitudes above 448 to 448 and keeps
    the sign of zero.  The saturating, subnormal-keeping RNE codec is the one whose cast error
    reproduces the E4M3 simulation table of [P3] ("How much it costs, if hit"), which the tests pin.
  * E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit; magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6};
    encoding rounds to nearest, ties to the even code, saturates at 6.
  * E8M0: an 8-bit biased exponent, value 2^(code - 127); code 255 is NaN.

Parity: pinned by exhaustive brute-force nearest-value searches in the CPU tests.
"""

import numpy as np


# ----------------------------------------------------------------------------- FP32 / BF16

def f32(x):
    """Round float64 values to the nearest float32 (ties to even), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16_bits_to_f64(bits):
    """Decode BF16 bit patterns (uint16) exactly to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f32_to_bf16_bits(x):
    """Encode float32 values to BF16 bit patterns, round to nearest, ties to even.

    A BF16 value is an FP32 value whose low 16 mantissa bits are zero, so rounding keeps the upper
    half and adds one unit in its last place when the dropped half exceeds 0x8000, or equals 0x8000
    and the kept half is odd.  NaN maps to the quiet NaN 0x7FC0 with the sign kept.
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    upper = u >> np.uint64(16)
    lower = u & np.uint64(0xFFFF)
    round_up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & np.uint64(1)) == 1))
    out = upper + round_up.astype(np.uint64)
    isnan = np.isnan(np.asarray(x, dtype=np.float32))
    out = np.where(isnan, (upper & np.uint64(0x8000)) | np.uint64(0x7FC0), out)
    return out.astype(np.uint16)


# ----------------------------------------------------------------------------- E4M3

def _e4m3_decode_scalar(code):
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_VALUES = np.array([_e4m3_decode_scalar(c) for c in range(256)], dtype=np.float64)
# codes 0..126 are the non-negative finite magnitudes in increasing order (127 is NaN)
E4M3_MAGS = E4M3_VALUES[:127].copy()
E4M3_MAX = 448.0


def e4m3_decode(codes):
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def _nearest_even(mags, a):
    """Index of the nearest entry of the increasing table ``mags`` to each a >= 0 (ties to even).

    Values beyond the last entry map to the last entry (saturation).
    """
    a = np.asarray(a, dtype=np.float64)
    top = len(mags) - 1
    hi = np.searchsorted(mags, a, side="left")  # mags[hi-1] < a <= mags[hi]
    hi = np.clip(hi, 0, top)
    lo = np.clip(hi - 1, 0, top)
    exact = mags[hi] == a
    mid = (mags[lo] + mags[hi]) / 2.0  # exact in float64 for these small tables
    pick_lo = a < mid
    pick_hi = a > mid
    tie_code = np.where(lo % 2 == 0, lo, hi)
    idx = np.where(pick_lo, lo, np.where(pick_hi, hi, tie_code))
    idx = np.where(exact, hi, idx)
    idx = np.where(a >= mags[top], top, idx)
    return idx.astype(np.int64)


def e4m3_encode(v):
    """Encode float64 values to E4M3 codes (uint8): RNE, saturating to +-448, sign of zero kept."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    idx = _nearest_even(E4M3_MAGS, np.where(np.isnan(a), 0.0, a))
    sign = np.signbit(v).astype(np.int64) << 7
    code = idx | sign
    code = np.where(np.isnan(v), 0x7F | sign, code)
    return code.astype(np.uint8)


# ----------------------------------------------------------------------------- E2M1

E2M1_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_VALUES = np.concatenate([E2M1_MAGS, -E2M1_MAGS])  # code 8..15 = negative (8 is -0)
E2M1_MAX = 6.0


def e2m1_decode(codes):
    return E2M1_VALUES[np.asarray(codes, dtype=np.uint8) & 0xF]


def e2m1_encode(v):
    """Encode float64 values to E2M1 codes (uint8 in 0..15): RNE, saturating at +-6."""
    v = np.asarray(v, dtype=np.float64)
    idx = _nearest_even(E2M1_MAGS, np.abs(v))
    return (idx | (np.signbit(v).astype(np.int64) << 3)).astype(np.uint8)


def pack_e2m1(codes):
    """Pack E2M1 codes along the last axis, two per byte: element 2i low nibble, 2i+1 high nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    assert c.shape[-1] % 2 == 0
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_e2m1(packed):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


# ----------------------------------------------------------------------------- E8M0

def e8m0_decode(codes):
    c = np.asarray(codes, dtype=np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))


def floor_log2(a):
    """floor(log2(a)) for positive finite float64 values, exact (from the binary exponent)."""
    _, e = np.frexp(np.asarray(a, dtype=np.float64))  # a = m * 2^e with m in [0.5, 1)
    return e.astype(np.int64) - 1
