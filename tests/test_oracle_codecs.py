"""Pins of the oracle's element codecs against brute force, closed forms and the pages' E4M3 table."""

import json
import os

import numpy as np
import pytest

from oracle import codecs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _all_finite_bf16_values():
    bits = np.arange(65536, dtype=np.uint32)
    v32 = (bits << 16).view(np.float32)
    return v32[np.isfinite(v32)].astype(np.float64)


def _brute_nearest(values, mags):
    """Nearest magnitude by exhaustive distance search; ties -> even index; sign re-applied.

    Independent of the oracle's search: computes every distance explicitly, in chunks.  Among the
    magnitudes at the minimal distance the even index wins when there is one (the even code of a
    tie), else the single nearest index.  Magnitudes above 2^20 are searched as 2^20: every value at or
    above the largest magnitude has that magnitude as its unique nearest one, and below 2^20 all the
    float64 differences are exact (beyond it, |a - m| rounds to the same double for neighbouring m
    and would fake ties).
    """
    a_all = np.minimum(np.abs(np.asarray(values, np.float64)), 2.0 ** 20)
    assert mags[-1] < 2.0 ** 20
    idx = np.empty(len(a_all), dtype=np.int64)
    even = (np.arange(len(mags)) % 2 == 0)[None, :]
    for c0 in range(0, len(a_all), 8192):
        a = a_all[c0:c0 + 8192, None]
        d = np.abs(a - mags[None, :])
        cand = d == d.min(axis=1, keepdims=True)
        ce = cand & even
        has_even = ce.any(axis=1)
        idx[c0:c0 + 8192] = np.where(has_even, np.argmax(ce, axis=1), np.argmax(cand, axis=1))
    return idx


@pytest.mark.parametrize("log2_scale", [-12, -6, -3, 0, 3, 6, 9])
def test_e4m3_encode_matches_brute_force(log2_scale):
    """Every finite BF16 pattern (65,280 of the 65,536; the other 256 are infinities and NaNs), scaled
    by 2^log2_scale: the encoder equals the nearest-magnitude search, saturation included (beyond 448
    the nearest magnitude is 448), sign of zero kept."""
    v = _all_finite_bf16_values() * 2.0 ** log2_scale
    assert len(v) == 65536 - 256
    mags = codecs.E4M3_MAGS
    idx = _brute_nearest(v, mags)
    want = idx | (np.signbit(v).astype(np.int64) << 7)
    got = codecs.e4m3_encode(v).astype(np.int64)
    assert np.array_equal(got, want)


def test_e4m3_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = codecs.e4m3_decode(codes)
    assert np.array_equal(codecs.e4m3_encode(vals), codes)
    assert codecs.E4M3_MAGS[-1] == 448.0 and codecs.E4M3_MAGS[1] == 2.0 ** -9


def test_e4m3_hand_values():
    cases = [(448.0, 0x7E), (464.0, 0x7E), (1e9, 0x7E), (-1e9, 0xFE), (1.0, 0x38), (2.0 ** -9, 0x01),
             (2.0 ** -10, 0x00), (1.5 * 2.0 ** -10, 0x01), (0.0, 0x00), (-0.0, 0x80), (240.0, 0x77),
             # 17 lies halfway between 16 (code 0x58) and 18 (0x59): ties to the even code
             (17.0, 0x58), (19.0, 0x5A)]
    for v, c in cases:
        assert int(codecs.e4m3_encode(np.array([v]))[0]) == c, v


def test_e2m1_encode_matches_brute_force():
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.uniform(-8, 8, 20000),
                        np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, -0.25, -5.0])])
    idx = _brute_nearest(v, codecs.E2M1_MAGS)
    want = idx | (np.signbit(v).astype(np.int64) << 3)
    assert np.array_equal(codecs.e2m1_encode(v).astype(np.int64), want)


def test_e2m1_ties_and_roundtrip():
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6, 6.5: 7, 100.0: 7}
    for v, c in ties.items():
        assert int(codecs.e2m1_encode(np.array([v]))[0]) == c, v
    codes = np.arange(16, dtype=np.uint8)
    assert np.array_equal(codecs.e2m1_encode(codecs.e2m1_decode(codes)), codes)
    packed = codecs.pack_e2m1(np.array([[1, 2, 3, 15]], dtype=np.uint8))
    assert packed.tolist() == [[0x21, 0xF3]]
    assert np.array_equal(codecs.unpack_e2m1(packed), [[1, 2, 3, 15]])


def test_bf16_rne_matches_nearest_search():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(200000).astype(np.float32)
    # add exact ties: values with low half exactly 0x8000
    u = x.view(np.uint32)
    ties = ((u[:2000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties])
    bits = codecs.f32_to_bf16_bits(x)
    got = codecs.bf16_bits_to_f64(bits)
    # candidates: truncation and the next BF16 value away from zero
    trunc = (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)
    up = ((x.view(np.uint32) & np.uint32(0xFFFF0000)) + np.uint32(0x10000)).view(np.float32).astype(np.float64)
    xd = x.astype(np.float64)
    dt, du = np.abs(xd - trunc), np.abs(xd - up)
    trunc_even = ((x.view(np.uint32) >> 16) & 1) == 0
    want = np.where(dt < du, trunc, np.where(du < dt, up, np.where(trunc_even, trunc, up)))
    assert np.array_equal(got, want)


def test_bf16_square_perturbation_is_two_bf16_half_ulps():
    """The ScaledTanhSReLU page (Description, after the table) says the BF16-saved FC1 output perturbs
    FC2's input by about 0.8%: rounding x to BF16 moves x^2 by at most 2 * 2^-8 relative (0.78%)."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal(1 << 20).astype(np.float32)
    xb = codecs.bf16_bits_to_f64(codecs.f32_to_bf16_bits(x))
    rel = np.abs(xb ** 2 - x.astype(np.float64) ** 2) / (x.astype(np.float64) ** 2)
    assert rel.max() <= 2 * 2.0 ** -8 * (1 + 2.0 ** -8)
    assert rel.max() > 0.99 * 2 * 2.0 ** -8 * (1 - 2.0 ** -7)
    assert abs(100 * rel.max() - 0.8) < 0.03


def _cast_error(x, scale):
    q = codecs.e4m3_decode(codecs.e4m3_encode(x * scale)) / scale
    return np.sqrt(np.mean((q - x) ** 2)) / np.sqrt(np.mean(x ** 2))


def test_e4m3_cast_error_table_reproduced():
    with open(os.path.join(GOLDEN, "e4m3_cast_error.json")) as f:
        table = json.load(f)
    rng = np.random.default_rng(0)
    for row in table["rows"]:
        x = rng.standard_normal(1 << 22) * row["sigma"]
        e1 = 100 * _cast_error(x, 1.0)
        ei = 100 * _cast_error(x, 448.0 / np.max(np.abs(x)))
        assert abs(e1 - row["err_scale1_pct"]) <= row["tol_pct"], (row, e1)
        assert abs(ei - row["err_ideal_pct"]) <= 0.01, (row, ei)


def test_e4m3_subnormal_closed_form():
    """At sigma = 0.005 almost every value falls in the subnormal range (step 2^-9), where the
    rounding error is uniform: RMS error / sigma = 2^-9 / sqrt(12) / 0.005 = 11.28%."""
    closed = 2.0 ** -9 / np.sqrt(12.0) / 0.005
    rng = np.random.default_rng(5)
    x = rng.standard_normal(1 << 21) * 0.005
    assert abs(_cast_error(x, 1.0) - closed) < 0.002


def test_floor_log2_and_e8m0():
    a = np.array([1.0, 1.9999, 2.0, 3.5, 448.0, 2.0 ** -130, 1e-45])
    assert codecs.floor_log2(a).tolist() == [0, 0, 1, 1, 8, -130, -150]
    assert codecs.e8m0_decode(np.array([127, 0, 254])).tolist() == [1.0, 2.0 ** -127, 2.0 ** 127]
    assert np.isnan(codecs.e8m0_decode(np.array([255]))[0])
