"""Shared helpers for the parity tests: moving seeded inputs to the GPU and comparing the library's
quantized outputs with the oracle's under the agreement criteria.

Criteria (applied in the tests):
  * SReLU / identity: codes and scales bit-exact.
  * TanhSReLU / SwiGLU / clamped SwiGLU: at most 0.1% of the quantized elements may differ, and a
    differing element may move by at most one step of the element grid (one code step; where the
    block scale itself moved, one step of the coarser of the two grids).
  * GEMM outputs: ||C - C_ref||_2 / ||C_ref||_2 <= 1e-3 over the whole tensor and per group.
"""

import json
import os

import numpy as np

from oracle import codecs
from oracle.quant import mx_scales_from_kstep


def to_dev_bf16(bits):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_host(t):
    import torch
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def u8(t):
    return t.detach().cpu().numpy().astype(np.uint8)


def f32(t):
    return t.detach().cpu().numpy().astype(np.float64)


def bf16_f64(bits):
    return codecs.bf16_bits_to_f64(bits)


# ---------------------------------------------------------------------------- dequantization views

def mx_elementwise(data, scales, rows, width):
    """Per-element (code, block scale value, dequantized value) of a [rows x width] MXFP8 matrix
    whose scales are in the K-step grouped layout."""
    q = np.asarray(data, np.uint8).reshape(rows, width)
    s = codecs.e8m0_decode(mx_scales_from_kstep(scales, rows, width))
    s = np.repeat(s, 32, axis=1)
    return q, s, codecs.e4m3_decode(q) * s


def nv_elementwise(data, scales, rows, width, s_dec):
    codes = codecs.unpack_e2m1(np.asarray(data, np.uint8).reshape(rows, width // 2))
    d = codecs.e4m3_decode(np.asarray(scales, np.uint8).reshape(rows, width // 16))
    d = np.repeat(d, 16, axis=1) * s_dec
    return codes, d, codecs.e2m1_decode(codes) * d


def _grid_step(fmt, v, scale):
    """Spacing of the element grid at |v| (dequantized units) for block scale ``scale``."""
    a = np.abs(v) / np.where(scale > 0, scale, 1.0)
    if fmt == "mxfp8":
        e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
        step = 2.0 ** (e - 3)
    else:
        step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    return step * scale


def compare_quantized(fmt, got, ref, max_frac=1e-3, extra=None):
    """got/ref: (codes, scale_per_element, dequant) triples.  Returns (n_diff, n_total).

    Raises AssertionError when more than ``max_frac`` of the elements differ or a differing element
    is further than one grid step (of the coarser grid) from the reference.  ``extra`` (same shape,
    optional): a further per-element allowance, for inputs that themselves differ by a bounded amount
    (a quantized GEMM output compared with the oracle's product).
    """
    gc, gs, gv = got
    rc, rs, rv = ref
    diff = (gc != rc) | (gs != rs)
    n = diff.size
    nd = int(diff.sum())
    assert nd <= max_frac * n, "%d of %d quantized elements differ (> %.3g%%)" % (nd, n, 100 * max_frac)
    if nd:
        scale = np.maximum(gs, rs)[diff]
        step = np.maximum(_grid_step(fmt, gv[diff], scale), _grid_step(fmt, rv[diff], scale))
        err = np.abs(gv[diff] - rv[diff])
        if extra is not None:
            step = step + np.broadcast_to(extra, diff.shape)[diff]
        assert np.all(err <= step * (1 + 1e-9)), "a differing element moved more than one step"
    return nd, n


def rel_rms(got, ref):
    ref = np.asarray(ref, np.float64)
    den = np.sqrt(np.sum(ref * ref))
    return np.sqrt(np.sum((np.asarray(got, np.float64) - ref) ** 2)) / (den if den > 0 else 1.0)


def recompute_bound_pct(fmt, kind):
    """Bound on the FC2-wgrad RMS deviation between recompute twins, in % of the tensor's RMS, from
    the deviation table of page "[PyTorch] Enable fused activation recompute for ScaledTanhSReLU"
    (Description; tests/golden/recompute_deviation_gb300.json): the table's value for the recipe and
    activation, or, for an activation it does not list, its largest value for the recipe; times 1.25
    for MXFP8 (whose values the oracle reproduces at the page's size) and as printed for NVFP4 (an
    upper bound only)."""
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                           "recompute_deviation_gb300.json")) as fh:
        rows = [r for r in json.load(fh)["rows"] if r["recipe"] == fmt]
    listed = [r["rms_pct"] for r in rows if r["act"] == kind]
    pct = listed[0] if listed else max(r["rms_pct"] for r in rows)
    return pct * (1.25 if fmt == "mxfp8" else 1.0)
