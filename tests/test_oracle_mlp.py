"""The oracle's expert-MLP step against what the recompute page measured.

Page "[PyTorch] Enable fused activation recompute for ScaledTanhSReLU", Description: the fused forward
activates FC1's FP32 accumulator, while the recompute regenerates FC2's input from the saved BF16 FC1
output; forward, dgrad, dprobs and FC1 wgrad stay bitwise equal and FC2's weight gradient deviates by
the RMS percentages of its table (hidden 256, 4 groups, GB300), stored in
tests/golden/recompute_deviation_gb300.json.

The oracle's step with act_input="fp32" is that reading; its FC2-wgrad deviation between the twins,
at hidden 256 and 4 groups, must land on the table's MXFP8 RMS values (within 25%: the pages give
neither token counts nor value distributions, so the N(0, 0.02) weights, N(0, 1) inputs and 256
tokens per group used here are this suite's choice).  The NVFP4 rows were measured with the
Hadamard-transformed recipe the page names NVFP4_RHT; the oracle runs NVFP4 with and without its
reading of that transform (oracle.quant), and both stay under the printed values, which serve as upper
bounds only.  The table's max-abs column is an extreme statistic that grows with the tensor
size the page does not give; it is printed, not asserted.
"""

import json
import os

import numpy as np
import pytest

import workloads
from oracle import mlp as M
from tests.helpers import bf16_f64, recompute_bound_pct

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _step_pair(kind, fmt, act_input, h=256, f=256, splits=(256, 256, 256, 256), seed=0, rht=None):
    rng = np.random.default_rng(seed)
    e, m = len(splits), int(sum(splits))
    f_in = 2 * f if kind in ("swiglu", "clamped_swiglu", "glu") else f
    x1 = workloads.normal_bf16(rng, (m, h))
    w1 = workloads.normal_bf16(rng, (e, f_in, h), 0.02)
    w2 = workloads.normal_bf16(rng, (e, h, f), 0.02)
    b1 = workloads.normal_bf16(rng, (e, f_in), 0.02)
    b2 = workloads.normal_bf16(rng, (e, h), 0.02)
    p = workloads.uniform_f32(rng, m)
    dy2 = workloads.normal_bf16(rng, (m, h))
    args = (kind, fmt, list(splits), bf16_f64(x1), bf16_f64(w1), bf16_f64(b1), bf16_f64(w2),
            bf16_f64(b2), p.astype(np.float64), bf16_f64(dy2))
    ap = {"s": 2.0} if kind == "tanh_srelu" else None
    off = M.mlp_step(*args, act_params=ap, act_input=act_input, recompute=False, rht=rht)
    on = M.mlp_step(*args, act_params=ap, act_input=act_input, recompute=True, rht=rht)
    return off, on


def _bound(kind, fmt):
    with open(os.path.join(GOLDEN, "recompute_deviation_gb300.json")) as fh:
        rows = json.load(fh)["rows"]
    return [r for r in rows if r["recipe"] == fmt and r["act"] == kind][0]


@pytest.mark.parametrize("kind,fmt,rht", [("srelu", "mxfp8", None), ("tanh_srelu", "mxfp8", None),
                                          ("srelu", "nvfp4", None), ("tanh_srelu", "nvfp4", None),
                                          ("srelu", "nvfp4", 0x6B35), ("tanh_srelu", "nvfp4", 0x6B35)])
def test_recompute_deviation_matches_pages_table(kind, fmt, rht):
    """With the Hadamard transform (the page's NVFP4_RHT recipe) the NVFP4 deviation rises (2.7 -> 3.9 %
    for SReLU, 2.5 -> 3.4 % for TanhSReLU here) toward the page's 8.8 % / 4.1 %, still below them."""
    off, on = _step_pair(kind, fmt, "fp32", rht=rht)
    for k in ("y2", "dx1", "dp", "dw1", "db1", "db2"):
        assert np.array_equal(on[k], off[k]), k
    diff = on["dw2"] - off["dw2"]
    rms = np.sqrt(np.mean(off["dw2"] ** 2))
    dev_pct = 100 * np.sqrt(np.mean(diff ** 2)) / rms
    print(kind, fmt, rht, "rms %.2f%%, max-abs %.1f%%, mean/rms %+.4f" % (
        dev_pct, 100 * np.max(np.abs(diff)) / rms, np.mean(diff) / rms))
    b = _bound(kind, fmt)
    assert abs(np.mean(diff)) / rms <= 0.01          # the table's mean column: 0.00
    if fmt == "mxfp8":
        assert 0.8 * b["rms_pct"] <= dev_pct <= 1.25 * b["rms_pct"], (dev_pct, b["rms_pct"])
    else:
        assert 0 < dev_pct <= b["rms_pct"], (dev_pct, b["rms_pct"])


@pytest.mark.parametrize("fmt", ["mxfp8", "nvfp4"])
@pytest.mark.parametrize("kind", ["gelu", "sigmoid", "glu", "swiglu"])
def test_recompute_deviation_other_activations(kind, fmt):
    """The same fused recompute for activations the page's review discussion names for the scheme
    (GeLU, sigmoid, the GLU family): the twins differ in FC2's weight gradient only, by a non-zero RMS
    within the recipe's bound (the page's largest value for that recipe), mean / RMS <= 0.01."""
    off, on = _step_pair(kind, fmt, "fp32")
    for k in ("y2", "dx1", "dp", "dw1", "db1", "db2"):
        assert np.array_equal(on[k], off[k]), k
    diff = on["dw2"] - off["dw2"]
    rms = np.sqrt(np.mean(off["dw2"] ** 2))
    dev_pct = 100 * np.sqrt(np.mean(diff ** 2)) / rms
    print(kind, fmt, "rms %.2f%%" % dev_pct)
    assert 0 < dev_pct <= recompute_bound_pct(fmt, kind), dev_pct
    assert abs(np.mean(diff)) / rms <= 0.01


def test_bf16_act_input_gives_equal_twins():
    """With the forward reading the BF16 FC1 output as the recompute does, nothing differs."""
    off, on = _step_pair("srelu", "mxfp8", "bf16", splits=(128, 64))
    for k in ("y2", "dx1", "dp", "dw1", "dw2", "db1", "db2"):
        assert np.array_equal(on[k], off[k]), k


def test_fp32_act_input_changes_only_the_forward_rounding():
    """The FP32-input forward differs from the BF16-input one by the BF16 rounding of FC1's output
    only: at most 2^-8 relative per element before the activation, so at most (1 + 2^-8)^2 - 1 for
    x^2 (the ~0.8% the page states), plus the FP32 rounding of the result; y2 then agrees to within
    a small fraction of its quantization noise."""
    a, _ = _step_pair("srelu", "mxfp8", "fp32", splits=(128, 64))
    b, _ = _step_pair("srelu", "mxfp8", "bf16", splits=(128, 64))
    assert not np.array_equal(a["a32"], b["a32"])
    rel = np.abs(a["a32"] - b["a32"]) / np.maximum(np.abs(b["a32"]), 1e-300)
    assert np.max(rel[b["a32"] != 0]) <= (1 + 2.0 ** -8) ** 2 - 1 + 2.0 ** -22
    y_rms = np.sqrt(np.mean(b["y2"] ** 2))
    assert np.sqrt(np.mean((a["y2"] - b["y2"]) ** 2)) / y_rms < 0.02
