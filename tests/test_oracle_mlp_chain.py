"""The oracle's expert-MLP step pinned against an unquantized float64 chain written out here.

Page "Activation + GroupedLinear Fusion for MOE", Sequence Diagram: the forward runs FC1, the scaled
activation and FC2 per expert group; the backward runs FC2's backward (giving the gradient of the
scaled activation output), the activation backward (activation gradient and the gradient of the
per-row scales) and FC1's backward.  Page "[PyTorch] Enable fused activation recompute for
ScaledTanhSReLU", Description: the step carries biases on both GEMMs.

This module writes that step without any quantization, in float64, with its own activation formulas
and its own chain rule (nothing from oracle/ is used for the reference).  Two pins follow:
  1. the reference's gradients equal central finite differences of the scalar loss
     L = sum(dY2 * Y2) on a tiny step, coordinate by coordinate (this fixes the chain rule itself);
  2. every one of the ten outputs of oracle.mlp.mlp_step (y1, y2, dA, dY1, dprobs, dX1, dW1, dW2,
     db1, db2) stays within quantization-level relative RMS of the reference, with hidden != ffn and
     a gated kind whose FC1 output is twice the activation width, so that a transposed operand, a
     swapped weight or a wrong group offset either raises on a shape or lands far outside the bound
     (an uncorrelated result is ~100 % off, the quantization noise a few %).
"""

import numpy as np
import pytest

import workloads
from oracle import mlp as M
from tests.helpers import bf16_f64


# ------------------------------------------------------------------ reference written out here

def _sig(z):
    return 1.0 / (1.0 + np.exp(-z))


def _act_ref(kind, y):
    """a(y) and the pieces of its derivative, for the two kinds used here."""
    if kind == "srelu":
        r = np.where(y > 0, y, 0.0)
        return r * r
    h = y.shape[1] // 2
    g, u = y[:, :h], y[:, h:]
    return g * _sig(g) * u


def _act_vjp(kind, y, da_p):
    """Gradient of sum(a(y) * w) w.r.t. y, for an upstream weight w = da_p (same shape as a)."""
    if kind == "srelu":
        return da_p * 2.0 * np.where(y > 0, y, 0.0)
    h = y.shape[1] // 2
    g, u = y[:, :h], y[:, h:]
    s = _sig(g)
    d_silu = s + g * s * (1.0 - s)          # d/dg of g * sigmoid(g)
    return np.concatenate([da_p * u * d_silu, da_p * g * s], axis=1)


def _bounds(splits):
    off = np.concatenate([[0], np.cumsum(splits)]).astype(int)
    return [(int(off[g]), int(off[g + 1])) for g in range(len(splits))]


def ref_forward(kind, splits, x1, w1, b1, w2, b2, p):
    """y1 = X1 W1_g^T + b1_g ; a = act(y1) * p ; y2 = a W2_g^T + b2_g  (group by group)."""
    m = x1.shape[0]
    y1 = np.zeros((m, w1.shape[1]))
    y2 = np.zeros((m, w2.shape[1]))
    for g, (r0, r1) in enumerate(_bounds(splits)):
        y1[r0:r1] = x1[r0:r1] @ w1[g].T + b1[g]
    a = _act_ref(kind, y1) * p[:, None]
    for g, (r0, r1) in enumerate(_bounds(splits)):
        y2[r0:r1] = a[r0:r1] @ w2[g].T + b2[g]
    return y1, a, y2


def ref_step(kind, splits, x1, w1, b1, w2, b2, p, dy2):
    """Forward and the chain rule of L = sum(dy2 * y2), written out."""
    y1, a, y2 = ref_forward(kind, splits, x1, w1, b1, w2, b2, p)
    e = len(splits)
    da = np.zeros_like(a)                   # dL/d(act * p)
    for g, (r0, r1) in enumerate(_bounds(splits)):
        da[r0:r1] = dy2[r0:r1] @ w2[g]
    act_out = _act_ref(kind, y1)
    dp = np.sum(da * act_out, axis=1)       # dL/dp
    dy1 = _act_vjp(kind, y1, da * p[:, None])
    dx1 = np.zeros_like(x1)
    dw1 = np.zeros_like(w1)
    dw2 = np.zeros_like(w2)
    db1 = np.zeros_like(b1)
    db2 = np.zeros_like(b2)
    for g, (r0, r1) in enumerate(_bounds(splits)):
        dx1[r0:r1] = dy1[r0:r1] @ w1[g]
        dw1[g] = dy1[r0:r1].T @ x1[r0:r1]
        dw2[g] = dy2[r0:r1].T @ a[r0:r1]
        db1[g] = dy1[r0:r1].sum(axis=0)
        db2[g] = dy2[r0:r1].sum(axis=0)
    assert dw1.shape == (e,) + w1.shape[1:] and dw2.shape == (e,) + w2.shape[1:]
    return dict(y1=y1, y2=y2, da=da, dy1=dy1, dp=dp, dx1=dx1, dw1=dw1, dw2=dw2, db1=db1, db2=db2)


# ------------------------------------------------------------------ pin 1: finite differences

@pytest.mark.parametrize("kind", ["srelu", "swiglu"])
def test_reference_chain_rule_matches_finite_differences(kind):
    rng = np.random.default_rng(7)
    splits = [2, 0, 3]
    e, m, h, f = 3, 5, 6, 4
    f_in = 2 * f if kind == "swiglu" else f
    x1 = rng.standard_normal((m, h))
    w1 = rng.standard_normal((e, f_in, h)) * 0.5
    b1 = rng.standard_normal((e, f_in)) * 0.5
    w2 = rng.standard_normal((e, h, f)) * 0.5
    b2 = rng.standard_normal((e, h)) * 0.5
    p = rng.random(m)
    dy2 = rng.standard_normal((m, h))
    params = dict(x1=x1, w1=w1, b1=b1, w2=w2, b2=b2, p=p)
    got = ref_step(kind, splits, x1, w1, b1, w2, b2, p, dy2)
    # SReLU has a kink at 0: keep every FC1 output away from it so differences stay one-sided-free
    y1, _, _ = ref_forward(kind, splits, x1, w1, b1, w2, b2, p)
    assert np.min(np.abs(y1)) > 1e-3

    def loss(**kw):
        args = dict(params)
        args.update(kw)
        _, _, y2 = ref_forward(kind, splits, **args)
        return float(np.sum(dy2 * y2))

    grads = {"x1": got["dx1"], "w1": got["dw1"], "b1": got["db1"], "w2": got["dw2"],
             "b2": got["db2"], "p": got["dp"]}
    eps = 1e-6
    for name, want in grads.items():
        base = params[name]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            hi = base.copy(); hi[idx] += eps
            lo = base.copy(); lo[idx] -= eps
            fd[idx] = (loss(**{name: hi}) - loss(**{name: lo})) / (2 * eps)
        assert np.allclose(fd, want, rtol=1e-6, atol=1e-7), name
    # dL/dY1 and dL/dA by perturbing the intermediate directly
    y1, a, _ = ref_forward(kind, splits, x1, w1, b1, w2, b2, p)

    def loss_from_a(av):
        out = 0.0
        for g, (r0, r1) in enumerate(_bounds(splits)):
            out += float(np.sum(dy2[r0:r1] * (av[r0:r1] @ w2[g].T + b2[g])))
        return out

    fd_a = np.zeros_like(a)
    for idx in np.ndindex(a.shape):
        hi = a.copy(); hi[idx] += eps
        lo = a.copy(); lo[idx] -= eps
        fd_a[idx] = (loss_from_a(hi) - loss_from_a(lo)) / (2 * eps)
    assert np.allclose(fd_a, got["da"], rtol=1e-6, atol=1e-7)
    fd_y1 = np.zeros_like(y1)
    for idx in np.ndindex(y1.shape):
        hi = y1.copy(); hi[idx] += eps
        lo = y1.copy(); lo[idx] -= eps
        fd_y1[idx] = (loss_from_a(_act_ref(kind, hi) * p[:, None])
                      - loss_from_a(_act_ref(kind, lo) * p[:, None])) / (2 * eps)
    assert np.allclose(fd_y1, got["dy1"], rtol=1e-6, atol=1e-7)


# ------------------------------------------------------------------ pin 2: the oracle's composition

# Relative-RMS bounds per output, about 1.5x what each recipe's quantization noise gives at these
# sizes and far below the ~100 % of a wiring mistake.  Measured (srelu / swiglu):
#   MXFP8 y1 .039/.039  y2 .023/.012  dA .043/.043  dY1 .059/.059  dp .068/.067  dX1 .078/.077
#         dW1 .078/.076 dW2 .068/.070 db1 .053/.061
#   NVFP4 y1 .120/.118  y2 .061/.032  dA .138/.134  dY1 .181/.186  dp .217/.207  dX1 .217/.229
#         dW1 .215/.226 dW2 .185/.208 db1 .160/.196
# db2 sums the unquantized dY2 on both sides: equal up to float64 summation order.
BOUNDS = {
    "mxfp8": dict(y1=0.06, y2=0.05, da=0.065, dy1=0.09, dp=0.10, dx1=0.12, dw1=0.12, dw2=0.105,
                  db1=0.095, db2=1e-12),
    "nvfp4": dict(y1=0.18, y2=0.12, da=0.21, dy1=0.28, dp=0.32, dx1=0.34, dw1=0.34, dw2=0.31,
                  db1=0.30, db2=1e-12),
}


def _inputs(kind, seed, splits, h, f):
    rng = np.random.default_rng(seed)
    e, m = len(splits), int(sum(splits))
    f_in = 2 * f if kind == "swiglu" else f
    x1 = bf16_f64(workloads.normal_bf16(rng, (m, h)))
    w1 = bf16_f64(workloads.normal_bf16(rng, (e, f_in, h), 0.05))
    b1 = bf16_f64(workloads.normal_bf16(rng, (e, f_in), 0.25))
    w2 = bf16_f64(workloads.normal_bf16(rng, (e, h, f), 0.05))
    b2 = bf16_f64(workloads.normal_bf16(rng, (e, h), 0.25))
    p = workloads.uniform_f32(rng, m).astype(np.float64)
    dy2 = bf16_f64(workloads.normal_bf16(rng, (m, h)))
    return x1, w1, b1, w2, b2, p, dy2


def _rel(got, ref):
    den = np.sqrt(np.sum(ref * ref))
    return float(np.sqrt(np.sum((got - ref) ** 2)) / den)


@pytest.mark.parametrize("fmt", ["mxfp8", "nvfp4"])
@pytest.mark.parametrize("kind", ["srelu", "swiglu"])
def test_oracle_step_matches_unquantized_chain(kind, fmt):
    splits = [96, 0, 160, 64]
    h, f = 96, 64
    x1, w1, b1, w2, b2, p, dy2 = _inputs(kind, 3, splits, h, f)
    ref = ref_step(kind, splits, x1, w1, b1, w2, b2, p, dy2)
    got = M.mlp_step(kind, fmt, splits, x1, w1, b1, w2, b2, p, dy2)
    errs = {}
    for k in ("y1", "y2", "da", "dy1", "dp", "dx1", "dw1", "dw2", "db1", "db2"):
        assert got[k].shape == ref[k].shape, (k, got[k].shape, ref[k].shape)
        errs[k] = _rel(got[k], ref[k])
    print(kind, fmt, {k: "%.4f" % v for k, v in errs.items()})
    for k, v in errs.items():
        assert v <= BOUNDS[fmt][k], (k, v, BOUNDS[fmt][k])
    # the empty group's weight and bias gradients are exactly zero
    for k in ("dw1", "dw2", "db1", "db2"):
        assert not np.any(got[k][1]), k


def test_planted_wiring_mistakes_fail_the_bound():
    """The bound separates the right composition from plausible wrong ones: each variant of the
    reference below (a transposed square weight, the wrong expert's weight, the bias dropped,
    dprobs taken from the scaled output) misses the oracle's result by far more than the bound."""
    splits = [96, 0, 160, 64]
    h, f = 64, 64                             # square weights: a transpose raises no shape error
    x1, w1, b1, w2, b2, p, dy2 = _inputs("srelu", 5, splits, h, f)
    got = M.mlp_step("srelu", "mxfp8", splits, x1, w1, b1, w2, b2, p, dy2)
    ref = ref_step("srelu", splits, x1, w1, b1, w2, b2, p, dy2)
    assert _rel(got["y2"], ref["y2"]) <= BOUNDS["mxfp8"]["y2"]
    wrong = {
        "w1 transposed": ref_step("srelu", splits, x1, np.swapaxes(w1, 1, 2), b1, w2, b2, p, dy2),
        "w2 of the next expert": ref_step("srelu", splits, x1, w1, b1, np.roll(w2, 1, axis=0), b2, p, dy2),
        "no FC1 bias": ref_step("srelu", splits, x1, w1, 0 * b1, w2, b2, p, dy2),
    }
    for name, r in wrong.items():
        worst = max(_rel(got[k], r[k]) / BOUNDS["mxfp8"][k] for k in ("y1", "y2", "dx1", "dw1", "dw2", "db1"))
        assert worst > 3, name
    # dprobs from act * p instead of act
    dp_wrong = np.sum(ref["da"] * _act_ref("srelu", ref["y1"]) * p[:, None], axis=1)
    assert _rel(got["dp"], dp_wrong) > 3 * BOUNDS["mxfp8"]["dp"]
