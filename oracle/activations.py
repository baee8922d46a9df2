"""Per-row scaled activations, forward and backward, in float64.

Test infrastructure only (see the package header).

Sources:
  * [P2] Greptile summary, first and second bullets, and the "Important Files Changed" row for
    csrc/extensions/activation.cpp: scaled SwiGLU, clamped SwiGLU and SReLU, each multiplied by a
    per-row scale (the MoE routing probability of the row) before grouped quantization; the backward
    returns the activation gradient and the gradient of the per-row scales ("grad_scales").
  * [P2] Sequence diagram, backward half: the backward kernel receives dL/d(act_out * scales).
  * [P1] title and Description: ScaledTanhSReLU is the clamped form of ScaledSReLU; the reviewer's
    suggested comment states that it bounds the activation at s**2.

Readings where the pages print no formula (each listed in the design notes):
  * SReLU:            a(x) = relu(x)^2
  * TanhSReLU(s):     a(x) = (s * tanh(relu(x) / s))^2, bounded by s^2 and -> relu(x)^2 as s -> inf.
  * SwiGLU:           the FC1 output row is [gate | up] (first half gate), a = silu(gate) * up.
  * ClampedSwiGLU(L, alpha, beta):
                      g' = min(gate, L), u' = clamp(up, -L, L), a = g' * sigmoid(alpha g') * (u' + beta);
                      default alpha = 1, beta = 0.  Gradients pass where gate <= L and -L <= up <= L
                      (inclusive), and are zero elsewhere.
  * relu'(0) = 0.
  * GeLU / sigmoid / GLU ([P1] review discussion: nothing in the fused recompute is specific to
    SReLU, and GeLU, sigmoid and the GLU family would use the same scheme; no formula is printed):
                      GeLU:    a(x) = x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)), the exact form
                               (the reading that needs no approximation choice);
                      sigmoid: a(x) = 1 / (1 + exp(-x));
                      GLU:     [gate | up], a = sigmoid(gate) * up.
Output of the forward: y = a(x) * p, evaluated in float64 and rounded once to float32 (the value that
is then block-quantized; it is never rounded to BF16 first).
Backward: dp[r] = sum_j dy[r, j] * a(x[r])_j ;  dx = dy * p * da/dx, rounded once to float32.

Parity: SReLU forward and backward are exact closed forms (pinned by exact representable inputs);
TanhSReLU, SwiGLU and ClampedSwiGLU gradients are pinned by central finite differences and limits;
GeLU by the textbook value Phi(1), the odd-part identity GeLU(x) - GeLU(-x) = x and its limits;
sigmoid by sigmoid(ln 3) = 3/4 and the symmetry sigmoid(x) + sigmoid(-x) = 1; GLU by its values at
gate = 0 and gate = ln 3; all gradients by central differences.  The formulas of TanhSReLU / SwiGLU /
ClampedSwiGLU / GeLU / sigmoid / GLU themselves are readings (parity unpinned as to the formula,
since the pages print none).
"""

import numpy as np
from scipy.special import erf

from .codecs import f32

SRELU = "srelu"
TANH_SRELU = "tanh_srelu"
SWIGLU = "swiglu"
CLAMPED_SWIGLU = "clamped_swiglu"
IDENTITY = "identity"
GELU = "gelu"
SIGMOID = "sigmoid"
GLU = "glu"

GATED = (SWIGLU, CLAMPED_SWIGLU, GLU)


def out_width(kind, width_in):
    return width_in // 2 if kind in GATED else width_in


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def act(kind, x, s=2.0, limit=7.0, alpha=1.0, beta=0.0):
    """a(x) without the per-row scale. x: float64 [rows, width_in]."""
    x = np.asarray(x, dtype=np.float64)
    if kind == IDENTITY:
        return x.copy()
    if kind == SRELU:
        r = np.maximum(x, 0.0)
        return r * r
    if kind == TANH_SRELU:
        r = np.maximum(x, 0.0)
        t = s * np.tanh(r / s)
        return t * t
    if kind == GELU:
        return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))
    if kind == SIGMOID:
        return _sigmoid(x)
    w = x.shape[-1] // 2
    g, u = x[..., :w], x[..., w:]
    if kind == SWIGLU:
        return g * _sigmoid(g) * u
    if kind == GLU:
        return _sigmoid(g) * u
    if kind == CLAMPED_SWIGLU:
        gc = np.minimum(g, limit)
        uc = np.clip(u, -limit, limit)
        return gc * _sigmoid(alpha * gc) * (uc + beta)
    raise ValueError(kind)


def act_grad(kind, x, s=2.0, limit=7.0, alpha=1.0, beta=0.0):
    """Partial derivatives of a(x).

    Unary kinds: returns da/dx, same shape as x (elementwise).
    Gated kinds: returns (da/dgate, da/dup), each [rows, width_in / 2].
    """
    x = np.asarray(x, dtype=np.float64)
    if kind == IDENTITY:
        return np.ones_like(x)
    if kind == SRELU:
        return 2.0 * np.maximum(x, 0.0)
    if kind == TANH_SRELU:
        r = np.maximum(x, 0.0)
        t = np.tanh(r / s)
        return np.where(x > 0.0, 2.0 * s * t * (1.0 - t * t), 0.0)
    if kind == GELU:
        # Phi(x) + x phi(x)
        return 0.5 * (1.0 + erf(x / np.sqrt(2.0))) + x * np.exp(-0.5 * x * x) / np.sqrt(2.0 * np.pi)
    if kind == SIGMOID:
        sg = _sigmoid(x)
        return sg * (1.0 - sg)
    w = x.shape[-1] // 2
    g, u = x[..., :w], x[..., w:]
    if kind == SWIGLU:
        sg = _sigmoid(g)
        return u * sg * (1.0 + g * (1.0 - sg)), g * sg
    if kind == GLU:
        sg = _sigmoid(g)
        return u * sg * (1.0 - sg), sg
    if kind == CLAMPED_SWIGLU:
        gc = np.minimum(g, limit)
        uc = np.clip(u, -limit, limit)
        sg = _sigmoid(alpha * gc)
        dg = np.where(g <= limit, (uc + beta) * sg * (1.0 + alpha * gc * (1.0 - sg)), 0.0)
        du = np.where((u >= -limit) & (u <= limit), gc * sg, 0.0)
        return dg, du
    raise ValueError(kind)


def scaled_act_fwd(kind, x, p, **params):
    """y32 = f32(a(x) * p): the float32 value that the quantizers consume. p: [rows]."""
    a = act(kind, x, **params)
    return f32(a * np.asarray(p, dtype=np.float64)[:, None])


def scaled_act_bwd(kind, x, dy, p, **params):
    """Returns (dx32, dp32).

    dy is dL/d(a(x) * p) [rows, width_out]; dx32 = f32(dy * p * da/dx) [rows, width_in];
    dp32 = f32(sum_j dy * a(x)) [rows], summed in float64.
    """
    dy = np.asarray(dy, dtype=np.float64)
    p = np.asarray(p, dtype=np.float64)[:, None]
    a = act(kind, x, **params)
    dp = f32(np.sum(dy * a, axis=-1))
    if kind in GATED:
        dg, du = act_grad(kind, x, **params)
        dx = np.concatenate([dy * p * dg, dy * p * du], axis=-1)
    else:
        dx = dy * p * act_grad(kind, x, **params)
    return f32(dx), dp
