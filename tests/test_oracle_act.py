"""Pins of the oracle's scaled activations: closed forms, limits, finite differences, exact dprobs."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import activations as A
from oracle.codecs import f32

KINDS = [A.SRELU, A.TANH_SRELU, A.SWIGLU, A.CLAMPED_SWIGLU, A.GELU, A.SIGMOID, A.GLU]


def test_srelu_exact_values():
    x = np.array([[1.5, -3.0, 0.0, 2.0]])
    p = np.array([0.5])
    y = A.scaled_act_fwd(A.SRELU, x, p)
    assert y.tolist() == [[1.125, 0.0, 0.0, 2.0]]
    dx, dp = A.scaled_act_bwd(A.SRELU, x, np.array([[1.0, 1.0, 1.0, 0.5]]), p)
    # dx = dy * p * 2 relu(x);  dp = sum dy * relu(x)^2
    assert dx.tolist() == [[1.5, 0.0, 0.0, 1.0]]
    assert dp.tolist() == [2.25 + 2.0]


def test_srelu_single_rounding_equals_fp32_sequence():
    """For BF16 x, x*x is exact in FP32, so one rounding of x^2 * p equals fl32(fl32(x*x) * p)."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal((64, 64)).astype(np.float32)
    x = (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)  # BF16 values
    p = rng.random(64).astype(np.float32)
    r = np.maximum(x, 0)
    seq = (r * r) * p[:, None]  # float32 arithmetic
    got = A.scaled_act_fwd(A.SRELU, x.astype(np.float64), p.astype(np.float64))
    assert np.array_equal(got, seq.astype(np.float64))


def test_tanh_srelu_bounds_and_limit():
    s = 2.0
    x = np.linspace(-5, 50, 2001)[None, :]
    y = A.act(A.TANH_SRELU, x, s=s)
    assert np.all(y <= s * s + 1e-12)
    assert np.all(y >= 0)
    assert abs(y[0, -1] - s * s) < 1e-12
    small = np.array([[1e-3, 1e-2]])
    rel = A.act(A.TANH_SRELU, small, s=s) / small ** 2 - 1
    assert np.all(np.abs(rel) < 1e-4)          # -> relu(x)^2 for x << s
    big_s = A.act(A.TANH_SRELU, np.array([[1.7]]), s=1e4)
    assert abs(big_s[0, 0] - 1.7 ** 2) < 1e-6   # -> relu(x)^2 as s -> inf


def test_swiglu_values():
    x = np.array([[0.0, 1.0, 3.0, 2.0]])  # gate [0, 1], up [3, 2]
    y = A.act(A.SWIGLU, x)
    assert y[0, 0] == 0.0
    assert abs(y[0, 1] - 1.0 / (1 + np.exp(-1.0)) * 2.0) < 1e-15


def test_clamped_swiglu_regions():
    L = 7.0
    # gate above the limit is held at L; up clamped to [-L, L]
    x = np.array([[9.0, 3.0, 20.0, -20.0]])
    y = A.act(A.CLAMPED_SWIGLU, x, limit=L)
    sig = 1 / (1 + np.exp(-L))
    assert abs(y[0, 0] - L * sig * L) < 1e-12
    assert abs(y[0, 1] - 3 * (1 / (1 + np.exp(-3.0))) * -L) < 1e-12
    dg, du = A.act_grad(A.CLAMPED_SWIGLU, x, limit=L)
    assert dg[0, 0] == 0.0 and du[0, 0] == 0.0 and du[0, 1] == 0.0 and dg[0, 1] != 0.0
    # equality passes the gradient (inclusive bounds)
    dg, du = A.act_grad(A.CLAMPED_SWIGLU, np.array([[7.0, -7.0]]), limit=L)
    assert dg[0, 0] != 0.0 and du[0, 0] != 0.0
    # alpha/beta variant reduces to plain SwiGLU far from the limits when alpha = 1, beta = 0
    z = np.array([[0.3, -1.2, 0.7, 2.5]])
    assert np.allclose(A.act(A.CLAMPED_SWIGLU, z, limit=L), A.act(A.SWIGLU, z), rtol=0, atol=1e-15)


def test_gelu_values_and_identities():
    """GeLU(x) = x Phi(x): the tabulated standard normal CDF Phi(1) = 0.841344746068543, GeLU(0) = 0,
    the odd-part identity GeLU(x) - GeLU(-x) = x (Phi(x) + Phi(-x) = 1), and the limits x and 0."""
    x = np.array([[1.0, -1.0, 0.0, 8.0, -8.0]])
    a = A.act(A.GELU, x)[0]
    assert abs(a[0] - 0.841344746068543) < 1e-14
    assert abs(a[1] + (1.0 - 0.841344746068543)) < 1e-14
    assert a[2] == 0.0
    assert abs(a[3] - 8.0) < 1e-12 and abs(a[4]) < 1e-12
    rng = np.random.default_rng(5)
    z = rng.standard_normal((3, 64)) * 3
    assert np.allclose(A.act(A.GELU, z) - A.act(A.GELU, -z), z, rtol=0, atol=1e-14)
    # the slope at 0 is Phi(0) = 1/2
    assert abs(A.act_grad(A.GELU, np.zeros((1, 1)))[0, 0] - 0.5) < 1e-15


def test_sigmoid_and_glu_values():
    """sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4 exactly in exact arithmetic, sigmoid(x) + sigmoid(-x) = 1;
    GLU = sigmoid(gate) * up at those gates; its up-gradient is sigmoid(gate)."""
    l3 = np.log(3.0)
    s = A.act(A.SIGMOID, np.array([[0.0, l3, -l3]]))[0]
    assert s[0] == 0.5 and abs(s[1] - 0.75) < 1e-15 and abs(s[2] - 0.25) < 1e-15
    rng = np.random.default_rng(6)
    z = rng.standard_normal((2, 32)) * 4
    assert np.allclose(A.act(A.SIGMOID, z) + A.act(A.SIGMOID, -z), 1.0, rtol=0, atol=1e-15)
    x = np.array([[0.0, l3, 2.0, -4.0]])   # gates 0, ln 3; ups 2, -4
    a = A.act(A.GLU, x)[0]
    assert a[0] == 1.0 and abs(a[1] + 3.0) < 1e-14
    dg, du = A.act_grad(A.GLU, x)
    assert du[0, 0] == 0.5 and abs(du[0, 1] - 0.75) < 1e-15
    assert abs(dg[0, 0] - 2.0 * 0.25) < 1e-15 and abs(dg[0, 1] + 4.0 * 0.75 * 0.25) < 1e-14


# alpha / beta exist for clamped SwiGLU only
@pytest.mark.parametrize("kind,params", [(k, {}) for k in KINDS]
                         + [(A.CLAMPED_SWIGLU, {"alpha": 1.702, "beta": 1.0})])
def test_gradients_match_central_differences(kind, params):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 16)) * 3.0
    # keep away from kinks (0 for relu, +-L for the clamp)
    x = np.where(np.abs(x) < 0.05, 0.3, x)
    x = np.where(np.abs(np.abs(x) - 7.0) < 0.05, 6.5, x)
    h = 1e-6
    base = A.act(kind, x, **params)
    if kind in A.GATED:
        dg, du = A.act_grad(kind, x, **params)
        grads = np.concatenate([dg, du], axis=1)
        w = x.shape[1] // 2
        for j in range(x.shape[1]):
            xp, xm = x.copy(), x.copy()
            xp[:, j] += h
            xm[:, j] -= h
            fd = (A.act(kind, xp, **params) - A.act(kind, xm, **params))[:, j % w] / (2 * h)
            assert np.allclose(fd, grads[:, j], rtol=1e-6, atol=1e-7)
    else:
        g = A.act_grad(kind, x, **params)
        fd = (A.act(kind, x + h, **params) - A.act(kind, x - h, **params)) / (2 * h)
        assert np.allclose(fd, g, rtol=1e-6, atol=1e-7)
    assert base.shape[1] == A.out_width(kind, x.shape[1])


@pytest.mark.parametrize("kind", KINDS)
def test_backward_matches_gradient_of_loss(kind):
    """dx and dp are the gradients of L = sum dy * a(x) * p (central differences in float64)."""
    rng = np.random.default_rng(2)
    m, w_in = 3, 8
    x = rng.standard_normal((m, w_in)) * 2
    x = np.where(np.abs(x) < 0.05, 0.4, x)
    p = rng.random(m)
    wa = A.out_width(kind, w_in)
    dy = rng.standard_normal((m, wa))

    def loss(xx, pp):
        return np.sum(dy * A.act(kind, xx) * pp[:, None])

    dx, dp = A.scaled_act_bwd(kind, x, dy, p)
    h = 1e-6
    for r in range(m):
        pp, pm = p.copy(), p.copy()
        pp[r] += h
        pm[r] -= h
        assert abs((loss(x, pp) - loss(x, pm)) / (2 * h) - dp[r]) <= 1e-6 * max(1.0, abs(dp[r]))
        for j in range(w_in):
            xp, xm = x.copy(), x.copy()
            xp[r, j] += h
            xm[r, j] -= h
            fd = (loss(xp, p) - loss(xm, p)) / (2 * h)
            assert abs(fd - dx[r, j]) <= 1e-5 * max(1.0, abs(fd))


def test_dprobs_exact_rationals_srelu():
    """Brute force with exact rationals: dp_r = sum_j dy_rj * relu(x_rj)^2, then one FP32 rounding."""
    rng = np.random.default_rng(3)
    m, w = 8, 64
    x = rng.standard_normal((m, w)).astype(np.float32)
    x = (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)
    dy = rng.standard_normal((m, w)).astype(np.float32)
    dy = (dy.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)
    p = rng.random(m)
    _, dp = A.scaled_act_bwd(A.SRELU, x, dy, p)
    for r in range(m):
        exact = sum(Fraction(float(dy[r, j])) * Fraction(float(max(x[r, j], 0.0))) ** 2 for j in range(w))
        want = f32(float(exact))  # float(Fraction) is correctly rounded
        ulp = abs(np.spacing(np.float32(want)))
        assert abs(dp[r] - want) <= ulp, (r, dp[r], want)


def test_dprobs_invariant():
    """sum_r dp_r p_r = sum_{r,j} dy_rj a_rj p_r (the scale gradient closes the chain rule)."""
    rng = np.random.default_rng(4)
    for kind in KINDS:
        x = rng.standard_normal((16, 32))
        p = rng.random(16)
        dy = rng.standard_normal((16, A.out_width(kind, 32)))
        _, dp = A.scaled_act_bwd(kind, x, dy, p)
        lhs = np.sum(dp * p)
        rhs = np.sum(dy * A.act(kind, x) * p[:, None])
        assert abs(lhs - rhs) <= 1e-6 * np.sum(np.abs(dy * A.act(kind, x))) + 1e-12
