"""Seeded synthetic inputs for the grouped scaled-activation / block-quantize / grouped GEMM path.

This module only draws random numbers and lays them out; it holds none of the method's arithmetic.
Both the oracle-based tests and the GPU path consume what it returns.  All draws come from one
``numpy.random.default_rng(seed)`` stream per workload, in the order documented in each function.

BF16 tensors are returned as uint16 bit patterns (float32 normal samples rounded to nearest-even);
FP32 tensors as float32 arrays; split sizes as int64.

The five named workloads follow the shapes and distributions of the method's test setups:
  srelu_small   4 experts, splits [64, 128, 32, 32], width 512, ScaledSReLU, MXFP8 rowwise, FC2 512 -> 256
  tanh_nvfp4    4 experts x 512 tokens, width 1024, ScaledTanhSReLU s = 2, NVFP4 row + col, fwd + bwd
  swiglu_zipf   8 experts, 8192 tokens Zipf(1.2) split (one empty expert), FC1 out 2 x 2048, MXFP8
  clamped_fc2   32 experts, 65536 tokens Zipf(1.2) split (four empty), clamped SwiGLU L = 7, FC2 to 7168
  mlp_step      16 experts x 2048 tokens, hidden 4096, ffn 4096, full FC1 -> act -> FC2 train step
"""

import numpy as np


def bf16_bits(x):
    """Round float32 samples to BF16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(rng, shape, std=1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return bf16_bits(x)


def uniform_f32(rng, n):
    return rng.random(size=n, dtype=np.float32)


def zipf_split(rng, n_tokens, n_experts, a=1.2, n_zero=0):
    """Zipf-skewed split sizes with ``n_zero`` empty experts.

    Rank weights w_k = k^-a for k <= n_experts - n_zero (0 for the rest), counts drawn from one
    multinomial over the weights, then assigned to experts by a random permutation.
    """
    k = np.arange(1, n_experts + 1, dtype=np.float64)
    w = np.where(k <= n_experts - n_zero, k ** -a, 0.0)
    counts = rng.multinomial(n_tokens, w / w.sum())
    order = rng.permutation(n_experts)
    splits = np.zeros(n_experts, dtype=np.int64)
    splits[order] = counts
    return splits


def top2_probs(rng, n_tokens, n_logits=8):
    """Routing probabilities: softmax over the two largest of n_logits N(0,1) logits per token.

    Returns 2 * n_tokens float32 values in token order (top-1, top-2 for each token).
    """
    logits = rng.standard_normal(size=(n_tokens, n_logits))
    top = -np.sort(-logits, axis=1)[:, :2]
    ex = np.exp(top - top[:, :1])
    pr = ex / ex.sum(axis=1, keepdims=True)
    return pr.reshape(-1).astype(np.float32)


WORKLOADS = ("srelu_small", "tanh_nvfp4", "swiglu_zipf", "clamped_fc2", "mlp_step")


def make(name, seed=0, tokens=None, act="srelu"):
    """Inputs of a named workload.  ``tokens`` shrinks the token count (tests only)."""
    rng = np.random.default_rng(seed)
    if name == "srelu_small":
        splits = np.array([64, 128, 32, 32], dtype=np.int64)
        m = int(splits.sum())
        return dict(name=name, kind="srelu", fmt="mxfp8", splits=splits, width_in=512, hidden=256,
                    x=normal_bf16(rng, (m, 512)), p=uniform_f32(rng, m),
                    w2=normal_bf16(rng, (4, 256, 512), 0.02))
    if name == "tanh_nvfp4":
        n = tokens or 2048
        splits = np.full(4, n // 4, dtype=np.int64)
        m = int(splits.sum())
        return dict(name=name, kind="tanh_srelu", fmt="nvfp4", splits=splits, width_in=1024, s=2.0,
                    x=normal_bf16(rng, (m, 1024), 1.5), p=uniform_f32(rng, m),
                    dy=normal_bf16(rng, (m, 1024)))
    if name == "swiglu_zipf":
        n = tokens or 8192
        splits = zipf_split(rng, n, 8, 1.2, 1)
        m = int(splits.sum())
        x = normal_bf16(rng, (m, 4096))
        p = top2_probs(rng, m // 2)
        return dict(name=name, kind="swiglu", fmt="mxfp8", splits=splits, width_in=4096, hidden=4096,
                    x=x, p=p, dy=normal_bf16(rng, (m, 2048)))
    if name == "clamped_fc2":
        n = tokens or 65536
        splits = zipf_split(rng, n, 32, 1.2, 4)
        m = int(splits.sum())
        return dict(name=name, kind="clamped_swiglu", fmt="mxfp8", splits=splits, width_in=4096,
                    hidden=7168, limit=7.0,
                    x=normal_bf16(rng, (m, 4096)), p=uniform_f32(rng, m),
                    w2=normal_bf16(rng, (32, 7168, 2048), 0.02),
                    dy2=normal_bf16(rng, (m, 7168)),
                    # upstream gradient of the activation output (isolated-kernel tests), drawn last
                    dy=normal_bf16(rng, (m, 2048)))
    if name == "mlp_step":
        n = tokens or 32768
        e = 16
        splits = np.full(e, n // e, dtype=np.int64)
        m = int(splits.sum())
        h, f = 4096, 4096
        return dict(name=name, kind=act, splits=splits, hidden=h, ffn=f, s=2.0,
                    x1=normal_bf16(rng, (m, h)),
                    w1=normal_bf16(rng, (e, f, h), 0.02), w2=normal_bf16(rng, (e, h, f), 0.02),
                    b1=normal_bf16(rng, (e, f), 0.02), b2=normal_bf16(rng, (e, h), 0.02),
                    p=uniform_f32(rng, m), dy2=normal_bf16(rng, (m, h)))
    raise ValueError(name)


def act_case(kind, splits, width_in, seed=0, std=1.0, with_dy=True):
    """A generic activation test case: x [M, width_in] ~ N(0, std^2) BF16, p ~ U(0,1), dy ~ N(0,1)."""
    rng = np.random.default_rng(seed)
    splits = np.asarray(splits, dtype=np.int64)
    m = int(splits.sum())
    wa = width_in // 2 if kind in ("swiglu", "clamped_swiglu", "glu") else width_in
    d = dict(kind=kind, splits=splits, width_in=width_in, x=normal_bf16(rng, (m, width_in), std),
             p=uniform_f32(rng, m))
    if with_dy:
        d["dy"] = normal_bf16(rng, (m, wa))
    return d
