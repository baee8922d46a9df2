"""The seeded input generators: determinism, shapes, split properties."""

import numpy as np

import workloads


def test_zipf_split_properties():
    rng = np.random.default_rng(0)
    s = workloads.zipf_split(rng, 65536, 32, 1.2, 4)
    assert s.sum() == 65536 and (s == 0).sum() >= 4 and s.max() > 10000
    s8 = workloads.zipf_split(np.random.default_rng(0), 8192, 8, 1.2, 1)
    assert s8.sum() == 8192 and (s8 == 0).sum() >= 1


def test_top2_probs_sum_to_one_per_token():
    p = workloads.top2_probs(np.random.default_rng(0), 100).reshape(100, 2)
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-6) and np.all(p[:, 0] >= p[:, 1])


def test_deterministic_and_bf16_rounding():
    a = workloads.make("srelu_small", seed=0)
    b = workloads.make("srelu_small", seed=0)
    assert np.array_equal(a["x"], b["x"]) and a["x"].dtype == np.uint16 and a["x"].shape == (256, 512)
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20], dtype=np.float32)
    # ties to even: 1 + 2^-8 -> 1.0; 1 + 3*2^-8 -> 1 + 2^-6; just above the tie rounds up
    assert workloads.bf16_to_f32(workloads.bf16_bits(x)).tolist() == [1.0, 1.015625, 1.0078125]


def test_small_token_variants():
    d = workloads.make("swiglu_zipf", tokens=512)
    assert d["x"].shape == (512, 4096) and d["p"].shape == (512,) and d["dy"].shape == (512, 2048)
