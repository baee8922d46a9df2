"""Parity at the full expert-MLP workload (16 experts x 2048 tokens, hidden 4096, ffn 4096,
ScaledSReLU, bias, activation recompute, delayed wgrad; MXFP8 and NVFP4), in the launch configuration
bench.py times.

Every quantity of the step is local to an expert: rowwise blocks lie inside a token row, the
columnwise blocks and the weight-gradient sums inside one expert's token range, each expert's weights
are quantized on their own, and the NVFP4 per-tensor amax is taken per expert.  So the oracle step run
on one expert's 2048 tokens and weights fixes that expert's FC1 output, FC2 output, dx1, dprobs, dW1,
dW2, db1 and db2 exactly as in the whole 16-expert step; the test compares all of them for the last
expert (non-zero row and column offsets).

Tolerances are those of the small oracle step test (chained BF16 and quantization roundings; rare bin
flips propagate), and the GEMM criterion for the FC1 output, which sees one quantization only.
"""

import numpy as np
import pytest

import workloads
from oracle import mlp as M
from tests.helpers import bf16_f64, bf16_host, f32, rel_rms, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

E, T, H, F = 16, 2048, 4096, 4096
GROUP = 15


@pytest.fixture(scope="module")
def step_inputs():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return workloads.make("mlp_step", seed=0, act="srelu")


@pytest.mark.parametrize("fmt", ["mxfp8", "nvfp4"])
def test_full_step_last_expert_matches_oracle(step_inputs, fmt):
    import torch
    from moe_grouped_scaled_amd.expert_mlp import ExpertMLP
    d = step_inputs
    splits = list(map(int, d["splits"]))
    assert splits == [T] * E and d["hidden"] == H and d["ffn"] == F
    mlp = ExpertMLP("srelu", fmt, to_dev_bf16(d["w1"]), to_dev_bf16(d["w2"]), to_dev_bf16(d["b1"]),
                    to_dev_bf16(d["b2"]), recompute=True, delay_wgrad=True, s=2.0)
    y2 = mlp.forward(to_dev_bf16(d["x1"]), to_dev(d["p"]), splits)
    sl = slice(GROUP * T, (GROUP + 1) * T)
    y1 = bf16_host(mlp.ctx["y1"][sl])
    g = mlp.backward(to_dev_bf16(d["dy2"]))
    g.update(mlp.backward_dw())
    torch.cuda.synchronize()
    got = {"y1": bf16_f64(y1), "y2": bf16_f64(bf16_host(y2[sl])), "dx1": bf16_f64(bf16_host(g["dx1"][sl])),
           "dp": f32(g["dprobs"][sl]), "dw1": f32(g["dw1"][GROUP]), "dw2": f32(g["dw2"][GROUP]),
           "db1": f32(g["db1"][GROUP]), "db2": f32(g["db2"][GROUP])}
    del mlp, y2, g
    ref = M.mlp_step("srelu", fmt, [T], bf16_f64(d["x1"][sl]), bf16_f64(d["w1"][GROUP][None]),
                     bf16_f64(d["b1"][GROUP][None]), bf16_f64(d["w2"][GROUP][None]),
                     bf16_f64(d["b2"][GROUP][None]), d["p"][sl].astype(np.float64), bf16_f64(d["dy2"][sl]))
    refs = {k: ref[k] for k in ("y1", "y2", "dx1", "dp")}
    refs.update({k: ref[k][0] for k in ("dw1", "dw2", "db1", "db2")})
    tol = {"y1": 1e-3, "y2": 5e-3, "dx1": 1e-2, "dp": 1e-2, "dw1": 1e-2, "dw2": 5e-3, "db1": 1e-2,
           "db2": 1e-5}
    errs = {k: rel_rms(got[k], refs[k]) for k in tol}
    print(fmt, "expert", GROUP, {k: "%.2e" % v for k, v in errs.items()}, flush=True)
    for k in tol:
        assert errs[k] <= tol[k], (k, errs[k])
