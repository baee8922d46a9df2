"""Device-resident split sizes: the graph-safe form of the step.

Page "Activation + GroupedLinear Fusion for MOE", Greptile summary, third bullet: GroupedLinear gains
a graph-safe forward (_fuser_forward_graph_safe), whose split sizes stay on the device so a captured
graph can run for a new routing.  Here the split sizes live in a device tensor, every kernel of the
step reads the group offsets a small kernel derives from them, and the layouts are strided for a row
capacity, so one captured HIP graph of the whole training step (forward, backward, delayed weight
gradients) is replayed over different routings.

Checks:
  * the step with device-resident split sizes equals the step with host split sizes bit for bit on
    every output row in use (the same kernels and arithmetic; only strides and grids differ), for
    both recipes, the FP32-output forward and Hadamard-transformed NVFP4 copies;
  * one graph captured once and replayed over alternating routings (with eager work and
    synchronizations between replays) gives, at every replay, the eager step's outputs bit for bit,
    and those agree with the oracle step at the same split sizes;
  * the NVFP4 step captured once follows each replay's routing (its per-group amax included);
  * invalid split sizes (a sum above the capacity, a negative one) set the status word and the calls
    write nothing;
  * the standalone column sum reads the device offsets.
"""

import numpy as np
import pytest

import workloads
from oracle import mlp as M
from tests.helpers import bf16_f64, bf16_host, f32, rel_rms, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

E, H, F, CAP = 4, 128, 128, 512
ROUTINGS = ([64, 0, 96, 37], [200, 150, 0, 100], [0, 0, 0, 512])


@pytest.fixture(scope="module")
def N():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from moe_grouped_scaled_amd import _native
    return _native


def _weights(kind, seed=3):
    rng = np.random.default_rng(seed)
    f_in = 2 * F if kind in ("swiglu", "clamped_swiglu", "glu") else F
    return dict(w1=workloads.normal_bf16(rng, (E, f_in, H), 0.05), w2=workloads.normal_bf16(rng, (E, H, F), 0.05),
                b1=workloads.normal_bf16(rng, (E, f_in), 0.05), b2=workloads.normal_bf16(rng, (E, H), 0.05),
                x1=workloads.normal_bf16(rng, (CAP, H)), p=workloads.uniform_f32(rng, CAP),
                dy2=workloads.normal_bf16(rng, (CAP, H)))


def _mlp(kind, d, fmt="mxfp8", fp32_act=False, rht=None):
    from moe_grouped_scaled_amd.expert_mlp import ExpertMLP
    return ExpertMLP(kind, fmt, to_dev_bf16(d["w1"]), to_dev_bf16(d["w2"]), to_dev_bf16(d["b1"]),
                     to_dev_bf16(d["b2"]), recompute=True, delay_wgrad=True, fuse_fc1_act="auto",
                     fc1_fp32_act=fp32_act, rht_signs=rht)


def _step(mlp, x1, p, dy2, splits):
    y2 = mlp.forward(x1, p, splits)
    g = mlp.backward(dy2)
    g.update(mlp.backward_dw())
    g["y2"] = y2
    return g


def _host(g, m):
    return {"y2": bf16_host(g["y2"][:m]), "dx1": bf16_host(g["dx1"][:m]), "dprobs": f32(g["dprobs"][:m]),
            "dw1": f32(g["dw1"]), "dw2": f32(g["dw2"]), "db1": f32(g["db1"]), "db2": f32(g["db2"])}


CASES = [("srelu", "mxfp8", False, None), ("swiglu", "mxfp8", False, None), ("srelu", "mxfp8", True, None),
         ("srelu", "nvfp4", False, None), ("tanh_srelu", "nvfp4", True, None), ("glu", "nvfp4", False, 0x6B35)]


@pytest.mark.parametrize("kind,fmt,fp32_act,rht", CASES)
def test_device_splits_step_equals_host_splits_step(N, kind, fmt, fp32_act, rht):
    """Both recipes, the FP32-output forward and the Hadamard-transformed NVFP4 copies: the step with
    device-resident split sizes writes the host-split step's bits on every row in use."""
    import torch
    d = _weights(kind)
    x1, p, dy2 = to_dev_bf16(d["x1"]), to_dev(d["p"]), to_dev_bf16(d["dy2"])
    dg = N.DeviceGroups(E, CAP)
    for splits in ROUTINGS:
        m = int(sum(splits))
        print("case:", kind, fmt, "fp32_act" if fp32_act else "", "rht" if rht else "", "splits", splits, flush=True)
        ref = _host(_step(_mlp(kind, d, fmt, fp32_act, rht), x1[:m].contiguous(), p[:m].contiguous(),
                          dy2[:m].contiguous(), splits), m)
        dg.splits.copy_(torch.tensor(splits, dtype=torch.int64))
        got = _host(_step(_mlp(kind, d, fmt, fp32_act, rht), x1, p, dy2, dg), m)
        torch.cuda.synchronize()
        assert int(dg.status.item()) == 0
        for k in ref:
            assert np.array_equal(got[k], ref[k]), (splits, k)


def test_one_graph_replayed_over_routings(N):
    """Capture the whole step once, then replay it for routings A, B, A, B, C with eager work and a
    synchronization between replays; every replay equals the eager host-splits step bit for bit and
    agrees with the oracle step at the same split sizes (the small-step tolerances)."""
    import torch
    kind = "srelu"
    d = _weights(kind)
    x1, p, dy2 = to_dev_bf16(d["x1"]), to_dev(d["p"]), to_dev_bf16(d["dy2"])
    dg = N.DeviceGroups(E, CAP)
    mlp = _mlp(kind, d)
    dg.splits.copy_(torch.tensor(ROUTINGS[0], dtype=torch.int64))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):                       # warm-up: the step's workspace exists before capture
            _step(mlp, x1, p, dy2, dg)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = _step(mlp, x1, p, dy2, dg)
    oracle_cache = {}
    for it, splits in enumerate([ROUTINGS[0], ROUTINGS[1], ROUTINGS[0], ROUTINGS[1], ROUTINGS[2]]):
        m = int(sum(splits))
        print("replay", it, "splits", splits, flush=True)
        dg.splits.copy_(torch.tensor(splits, dtype=torch.int64))
        graph.replay()
        torch.cuda.synchronize()
        got = _host(out, m)
        assert int(dg.status.item()) == 0
        # eager work between replays, then the eager host-splits step as the reference
        ref = _host(_step(_mlp(kind, d), x1[:m].contiguous(), p[:m].contiguous(), dy2[:m].contiguous(), splits), m)
        torch.cuda.synchronize()
        for k in ref:
            assert np.array_equal(got[k], ref[k]), (it, splits, k)
        key = tuple(splits)
        if key not in oracle_cache:
            oracle_cache[key] = M.mlp_step(kind, "mxfp8", list(splits), bf16_f64(d["x1"][:m]), bf16_f64(d["w1"]),
                                           bf16_f64(d["b1"]), bf16_f64(d["w2"]), bf16_f64(d["b2"]),
                                           d["p"][:m].astype(np.float64), bf16_f64(d["dy2"][:m]), recompute=True)
        o = oracle_cache[key]
        # the small-step MXFP8 bounds; db2 is an FP32 column sum of BF16 dY2 in a fixed order, whose
        # relative RMS error against the exact float64 sum stays below one unit roundoff (2^-24) at
        # these group sizes (measured 2.1e-8 over a 512-token group)
        tol = {"y2": 7e-3, "dx1": 7e-3, "dprobs": 8e-4, "dw1": 7e-3, "dw2": 8e-3, "db1": 8e-4, "db2": 2.0 ** -24}
        vals = {"y2": bf16_f64(got["y2"]), "dx1": bf16_f64(got["dx1"]), "dprobs": got["dprobs"], "dw1": got["dw1"],
                "dw2": got["dw2"], "db1": got["db1"], "db2": got["db2"]}
        refs = {"y2": o["y2"], "dx1": o["dx1"], "dprobs": o["dp"], "dw1": o["dw1"], "dw2": o["dw2"],
                "db1": o["db1"], "db2": o["db2"]}
        for k in tol:
            err = rel_rms(vals[k], refs[k])
            assert err <= tol[k], (it, splits, k, err)
        for g in range(E):
            if splits[g] == 0:
                assert not np.any(got["dw1"][g]) and not np.any(got["dw2"][g])


def test_invalid_device_splits_write_nothing(N):
    """A sum above the capacity or a negative split: status 1, and the quantizer and the M-grouped
    GEMM leave their outputs as they were."""
    import torch
    dg = N.DeviceGroups(E, CAP)
    x = torch.randn(CAP, H, device="cuda").to(torch.bfloat16)
    for bad in ([300, 300, 0, 0], [10, -5, 0, 0]):
        print("case: invalid splits", bad, flush=True)
        dg.splits.copy_(torch.tensor(bad, dtype=torch.int64))
        dg.update()
        qr = N.QTensor("mxfp8", False, dg, H)
        qr.data.fill_(0xA5)
        qr.scales.fill_(0xA5)
        N.grouped_mx_quantize("mxfp8", dg, H, x, qr, None)
        w = N.QTensor("mxfp8", False, [F] * E, H)
        N.grouped_mx_quantize("mxfp8", [F] * E, H, (torch.randn(E * F, H, device="cuda") * 0.05).to(torch.bfloat16), w, None)
        c = torch.full((CAP, F), 3.0, dtype=torch.float32, device="cuda")
        N.grouped_gemm_mx("fprop", "mxfp8", dg, CAP, F, H, qr, w, c)
        torch.cuda.synchronize()
        assert int(dg.status.item()) == 1
        assert bool((qr.data == 0xA5).all()) and bool((qr.scales == 0xA5).all())
        assert bool((c == 3.0).all())


def test_nvfp4_graph_replayed_over_routings(N):
    """The NVFP4 step (per-group amax and S_dec taken over each replay's rows) captured once and
    replayed over routings A, B, A, C: every replay equals the eager host-split step bit for bit."""
    import torch
    kind = "srelu"
    d = _weights(kind)
    x1, p, dy2 = to_dev_bf16(d["x1"]), to_dev(d["p"]), to_dev_bf16(d["dy2"])
    dg = N.DeviceGroups(E, CAP)
    mlp = _mlp(kind, d, "nvfp4")
    dg.splits.copy_(torch.tensor(ROUTINGS[0], dtype=torch.int64))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            _step(mlp, x1, p, dy2, dg)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = _step(mlp, x1, p, dy2, dg)
    for it, splits in enumerate([ROUTINGS[0], ROUTINGS[1], ROUTINGS[0], ROUTINGS[2]]):
        m = int(sum(splits))
        print("nvfp4 replay", it, "splits", splits, flush=True)
        dg.splits.copy_(torch.tensor(splits, dtype=torch.int64))
        graph.replay()
        torch.cuda.synchronize()
        got = _host(out, m)
        assert int(dg.status.item()) == 0
        ref = _host(_step(_mlp(kind, d, "nvfp4"), x1[:m].contiguous(), p[:m].contiguous(), dy2[:m].contiguous(),
                          splits), m)
        torch.cuda.synchronize()
        for k in ref:
            assert np.array_equal(got[k], ref[k]), (it, splits, k)


def test_col_sum_with_device_splits(N):
    """The standalone per-group column sum reads the device offsets: equal to the host-split call."""
    import torch
    x = (torch.randn(CAP, H, device="cuda")).to(torch.bfloat16)
    dg = N.DeviceGroups(E, CAP)
    for splits in ROUTINGS:
        m = int(sum(splits))
        dg.splits.copy_(torch.tensor(splits, dtype=torch.int64))
        dg.update()
        got = torch.full((E, H), 7.0, device="cuda")
        N.grouped_col_sum(dg, H, x, got)
        ref = torch.empty(E, H, device="cuda")
        N.grouped_col_sum(splits, H, x[:m].contiguous(), ref)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), splits
