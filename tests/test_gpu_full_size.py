"""Parity at the full expert-MLP workload (16 experts x 2048 tokens, hidden 4096, ffn 4096,
ScaledSReLU, bias, activation recompute, delayed wgrad; MXFP8 and NVFP4), in the launch configuration
bench.py times.

Every quantity of the step is local to an expert: rowwise blocks lie inside a token row, the
columnwise blocks and the weight-gradient sums inside one expert's token range, each expert's weights
are quantized on their own, and the NVFP4 per-tensor amax is taken per expert.  So the oracle step run
on one expert's 2048 tokens and weights fixes that expert's FC1 output, FC2 output, dx1, dprobs, dW1,
dW2, db1 and db2 exactly as in the whole 16-expert step.

Two tests use that oracle step of the last expert (non-zero row and column offsets):
  * the chained step: every output of the GPU step against the oracle's, within about twice the
    relative RMS each recipe measures (chained BF16 and quantization roundings; rare bin flips
    propagate through the chain);
  * the six grouped GEMMs of the step on identical operands: the oracle's quantized operands of that
    expert (FC1 input, weights, FC2 input, dY2, dY1) are quantized again on the GPU from the same
    values, asserted byte-identical, replicated to 16 experts (the step's grid), and every GEMM
    (FP32 output, and BF16 output where the step writes BF16) is within 1e-3 relative RMS of the
    oracle's float64 product for every expert.
"""

import numpy as np
import pytest

import workloads
from oracle import codecs
from oracle import gemm as G
from oracle import mlp as M
from tests.helpers import bf16_f64, bf16_host, f32, rel_rms, to_dev, to_dev_bf16, u8

pytestmark = pytest.mark.gpu

E, T, H, F = 16, 2048, 4096, 4096
GROUP = 15
TOL = 1e-3


@pytest.fixture(scope="module")
def step_inputs():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return workloads.make("mlp_step", seed=0, act="srelu")


@pytest.fixture(scope="module")
def oracle_last_expert(step_inputs):
    """The oracle step on the last expert's tokens and weights, per recipe (computed once)."""
    cache = {}

    def get(fmt):
        if fmt not in cache:
            d = step_inputs
            sl = slice(GROUP * T, (GROUP + 1) * T)
            cache[fmt] = M.mlp_step("srelu", fmt, [T], bf16_f64(d["x1"][sl]), bf16_f64(d["w1"][GROUP][None]),
                                    bf16_f64(d["b1"][GROUP][None]), bf16_f64(d["w2"][GROUP][None]),
                                    bf16_f64(d["b2"][GROUP][None]), d["p"][sl].astype(np.float64),
                                    bf16_f64(d["dy2"][sl]))
        return cache[fmt]
    return get


# measured relative RMS of the chained step (last expert, both recipes) and the bounds, about twice
# those: MXFP8 y1 2.3e-4, y2 1.4e-3, dx1 1.8e-3, dprobs 4.3e-4, dW1 1.2e-3, dW2 1.0e-3, db1 3.5e-4,
# db2 3.4e-8; NVFP4 every output <= 1.7e-5 (its dequantized products are exact in FP16 and its
# coarser grid sees no bin flips here)
CHAIN_TOL = {
    "mxfp8": {"y1": 5e-4, "y2": 3e-3, "dx1": 4e-3, "dp": 1e-3, "dw1": 2.5e-3, "dw2": 2e-3, "db1": 7e-4,
              "db2": 1e-7},
    "nvfp4": {"y1": 4e-5, "y2": 4e-5, "dx1": 4e-5, "dp": 4e-5, "dw1": 4e-5, "dw2": 4e-5, "db1": 4e-5,
              "db2": 1e-7},
}


@pytest.mark.parametrize("fmt", ["mxfp8", "nvfp4"])
def test_full_step_last_expert_matches_oracle(step_inputs, oracle_last_expert, fmt):
    import torch
    from moe_grouped_scaled_amd.expert_mlp import ExpertMLP
    d = step_inputs
    splits = list(map(int, d["splits"]))
    assert splits == [T] * E and d["hidden"] == H and d["ffn"] == F
    print("case: full step, 16 x 2048 tokens, 4096 / 4096, srelu", fmt, flush=True)
    mlp = ExpertMLP("srelu", fmt, to_dev_bf16(d["w1"]), to_dev_bf16(d["w2"]), to_dev_bf16(d["b1"]),
                    to_dev_bf16(d["b2"]), recompute=True, delay_wgrad=True, s=2.0, fuse_fc1_act="auto")
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
    ref = oracle_last_expert(fmt)
    refs = {k: ref[k] for k in ("y1", "y2", "dx1", "dp")}
    refs.update({k: ref[k][0] for k in ("dw1", "dw2", "db1", "db2")})
    tol = CHAIN_TOL[fmt]
    errs = {k: rel_rms(got[k], refs[k]) for k in tol}
    print(fmt, "expert", GROUP, {k: "%.2e" % v for k, v in errs.items()}, flush=True)
    for k in tol:
        assert errs[k] <= tol[k], (k, errs[k])


# ------------------------------------------------------------------ the six GEMMs, identical operands

def _quant_dev(N, fmt, splits, width, values, f32_input):
    """Identity quantization (row + col) on the GPU of a [M x width] tensor: BF16 bits or FP32."""
    import torch
    qr, qc = N.QTensor(fmt, False, splits, width), N.QTensor(fmt, True, splits, width)
    amax = torch.empty(len(splits), dtype=torch.float32, device="cuda") if fmt == "nvfp4" else None
    if f32_input:
        N.grouped_scaled_act_fwd_f32(N.act_params("identity"), fmt, splits, width, values, None, qr, qc, amax)
    else:
        N.grouped_mx_quantize(fmt, splits, width, values, qr, qc, amax)
    return qr, qc


def _group_bytes(q, fmt, colwise, splits, width, g):
    """Group g's bytes of a GPU qtensor, laid out as a single-group quantization of its rows."""
    m = int(sum(splits))
    off = np.concatenate([[0], np.cumsum(splits)])
    pad = [-(-int(s) // 128) * 128 for s in splits]
    coff = np.concatenate([[0], np.cumsum(pad)])
    if colwise:
        c0, c1 = int(coff[g]), int(coff[g + 1])
        db, sb = (1, 32) if fmt == "mxfp8" else (2, 16)
        return u8(q.data[width * c0 // db: width * c1 // db]), u8(q.scales[width * c0 // sb: width * c1 // sb])
    r0, r1 = int(off[g]), int(off[g + 1])
    if fmt == "mxfp8":
        steps = -(-width // 128)
        return (u8(q.data.view(m, width)[r0:r1]).reshape(-1),
                u8(q.scales.view(steps, m, 4)[:, r0:r1, :]).reshape(-1))
    return u8(q.data.view(m, width // 2)[r0:r1]).reshape(-1), u8(q.scales.view(m, width // 16)[r0:r1]).reshape(-1)


def _assert_same_operand(q_row, q_col, ref, fmt, splits, width, g, name):
    import torch
    for colwise, q in ((False, q_row), (True, q_col)):
        pre = "col" if colwise else "row"
        dat, sc = _group_bytes(q, fmt, colwise, splits, width, g)
        assert np.array_equal(dat, np.asarray(ref[pre + "_data"]).reshape(-1)), (name, pre, "data")
        assert np.array_equal(sc, np.asarray(ref[pre + "_scales"]).reshape(-1)), (name, pre, "scales")
        if fmt == "nvfp4":
            gs = f32(q.group_scale[g:g + 1])
            want = np.asarray(ref.get("col_group_scale" if colwise else "group_scale", ref["group_scale"]))[:1]
            assert np.array_equal(gs, want.astype(np.float64)), (name, pre, "group scale")


@pytest.mark.parametrize("fmt", ["mxfp8", "nvfp4"])
def test_full_step_gemms_on_identical_operands(step_inputs, oracle_last_expert, fmt):
    import torch
    from moe_grouped_scaled_amd import _native as N
    d = step_inputs
    ref = oracle_last_expert(fmt)
    print("case: six GEMMs of the full step on identical operands,", fmt, flush=True)
    splits = [T] * E
    sl = slice(GROUP * T, (GROUP + 1) * T)
    rep = lambda t: t.repeat(E, 1).contiguous()
    # operands on the GPU: the last expert's values, replicated to all 16 experts
    x1 = rep(to_dev_bf16(d["x1"][sl]))
    w1 = rep(to_dev_bf16(d["w1"][GROUP]))                  # [E * F x H]
    w2 = rep(to_dev_bf16(d["w2"][GROUP]))                  # [E * H x F]
    dy2 = rep(to_dev_bf16(d["dy2"][sl]))
    a32 = rep(to_dev(ref["a32"].astype(np.float32)))       # FC2's input, FP32 (the quantizer's input)
    dy1 = rep(to_dev(ref["dy1"].astype(np.float32)))       # FP32 dL/dY1
    b1 = to_dev_bf16(np.tile(d["b1"][GROUP][None], (E, 1)))
    b2 = to_dev_bf16(np.tile(d["b2"][GROUP][None], (E, 1)))
    x1r, x1c = _quant_dev(N, fmt, splits, H, x1, False)
    w1r, w1c = _quant_dev(N, fmt, [F] * E, H, w1, False)
    w2r, w2c = _quant_dev(N, fmt, [H] * E, F, w2, False)
    dy2r, dy2c = _quant_dev(N, fmt, splits, H, dy2, False)
    ar, ac = _quant_dev(N, fmt, splits, F, a32, True)
    dy1r, dy1c = _quant_dev(N, fmt, splits, F, dy1, True)
    torch.cuda.synchronize()
    for qr, qc, key, sp, w, name in ((x1r, x1c, "q_x1", splits, H, "X1"), (w1r, w1c, "q_w1", [F] * E, H, "W1"),
                                     (w2r, w2c, "q_w2", [H] * E, F, "W2"), (dy2r, dy2c, "q_dy2", splits, H, "dY2"),
                                     (ar, ac, "q_a", splits, F, "A"), (dy1r, dy1c, "q_dy1", splits, F, "dY1")):
        _assert_same_operand(qr, qc, ref[key], fmt, sp, w, GROUP, name)
    # the oracle's products on its own (now known identical) operands
    deq_r = lambda q, rows, w: G.dequant_row_grouped(fmt, q["row_data"], q["row_scales"], [rows], w, q.get("group_scale"))
    deq_c = lambda q, w, n: G.dequant_col_grouped(fmt, q["col_data"], q["col_scales"], [n], w,
                                                  q.get("col_group_scale", q.get("group_scale")))[0]
    qx, qw1, qa, qw2, qd2, qd1 = (ref[k] for k in ("q_x1", "q_w1", "q_a", "q_w2", "q_dy2", "q_dy1"))
    b1f, b2f = bf16_f64(d["b1"][GROUP]), bf16_f64(d["b2"][GROUP])
    refs = {
        "fc1_fprop": deq_r(qx, T, H) @ deq_r(qw1, F, H).T + b1f,            # [T x F]
        "fc2_fprop": deq_r(qa, T, F) @ deq_r(qw2, H, F).T + b2f,            # [T x H]
        "fc2_dgrad": deq_r(qd2, T, H) @ deq_c(qw2, F, H)[:, :H].T,          # dY2 . W2 -> [T x F]
        "fc1_dgrad": deq_r(qd1, T, F) @ deq_c(qw1, H, F)[:, :F].T,          # dY1 . W1 -> [T x H]
        "fc2_wgrad": deq_c(qd2, H, T) @ deq_c(qa, F, T).T,                  # [H x F]
        "fc1_wgrad": deq_c(qd1, F, T) @ deq_c(qx, H, T).T,                  # [F x H]
    }
    m = E * T
    runs = {
        "fc1_fprop": ("fprop", m, F, H, x1r, w1r, (m, F), b1),
        "fc2_fprop": ("fprop", m, H, F, ar, w2r, (m, H), b2),
        "fc2_dgrad": ("dgrad", m, F, H, dy2r, w2c, (m, F), None),
        "fc1_dgrad": ("dgrad", m, H, F, dy1r, w1c, (m, H), None),
        "fc2_wgrad": ("wgrad", H, F, m, dy2c, ac, (E, H, F), None),
        "fc1_wgrad": ("wgrad", F, H, m, dy1c, x1c, (E, F, H), None),
    }
    worst = {}
    for name, (mode, mm, nn, kk, qa_, qb_, shape, bias) in runs.items():
        for dt in ((torch.float32, torch.bfloat16) if mode != "wgrad" else (torch.float32,)):
            c = torch.empty(shape, dtype=dt, device="cuda")
            N.grouped_gemm_mx(mode, fmt, splits, mm, nn, kk, qa_, qb_, c, bias=bias)
            torch.cuda.synchronize()
            want = refs[name]
            if dt == torch.bfloat16:
                want = bf16_f64(codecs.f32_to_bf16_bits(codecs.f32(want).astype(np.float32)))
            for g in range(E):
                part = c[g] if mode == "wgrad" else c[g * T:(g + 1) * T]
                got = f32(part) if dt == torch.float32 else bf16_f64(bf16_host(part))
                err = rel_rms(got, want)
                key = name + ("" if dt == torch.float32 else " bf16")
                worst[key] = max(worst.get(key, 0.0), err)
                assert err <= TOL, (name, str(dt), g, err)
            del c
    print(fmt, {k: "%.2e" % v for k, v in worst.items()}, flush=True)

