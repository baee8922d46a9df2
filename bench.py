"""Benchmark of the fused MoE expert-MLP hot path on one MI355X.

One step = one pass of the whole path over one batch: FC1 input / weight quantization, the FC1
grouped GEMM (+ bias), the fused per-row scaled activation + MXFP8 quantize, FC2, then the backward
(upstream-gradient quantization, FC2 dgrad, the fused activation backward with dprobs and the
recompute of FC2's columnwise input, FC1 dgrad) and the delayed weight gradients (FC2 and FC1 wgrad,
both bias gradients).  Workload: 16 experts x 2048 tokens, hidden 4096, ffn 4096, ScaledSReLU, bias on,
recompute on, delayed wgrad, seeded synthetic inputs already resident in HBM.

Prints one JSON line.  `value` is the step's GEMM work over the whole step time (TFLOP/s); the line
also carries the per-kernel breakdown (fused act+quant GB/s forward and backward, grouped GEMM TFLOP/s),
the roofline of the dominant kernel (the grouped GEMM) and the oracle's CPU throughput on a bounded
sample of the same workload.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused act+MX-quant GB/s (% of HBM peak) fwd/bwd; grouped MX GEMM TFLOP/s"
HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = {"mxfp8": 5000.0, "nvfp4": 2500.0}   # FP8 dense; NVFP4 runs on the FP16 MFMA
# The bars this implementation is held to: the fused act + quantize kernels at >= 70 % of HBM peak,
# the grouped MX GEMM at >= 60 % of the dense MFMA peak.  Every fraction in the JSON line is reported
# next to its bar and the ratio to it ("of_target": 1.0 = bar met).
TARGET_FRAC_HBM = 0.70
TARGET_FRAC_MFMA = 0.60


def vs_target(frac, target):
    return {"target_frac": target, "of_target": frac / target}
FC1_ACT = {"auto": "auto", "epilogue": True, "separate": False}   # --fc1-act -> ExpertMLP(fuse_fc1_act=)


def act_fwd_bytes(m, w_in, w_a, fmt, row=True, col=False, col_rows=None):
    """Algorithmic bytes of one fused forward: x read once, p read once, each requested output
    written once (codes + scales)."""
    b = 2 * m * w_in + 4 * m
    per = (w_a + w_a // 32) if fmt == "mxfp8" else (w_a // 2 + w_a // 16)
    if row:
        b += m * per
    if col:
        b += (col_rows if col_rows is not None else m) * per
    return b


def act_bwd_bytes(m, w_in, w_a, fmt, dense=True, row=True, col=True, dprobs=True, recompute=True,
                  col_rows=None, col_sum_groups=0):
    """Algorithmic bytes of one fused backward: x, dy and p read once, each requested output written
    once; the bias gradient (per-group column sums, `col_sum_groups` experts) is E x w_in FP32."""
    cr = col_rows if col_rows is not None else m
    b = 2 * m * w_in + 2 * m * w_a + 4 * m
    per_in = (w_in + w_in // 32) if fmt == "mxfp8" else (w_in // 2 + w_in // 16)
    per_a = (w_a + w_a // 32) if fmt == "mxfp8" else (w_a // 2 + w_a // 16)
    if dense:
        b += 2 * m * w_in
    if row:
        b += m * per_in
    if col:
        b += cr * per_in
    if dprobs:
        b += 4 * m
    if recompute:
        b += cr * per_a
    b += 4 * col_sum_groups * w_in
    return b


class Timer:
    """Wraps the binding's entry points to record HIP events around every call on the stream the
    library launches on (torch's current stream).

    The events come from a pool created with the Timer, before the warm-up steps.  Creating timing
    events during the timed steps, or creating none at all, left one ~35 ms host stall in the timed
    region about 140 kernel dispatches after the synchronization that opens it: the GPU drained and
    idled, and its clocks took the next ~15 launches to recover (one launch measured 15-50 ms, the
    step 4.9-5.1 instead of 4.25 ms).  With the pool created first, no stall occurs."""

    POOL = 4000

    def __init__(self, N):
        import torch
        self.torch, self.N = torch, N
        self.records = []
        self.pool = [torch.cuda.Event(enable_timing=True) for _ in range(self.POOL)]
        self.enabled = False
        self._orig = {}
        for name in ("grouped_scaled_act_fwd", "grouped_scaled_act_fwd_f32", "grouped_scaled_act_bwd",
                     "grouped_mx_quantize", "grouped_gemm_mx", "grouped_gemm_mx_fprop_act"):
            self._wrap(name)

    def _wrap(self, name):
        orig = getattr(self.N, name)
        self._orig[name] = orig
        torch = self.torch

        def wrapped(*a, **kw):
            if not self.enabled:
                return orig(*a, **kw)
            if len(self.pool) >= 2:
                s, e = self.pool.pop(), self.pool.pop()
            else:
                s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            r = orig(*a, **kw)
            e.record()
            tag = "gemm_" + a[0] if name == "grouped_gemm_mx" else name
            self.records.append((tag, s, e))
            return r

        setattr(self.N, name, wrapped)

    def durations(self):
        out = {}
        for tag, s, e in self.records:
            out.setdefault(tag, []).append(s.elapsed_time(e) * 1e-3)
        return out


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_traffic.json")
GEMM_SOURCE = os.path.join(ROOT, "moe_grouped_scaled_amd", "csrc", "gemm_mx.hip")


def gemm_source_sha():
    with open(GEMM_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(fmt):
    """HBM bytes per GEMM launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE runs, scaled by
    the copy-kernel calibration; None when the counters were taken on a different GEMM source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != gemm_source_sha() or t.get("recipe") != fmt:
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(kind, fmt, seed=0):
    """The oracle's expert-MLP step on a bounded sample of the workload: one of the 16 experts with
    1536 tokens, full hidden 4096 / ffn 4096 weights (about 10 s on the host).  Returns the oracle's GEMM
    TFLOP/s."""
    from oracle import mlp as M
    import workloads
    from oracle.codecs import bf16_bits_to_f64
    rng = np.random.default_rng(seed)
    e, tok, h, f = 1, 1536, 4096, 4096
    splits = [tok] * e
    m = e * tok
    x1 = bf16_bits_to_f64(workloads.normal_bf16(rng, (m, h)))
    w1 = bf16_bits_to_f64(workloads.normal_bf16(rng, (e, f, h), 0.02))
    w2 = bf16_bits_to_f64(workloads.normal_bf16(rng, (e, h, f), 0.02))
    b1 = bf16_bits_to_f64(workloads.normal_bf16(rng, (e, f), 0.02))
    b2 = bf16_bits_to_f64(workloads.normal_bf16(rng, (e, h), 0.02))
    p = workloads.uniform_f32(rng, m).astype(np.float64)
    dy2 = bf16_bits_to_f64(workloads.normal_bf16(rng, (m, h)))
    t0 = time.perf_counter()
    M.mlp_step(kind, fmt, splits, x1, w1, b1, w2, b2, p, dy2)
    dt = time.perf_counter() - t0
    flops = 2 * m * (h * f + f * h) * 3
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # threadpoolctl missing: report the visible cores
        threads = os.cpu_count()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": "oracle expert-MLP step (numpy float64), 1 expert x %d tokens, hidden 4096, "
                      "ffn 4096, same recipe; %.1f s wall" % (tok, dt)}


def gemm_roofline_time(mode, splits, m_or_n, n, k, fmt, c_bytes):
    """T* = sum over groups of max(FLOP_g / P, bytes_g / 8 TB/s) for one grouped GEMM launch:
    operands read once (codes + scales) and the output written once.  FPROP / DGRAD (grouped over
    M): group g is an [m_g x k] . [n x k]^T product; WGRAD (grouped over K): [m x m_g] . [n x m_g]^T
    with an [m x n] output per group, written even for an empty group."""
    per_el = (1 + 1 / 32) if fmt == "mxfp8" else (0.5 + 1 / 16)
    peak = MFMA_PEAK_TFLOPS[fmt] * 1e12
    t = 0.0
    for mg in splits:
        if mode == "wgrad":
            flop = 2.0 * m_or_n * n * mg
            byts = (m_or_n + n) * mg * per_el + m_or_n * n * c_bytes
        else:
            flop = 2.0 * mg * n * k
            byts = (mg + n) * k * per_el + mg * n * c_bytes if mg else 0.0
        t += max(flop / peak, byts / (HBM_PEAK_GBPS * 1e9))
    return t


def bench_zipf(args):
    """The two Zipf-split workloads, each as its own JSON line:
      swiglu_zipf  scaled SwiGLU forward + backward, MXFP8 rowwise and columnwise: 8 experts, 8192
                   tokens in a Zipf(1.2) split with one empty expert, FC1 output 2 x 2048;
      clamped_fc2  clamped SwiGLU (limit 7) forward + backward with FC2's grouped MXFP8 GEMMs (fprop,
                   dgrad, wgrad): 32 experts, 65536 tokens in a Zipf(1.2) split with four empty
                   experts, ffn 2048 (x2 gated), hidden 7168; the FC2 weight and the upstream gradient
                   are quantized row + col in the step, recompute on (the backward regenerates FC2's
                   columnwise input).
    A step runs every launch of the workload once; the line reports each kernel's GB/s or TFLOP/s
    and, per GEMM mode, T*/t with T* the per-group roofline time."""
    import torch
    import workloads
    from moe_grouped_scaled_amd import _native as N

    d = workloads.make(args.workload)
    splits = list(map(int, d["splits"]))
    e, m = len(splits), int(sum(splits))
    w_in, w_a = 4096, 2048
    kind = "swiglu" if args.workload == "swiglu_zipf" else "clamped_swiglu"
    act = N.act_params(kind, limit=7.0)

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    x, p = dev(d["x"]), torch.from_numpy(d["p"]).cuda()
    dy = dev(d["dy"])
    fc2 = args.workload == "clamped_fc2"
    if fc2:
        hid = d["hidden"]
        w2, dy2 = dev(d["w2"].reshape(e * hid, w_a)), dev(d["dy2"])
    del d
    ws = torch.empty(N.act_bwd_workspace_bytes(act, splits, w_in), dtype=torch.uint8, device="cuda")

    def step():
        if not fc2:
            # forward with both copies (no GEMM consumes them here), backward with every output
            ar, ac = N.QTensor("mxfp8", False, splits, w_a), N.QTensor("mxfp8", True, splits, w_a)
            N.grouped_scaled_act_fwd(act, "mxfp8", splits, w_in, x, p, ar, ac)
            dxr, dxc = N.QTensor("mxfp8", False, splits, w_in), N.QTensor("mxfp8", True, splits, w_in)
            dx = torch.empty((m, w_in), dtype=torch.bfloat16, device="cuda")
            dp = torch.empty(m, dtype=torch.float32, device="cuda")
            N.grouped_scaled_act_bwd(act, "mxfp8", splits, w_in, x, dy, p, dx=dx, dx_row=dxr, dx_col=dxc,
                                     dprobs=dp, workspace=ws)
            return
        w2r, w2c = N.QTensor("mxfp8", False, [hid] * e, w_a), N.QTensor("mxfp8", True, [hid] * e, w_a)
        N.grouped_mx_quantize("mxfp8", [hid] * e, w_a, w2, w2r, w2c)
        ar = N.QTensor("mxfp8", False, splits, w_a)
        N.grouped_scaled_act_fwd(act, "mxfp8", splits, w_in, x, p, ar, None)
        y2 = torch.empty((m, hid), dtype=torch.bfloat16, device="cuda")
        N.grouped_gemm_mx("fprop", "mxfp8", splits, m, hid, w_a, ar, w2r, y2)
        del ar, y2
        g2r, g2c = N.QTensor("mxfp8", False, splits, hid), N.QTensor("mxfp8", True, splits, hid)
        N.grouped_mx_quantize("mxfp8", splits, hid, dy2, g2r, g2c)
        da = torch.empty((m, w_a), dtype=torch.bfloat16, device="cuda")
        N.grouped_gemm_mx("dgrad", "mxfp8", splits, m, w_a, hid, g2r, w2c, da)
        dxr, dxc = N.QTensor("mxfp8", False, splits, w_in), N.QTensor("mxfp8", True, splits, w_in)
        ac = N.QTensor("mxfp8", True, splits, w_a)
        dp = torch.empty(m, dtype=torch.float32, device="cuda")
        N.grouped_scaled_act_bwd(act, "mxfp8", splits, w_in, x, da, p, dx_row=dxr, dx_col=dxc, dprobs=dp,
                                 act_col=ac, workspace=ws)
        dw2 = torch.empty((e, hid, w_a), dtype=torch.float32, device="cuda")
        N.grouped_gemm_mx("wgrad", "mxfp8", splits, hid, w_a, m, g2c, ac, dw2)

    timer = Timer(N)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timer.enabled = True
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timer.enabled = False
    dur = {k: float(np.mean(v)) for k, v in timer.durations().items()}
    if not fc2:
        fwd_b = act_fwd_bytes(m, w_in, w_a, "mxfp8", row=True, col=True)
        bwd_b = act_bwd_bytes(m, w_in, w_a, "mxfp8", dense=True, row=True, col=True, dprobs=True,
                              recompute=False)
    else:
        fwd_b = act_fwd_bytes(m, w_in, w_a, "mxfp8", row=True, col=False)
        bwd_b = act_bwd_bytes(m, w_in, w_a, "mxfp8", dense=False, row=True, col=True, dprobs=True,
                              recompute=True)
    t_fwd, t_bwd = dur["grouped_scaled_act_fwd"], dur["grouped_scaled_act_bwd"]
    kernels = {
        "act_fwd": {"GB/s": fwd_b / t_fwd / 1e9, "frac_hbm": fwd_b / t_fwd / 1e9 / HBM_PEAK_GBPS,
                    **vs_target(fwd_b / t_fwd / 1e9 / HBM_PEAK_GBPS, TARGET_FRAC_HBM),
                    "us": t_fwd * 1e6, "bytes": fwd_b},
        "act_bwd": {"GB/s": bwd_b / t_bwd / 1e9, "frac_hbm": bwd_b / t_bwd / 1e9 / HBM_PEAK_GBPS,
                    **vs_target(bwd_b / t_bwd / 1e9 / HBM_PEAK_GBPS, TARGET_FRAC_HBM),
                    "us": t_bwd * 1e6, "bytes": bwd_b},
    }
    ms = wall / args.steps * 1e3
    if not fc2:
        tot_b = fwd_b + bwd_b
        value, unit = tot_b / (t_fwd + t_bwd) / 1e9, "GB/s"
        roof = {"bound": "hbm", "achieved": bwd_b / t_bwd / 1e9, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": bwd_b / t_bwd / 1e9 / HBM_PEAK_GBPS, "traffic": None}
        wl = ("scaled SwiGLU fwd + bwd, MXFP8 row + col: 8 experts, 8192 tokens Zipf(1.2) split "
              "(one empty), FC1 out 2 x 2048")
    else:
        flops = 2.0 * m * hid * w_a
        gemm = {}
        for mode, (mm, nn, kk, cb) in {"fprop": (m, hid, w_a, 2), "dgrad": (m, w_a, hid, 2),
                                       "wgrad": (hid, w_a, m, 4)}.items():
            t = dur["gemm_" + mode]
            tstar = gemm_roofline_time(mode, splits, mm, nn, kk, "mxfp8", cb)
            gemm[mode] = {"us": t * 1e6, "TFLOP/s": flops / t / 1e12,
                          "frac_mfma": flops / t / 1e12 / MFMA_PEAK_TFLOPS["mxfp8"],
                          **vs_target(flops / t / 1e12 / MFMA_PEAK_TFLOPS["mxfp8"], TARGET_FRAC_MFMA),
                          "t_star_us": tstar * 1e6, "t_star_over_t": tstar / t}
        kernels["gemm"] = gemm
        kernels["mx_quantize_us"] = dur["grouped_mx_quantize"] * 1e6   # W2 and dY2, row + col, averaged
        t_g = float(np.mean([dur["gemm_" + k] for k in ("fprop", "dgrad", "wgrad")]))
        value, unit = 3 * flops / (ms * 1e-3) / 1e12, "TFLOP/s"
        roof = {"bound": "mfma", "achieved": flops / t_g / 1e12, "peak": MFMA_PEAK_TFLOPS["mxfp8"],
                "unit": "TFLOP/s", "frac": flops / t_g / 1e12 / MFMA_PEAK_TFLOPS["mxfp8"], "traffic": None}
        wl = ("clamped SwiGLU (limit 7) fwd + bwd + FC2 grouped MXFP8 fprop/dgrad/wgrad: 32 experts, 65536 "
              "tokens Zipf(1.2) split (four empty), ffn 2048 (x2 gated), hidden 7168, recompute on")
    line = {"metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "fp8", "data": "synthetic",
            "config": {"workload": wl, "experts": e, "tokens": m, "splits": splits},
            "roofline": roof, "kernels": kernels}
    print(json.dumps(line))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", default="mlp_step", choices=["mlp_step", "swiglu_zipf", "clamped_fc2"],
                    help="mlp_step (default): the full expert-MLP training step; swiglu_zipf / clamped_fc2: the "
                         "Zipf-split SwiGLU and clamped-SwiGLU + FC2 workloads, one line each")
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--fmt", default="mxfp8", choices=["mxfp8", "nvfp4"])
    ap.add_argument("--act", default="srelu", choices=["srelu", "tanh_srelu", "gelu", "sigmoid"])
    ap.add_argument("--fc1-fp32-act", action="store_true",
                    help="activate FC1's FP32 output in the forward (the recompute then regenerates FC2's "
                         "input from its BF16 copy)")
    ap.add_argument("--fc1-act", default="auto", choices=["auto", "epilogue", "separate"],
                    help="run the forward activation + quantization in FC1's GEMM epilogue (MXFP8, unary "
                         "activations) or as its own fused pass; auto: the epilogue where it is faster "
                         "(SReLU, sigmoid)")
    ap.add_argument("--rht", type=lambda v: int(v, 0), default=None,
                    help="NVFP4: Hadamard-transform the weight-gradient operands with this 16-bit sign mask")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured once in a HIP graph with device-resident split "
                         "sizes and replayed (the uniform routing, then alternating it with a Zipf(1.2) "
                         "routing of the same tokens); reported under \"graph_replay\"")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one plain 1 GiB device copy (counter calibration under rocprofv3)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (expert-parallel "
              "sharding is a design note); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    from moe_grouped_scaled_amd import _native as N
    from moe_grouped_scaled_amd.expert_mlp import ExpertMLP, gemm_flops

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.workload != "mlp_step":
        bench_zipf(args)
        return
    d = workloads.make("mlp_step", seed=0, act=args.act)
    splits = list(map(int, d["splits"]))
    e, h, f = 16, d["hidden"], d["ffn"]
    m = int(sum(splits))

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    x1, w1, w2, b1, b2, dy2 = (dev(d[k]) for k in ("x1", "w1", "w2", "b1", "b2", "dy2"))
    p = torch.from_numpy(d["p"]).cuda()
    del d
    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # recompute memory drop, measured between forward and backward
    held = {}
    for rc in (False, True):
        mlp = ExpertMLP(args.act, args.fmt, w1, w2, b1, b2, recompute=rc, delay_wgrad=True, s=2.0,
                        fc1_fp32_act=args.fc1_fp32_act, fuse_fc1_act=FC1_ACT[args.fc1_act],
                        rht_signs=args.rht)
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        y = mlp.forward(x1, p, splits)
        torch.cuda.synchronize()
        held[rc] = torch.cuda.memory_allocated() - base
        mlp.backward(dy2)
        mlp.backward_dw()
        del y, mlp
    col_rows = m  # every expert's token count is a multiple of 32
    drop_closed = col_rows * f + col_rows * f // 32 if args.fmt == "mxfp8" else col_rows * f // 2 + col_rows * f // 16

    mlp = ExpertMLP(args.act, args.fmt, w1, w2, b1, b2, recompute=True, delay_wgrad=True, s=2.0,
                    fc1_fp32_act=args.fc1_fp32_act, fuse_fc1_act=FC1_ACT[args.fc1_act],
                    rht_signs=args.rht)

    def step():
        mlp.forward(x1, p, splits)
        mlp.backward(dy2)
        mlp.backward_dw()

    timer = Timer(N)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timer.enabled = True
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timer.enabled = False
    fused_fc1 = mlp.fused_fc1_calls > 0
    if fused_fc1:
        # the step ran the forward activation inside FC1's epilogue; time the separate fused pass on
        # the same FC1 output on its own, for its GB/s (not part of the step time)
        y1 = torch.empty((m, f), dtype=torch.bfloat16, device="cuda")
        qx, qw = N.QTensor(args.fmt, False, splits, h), N.QTensor(args.fmt, False, [f] * e, h)
        N.grouped_mx_quantize(args.fmt, splits, h, x1, qx)
        N.grouped_mx_quantize(args.fmt, [f] * e, h, w1.view(e * f, h), qw)
        ya = N.QTensor(args.fmt, False, splits, f)
        if args.fc1_fp32_act:
            y1f = torch.empty((m, f), dtype=torch.float32, device="cuda")
            N.grouped_gemm_mx("fprop", args.fmt, splits, m, f, h, qx, qw, y1f, bias=b1)
            run_fwd = lambda: N.grouped_scaled_act_fwd_f32(mlp.act, args.fmt, splits, f, y1f, p, ya, x_bf16_out=y1)
        else:
            N.grouped_gemm_mx("fprop", args.fmt, splits, m, f, h, qx, qw, y1, bias=b1)
            run_fwd = lambda: N.grouped_scaled_act_fwd(mlp.act, args.fmt, splits, f, y1, p, ya)
        run_fwd()
        torch.cuda.synchronize()
        timer.enabled = True
        for _ in range(args.steps):
            run_fwd()
        torch.cuda.synchronize()
        timer.enabled = False
    dur = timer.durations()

    ms_per_step = wall / args.steps * 1e3
    flops_step = gemm_flops(m, h, f, f)
    value = flops_step / (wall / args.steps) / 1e12

    gemm_t = []
    for tag in ("gemm_fprop", "gemm_dgrad", "gemm_wgrad", "grouped_gemm_mx_fprop_act"):
        gemm_t += dur.get(tag, [])    # the six GEMM launches of each step (FC1's may carry the activation)
    flops_launch = 2 * m * h * f          # every one of the six GEMMs has this size here
    gemm_avg = float(np.mean(gemm_t))
    gemm_tflops = flops_launch / gemm_avg / 1e12
    peak = MFMA_PEAK_TFLOPS[args.fmt]
    fwd_b = act_fwd_bytes(m, f, f, args.fmt, row=True, col=False)
    fwd_name = "grouped_scaled_act_fwd"
    if args.fc1_fp32_act:
        # FP32 input instead of BF16, plus the BF16 copy the backward keeps
        fwd_b += 2 * m * f + 2 * m * f
        fwd_name = "grouped_scaled_act_fwd_f32"
    # the step asks the backward for quantized dY1 (row + col), dprobs, the recomputed FC2 input and
    # FC1's bias gradient; the dense BF16 dY1 is not written
    bwd_b = act_bwd_bytes(m, f, f, args.fmt, dense=False, row=True, col=True, dprobs=True, recompute=True,
                          col_sum_groups=e)
    t_fwd = float(np.mean(dur[fwd_name]))
    t_bwd = float(np.mean(dur["grouped_scaled_act_bwd"]))
    kernels = {
        "act_fwd": {"GB/s": fwd_b / t_fwd / 1e9, "frac_hbm": fwd_b / t_fwd / 1e9 / HBM_PEAK_GBPS,
                    **vs_target(fwd_b / t_fwd / 1e9 / HBM_PEAK_GBPS, TARGET_FRAC_HBM),
                    "us": t_fwd * 1e6, "bytes": fwd_b,
                    "in_step": "no: FC1's epilogue ran it; timed alone on the same data" if fused_fc1 else "yes"},
        "act_bwd": {"GB/s": bwd_b / t_bwd / 1e9, "frac_hbm": bwd_b / t_bwd / 1e9 / HBM_PEAK_GBPS,
                    **vs_target(bwd_b / t_bwd / 1e9 / HBM_PEAK_GBPS, TARGET_FRAC_HBM),
                    "us": t_bwd * 1e6, "bytes": bwd_b},
        "gemm": {"TFLOP/s": gemm_tflops, "frac_mfma": gemm_tflops / peak,
                 **vs_target(gemm_tflops / peak, TARGET_FRAC_MFMA), "us_avg": gemm_avg * 1e6,
                 "flops_per_launch": flops_launch,
                 "us_by_mode": {t: float(np.mean(dur[t])) * 1e6 for t in ("gemm_fprop", "gemm_dgrad", "gemm_wgrad") if t in dur}},
        # four plain quantize launches per step: X1, W1, W2 and dY2 (the last also takes FC2's bias
        # gradient in the same pass)
        "mx_quantize_us": float(np.mean(dur["grouped_mx_quantize"])) * 1e6,
    }
    if fused_fc1:
        kernels["gemm_fprop_act_us"] = float(np.mean(dur["grouped_gemm_mx_fprop_act"])) * 1e6
    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8" if args.fmt == "mxfp8" else "fp4", "data": "synthetic",
        "config": {"workload": "expert-MLP train step: 16 experts x 2048 tokens, hidden 4096, ffn 4096, "
                               "%s, %s, bias, recompute on, delayed wgrad%s%s" % (
                                   args.act, args.fmt.upper(), ", FP32 FC1 output activated" if args.fc1_fp32_act else "",
                                   ", activation in FC1's epilogue" if fused_fc1 else ""),
                   "experts": e, "tokens": m, "hidden": h, "ffn": f, "recipe": args.fmt, "act": args.act,
                   "act_input": "fp32" if args.fc1_fp32_act else "bf16",
                   "rht": None if args.rht is None else hex(args.rht),
                   "fc1_act": "epilogue" if fused_fc1 else "separate"},
        "roofline": {"bound": "mfma", "achieved": gemm_tflops, "peak": peak, "unit": "TFLOP/s",
                     "frac": gemm_tflops / peak, "traffic": measured_traffic(args.fmt)},
        "kernels": kernels,
        "recompute_memory_drop_bytes": {"measured": held[False] - held[True], "closed_form": drop_closed},
    }
    if args.graph:
        line["graph_replay"] = graph_replay(args, N, ExpertMLP, (x1, w1, w2, b1, b2, dy2, p), splits, ms_per_step)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.act, args.fmt)
    print(json.dumps(line))


def graph_replay(args, N, ExpertMLP, tensors, splits, eager_ms):
    """The step captured once in a HIP graph with device-resident split sizes (capacity = the tokens of
    the step), then replayed: `steps` replays of the uniform routing, and `steps` replays alternating
    it with a Zipf(1.2) routing of the same tokens (the split tensor is rewritten between replays)."""
    import torch
    import workloads
    x1, w1, w2, b1, b2, dy2, p = tensors
    e, m = len(splits), int(sum(splits))
    zipf = list(map(int, workloads.zipf_split(np.random.default_rng(7), m, e, 1.2, 0)))
    dg = N.DeviceGroups(e, m)
    mlp = ExpertMLP(args.act, args.fmt, w1, w2, b1, b2, recompute=True, delay_wgrad=True, s=2.0,
                    fc1_fp32_act=args.fc1_fp32_act, fuse_fc1_act=FC1_ACT[args.fc1_act], rht_signs=args.rht)
    uniform = torch.tensor(splits, dtype=torch.int64, device="cuda")
    skewed = torch.tensor(zipf, dtype=torch.int64, device="cuda")

    def step():
        mlp.forward(x1, p, dg)
        mlp.backward(dy2)
        mlp.backward_dw()

    dg.splits.copy_(uniform)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(max(args.warmup, 2)):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    out = {"capacity_rows": m, "zipf_splits": zipf}
    for name, seq in (("uniform", [uniform] * args.steps), ("alternating", [uniform, skewed] * (args.steps // 2))):
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for sp in seq:
            dg.splits.copy_(sp)
            graph.replay()
        torch.cuda.synchronize()
        out["ms_per_step_" + name] = (time.perf_counter() - t0) / len(seq) * 1e3
    assert int(dg.status.item()) == 0
    out["eager_ms_per_step"] = eager_ms
    return out


if __name__ == "__main__":
    main()
