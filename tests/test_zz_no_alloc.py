"""The allocation-free backward (mgs_grouped_scaled_act_bwd_noalloc) against the backward with a caller
workspace: same kernels, so every output must be bit-identical, over consecutive calls that share
the static scratch (the second smaller than the first, then an NVFP4 call whose transformed recompute
keeps its group maxima in the scratch).

Page "Activation + GroupedLinear Fusion for MOE", sequence diagram (the backward activation call and
its three outputs); page "[PyTorch] Enable fused activation recompute for ScaledTanhSReLU",
Description (the recompute output of the backward).
"""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

RHT_MASK = 0x6B35


@pytest.fixture(scope="module")
def N():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from moe_grouped_scaled_amd import _native
    return _native


def _inputs(kind, splits, width_in, seed):
    import torch
    gen = torch.Generator(device="cuda").manual_seed(seed)
    m = int(sum(splits))
    wa = width_in // 2 if kind in ("swiglu", "clamped_swiglu", "glu") else width_in
    x = torch.randn(m, width_in, generator=gen, device="cuda").to(torch.bfloat16)
    dy = torch.randn(m, wa, generator=gen, device="cuda").to(torch.bfloat16)
    p = torch.rand(m, generator=gen, device="cuda")
    return x, dy, p, wa


def _outputs(N, fmt, splits, width_in, wa, rht=None):
    import torch
    m, e = int(sum(splits)), len(splits)
    o = dict(dx=torch.empty(m, width_in, dtype=torch.bfloat16, device="cuda"),
             dx_row=N.QTensor(fmt, False, splits, width_in),
             dx_col=N.QTensor(fmt, True, splits, width_in, rht=rht),
             dprobs=torch.empty(m, dtype=torch.float32, device="cuda"),
             dx_col_sum=torch.empty(e, width_in, dtype=torch.float32, device="cuda"),
             act_col=N.QTensor(fmt, True, splits, wa, rht=rht))
    if fmt == "nvfp4":
        o["dx_group_amax"] = torch.empty(2 * e, dtype=torch.float32, device="cuda")
    # garbage in every output so that an unwritten element cannot pass for a written one
    for v in o.values():
        for t in ([v] if isinstance(v, torch.Tensor) else [v.data, v.scales, v.group_scale]):
            if t is not None and t.numel():
                t.view(torch.uint8).fill_(0xA5)
    return o


def _host(o):
    import torch
    out = {}
    for k, v in o.items():
        ts = {"": v} if isinstance(v, torch.Tensor) else {".data": v.data, ".scales": v.scales,
                                                          ".group_scale": v.group_scale}
        for suf, t in ts.items():
            if t is not None:
                out[k + suf] = t.detach().view(torch.uint8).cpu().numpy() if t.numel() else np.zeros(0, np.uint8)
    return out


def _run_pair(N, kind, fmt, splits, width_in, seed, rht=None, saved_amax=None):
    """(workspace entry outputs, no-alloc entry outputs) on the same inputs."""
    import torch
    x, dy, p, wa = _inputs(kind, splits, width_in, seed)
    act = N.act_params(kind)
    saved = None
    if fmt == "nvfp4" and rht is None:
        # the forward's group amax, which an untransformed NVFP4 recompute needs
        fr = N.QTensor(fmt, False, splits, wa)
        saved = torch.empty(len(splits), dtype=torch.float32, device="cuda")
        N.grouped_scaled_act_fwd(act, fmt, splits, width_in, x, p, fr, None, saved)
    res = []
    for noalloc in (False, True):
        o = _outputs(N, fmt, splits, width_in, wa, rht=rht)
        kw = dict(dx=o["dx"], dx_row=o["dx_row"], dx_col=o["dx_col"], dx_group_amax=o.get("dx_group_amax"),
                  dprobs=o["dprobs"], dx_col_sum=o["dx_col_sum"], act_col=o["act_col"], saved_group_amax=saved)
        if noalloc:
            N.grouped_scaled_act_bwd_noalloc(act, fmt, splits, width_in, x, dy, p, **kw)
        else:
            ws = torch.empty(N.act_bwd_workspace_bytes(act, splits, width_in), dtype=torch.uint8, device="cuda")
            ws.fill_(0x5A)
            N.grouped_scaled_act_bwd(act, fmt, splits, width_in, x, dy, p, workspace=ws, **kw)
        torch.cuda.synchronize()
        res.append(_host(o))
    return res


def test_noalloc_backward_equals_workspace_backward_on_consecutive_calls(N):
    print("case: srelu mxfp8 16 x 2048 x 4096, then swiglu mxfp8 [300, 0, 212] x 2048, then srelu nvfp4 "
          "[37, 0, 256, 95] x 512 with the Hadamard transform", flush=True)
    cases = [
        ("srelu", "mxfp8", [2048] * 16, 4096, 1, None),       # the bench step's backward (8 MiB scratch)
        ("swiglu", "mxfp8", [300, 0, 212], 2048, 2, None),     # smaller, after the larger one
        ("srelu", "nvfp4", [37, 0, 256, 95], 512, 3, RHT_MASK),  # group maxima in the scratch
        ("tanh_srelu", "nvfp4", [64, 64], 512, 4, None),
    ]
    for kind, fmt, splits, w, seed, rht in cases:
        ref, got = _run_pair(N, kind, fmt, splits, w, seed, rht=rht)
        assert set(ref) == set(got)
        for k in ref:
            assert np.array_equal(ref[k], got[k]), (kind, fmt, splits, k)


def test_noalloc_backward_rejects_oversize_request(N):
    """A request whose workspace exceeds the static scratch is refused before anything is enqueued."""
    import torch
    splits = [4096] * 16
    act = N.act_params("srelu")
    assert N.act_bwd_workspace_bytes(act, splits, 4096) > N.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(1, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(N.MgsError) as ei:
        N.grouped_scaled_act_bwd_noalloc(act, "mxfp8", splits, 4096, x, x, None,
                                         dprobs=torch.zeros(1, device="cuda"))
    assert ei.value.code == -2 and "static scratch" in str(ei.value)
