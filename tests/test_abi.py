"""Host-side checks of the C ABI: the library loads, exports every declared symbol, and rejects bad
arguments before anything touches a GPU (validation runs on the host, so these run without one)."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    src = open(os.path.join(ROOT, "include", "mgs.h")).read()
    return sorted(set(re.findall(r"\b(mgs_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_four_entry_points():
    syms = _declared_symbols()
    for name in ("mgs_grouped_scaled_act_fwd", "mgs_grouped_scaled_act_bwd", "mgs_grouped_mx_quantize",
                 "mgs_grouped_gemm_mx"):
        assert name in syms


def test_library_exports_every_declared_symbol():
    from moe_grouped_scaled_amd import _native
    lib = ctypes.CDLL(_native.LIB_PATH)
    for name in _declared_symbols():
        assert hasattr(lib, name), name
    assert set(_native.EXPORTED) == set(_declared_symbols())
    assert _native.abi_version() == 8


def test_qtensor_nbytes_layouts():
    from moe_grouped_scaled_amd import _native as N
    from oracle.quant import qtensor_nbytes as oracle_nbytes
    for splits in ([64, 128, 32, 32], [0, 1, 31, 33, 64], [512] * 4):
        for fmt in ("mxfp8", "nvfp4"):
            for col in (False, True):
                d, s = oracle_nbytes(fmt, col, splits, 96)
                assert N.qtensor_nbytes(fmt, col, splits, 96, "data") == d
                assert N.qtensor_nbytes(fmt, col, splits, 96, "scales") == s
        assert N.qtensor_nbytes("nvfp4", False, splits, 96, "group_scale") == 4 * len(splits)
        assert N.qtensor_nbytes("mxfp8", False, splits, 96, "group_scale") == 0


def _expect(code, fn, *args, match=None, **kw):
    from moe_grouped_scaled_amd import _native as N
    with pytest.raises(N.MgsError) as ei:
        fn(*args, **kw)
    assert ei.value.code == code, str(ei.value)
    if match:
        assert re.search(match, str(ei.value)), str(ei.value)


FAKE = 0x1000  # never dereferenced: every call below fails validation before any launch


class _FakeQ:
    def __init__(self, gs=True):
        from moe_grouped_scaled_amd import _native as N
        self.q = N.QBuf(FAKE, FAKE, FAKE if gs else None)


def test_argument_validation_act_fwd():
    from moe_grouped_scaled_amd import _native as N
    act = N.act_params("srelu")
    q = _FakeQ().q
    f = N.grouped_scaled_act_fwd
    _expect(-2, f, act, "mxfp8", [32, -1], 64, FAKE, FAKE, out_row=q, stream=0, match="negative")
    _expect(-2, f, act, "mxfp8", [32], 48, FAKE, FAKE, out_row=q, stream=0, match="multiple of 32")
    _expect(-2, f, N.act_params("swiglu"), "mxfp8", [32], 96, FAKE, FAKE, out_row=q, stream=0)
    _expect(-1, f, act, "mxfp8", [32], 64, None, FAKE, out_row=q, stream=0, match="x_bf16")
    _expect(-1, f, act, "mxfp8", [32], 64, FAKE, FAKE, stream=0, match="no output")
    _expect(-1, f, act, "nvfp4", [32], 64, FAKE, FAKE, out_row=q, stream=0, match="group_amax")
    _expect(-1, f, act, "nvfp4", [32], 64, FAKE, FAKE, out_row=_FakeQ(gs=False).q, group_amax=FAKE,
            stream=0, match="group_scale")
    _expect(-1, f, N.act_params("tanh_srelu", s=0.0), "mxfp8", [32], 64, FAKE, FAKE, out_row=q, stream=0)
    _expect(-1, f, N.ActParams(9, 1, 1, 1, 0), "mxfp8", [32], 64, FAKE, FAKE, out_row=q, stream=0)
    _expect(-1, f, act, "mxfp8", [1] * 257, 64, FAKE, FAKE, out_row=q, stream=0, match="num_groups")


def test_argument_validation_act_bwd_and_recompute():
    from moe_grouped_scaled_amd import _native as N
    act = N.act_params("srelu")
    q = _FakeQ().q
    b = N.grouped_scaled_act_bwd
    _expect(-1, b, act, "mxfp8", [32], 64, FAKE, None, FAKE, dx=FAKE, stream=0, match="dy_bf16")
    _expect(-1, b, act, "mxfp8", [32], 64, FAKE, FAKE, FAKE, stream=0, match="no output")
    _expect(-3, b, act, "nvfp4", [32], 64, FAKE, FAKE, FAKE, act_col=q, stream=0, match="saved_group_amax")
    _expect(-1, b, act, "nvfp4", [32], 64, FAKE, FAKE, FAKE, dx_row=q, stream=0, match="dx_group_amax")
    import torch
    small = torch.empty(4 * 32 - 1, dtype=torch.uint8)  # host memory: validation fails before any use
    _expect(-1, b, act, "mxfp8", [32], 256, FAKE, FAKE, FAKE, dprobs=FAKE, workspace=small, stream=0,
            match="workspace")
    need = N.act_bwd_workspace_bytes(act, [32], 256)
    short = torch.empty(need - 1, dtype=torch.uint8)
    _expect(-1, b, act, "mxfp8", [32], 256, FAKE, FAKE, FAKE, dx_col_sum=FAKE, workspace=short, stream=0,
            match="dx_col_sum needs a workspace")


def test_noalloc_backward_validates_like_the_workspace_one_and_rejects_oversize():
    """The allocation-free backward runs the same host validation, and rejects a request whose
    workspace would exceed its static scratch before touching any device (no GPU needed here)."""
    from moe_grouped_scaled_amd import _native as N
    act = N.act_params("srelu")
    b = N.grouped_scaled_act_bwd_noalloc
    _expect(-1, b, act, "mxfp8", [32], 64, FAKE, None, FAKE, dx=FAKE, stream=0, match="dy_bf16")
    _expect(-1, b, act, "mxfp8", [32], 64, FAKE, FAKE, FAKE, stream=0, match="no output")
    _expect(-3, b, act, "nvfp4", [32], 64, FAKE, FAKE, FAKE, act_col=_FakeQ().q, stream=0,
            match="saved_group_amax")
    big = [4096] * 16                       # 65536 rows x 4096: 8 MiB dprobs + 8 MiB column partials
    need = N.act_bwd_workspace_bytes(act, big, 4096)
    assert need > N.NOALLOC_SCRATCH_BYTES
    _expect(-2, b, act, "mxfp8", big, 4096, FAKE, FAKE, FAKE, dprobs=FAKE, stream=0, match="static scratch")
    _expect(-2, b, act, "mxfp8", big, 4096, FAKE, FAKE, FAKE, dx_col_sum=FAKE, stream=0, match="static scratch")
    # the bench workload's request fits
    assert N.act_bwd_workspace_bytes(act, [2048] * 16, 4096) <= N.NOALLOC_SCRATCH_BYTES


def test_argument_validation_quantize_col_sum():
    from moe_grouped_scaled_amd import _native as N
    import torch
    q = _FakeQ().q
    f = N.grouped_mx_quantize
    _expect(-1, f, "mxfp8", [32], 64, FAKE, stream=0, match="no output")
    need = N.quantize_workspace_bytes([32, 200], 64)
    short = torch.empty(need - 1, dtype=torch.uint8)
    _expect(-1, f, "mxfp8", [32, 200], 64, FAKE, out_row=q, col_sum=FAKE, workspace=short, stream=0,
            match="col_sum needs a workspace")
    # NVFP4 needs the group amax only when something is quantized
    _expect(-1, f, "nvfp4", [32], 64, FAKE, out_row=q, stream=0, match="group_amax")
    _expect(-2, f, "mxfp8", [32], 48, FAKE, out_row=q, stream=0, match="multiple of 32")


def _padded_rows(splits):
    return sum(-(-m // 128) * 128 for m in splits)


def test_workspace_bytes():
    """Closed forms: dprobs partials (one FP32 per row and 128-column tile, rounded up to 256 bytes)
    followed by one FP32 column partial per 128-token block of the columnwise-padded rows, then (at
    the next 256-byte boundary) 2 E FP32 group maxima for a Hadamard-transformed recompute."""
    from moe_grouped_scaled_amd import _native as N
    for kind, w_in, wa in (("srelu", 4096, 4096), ("swiglu", 4096, 2048), ("identity", 96, 96)):
        for splits in ([64, 128, 32, 32], [0, 1, 31, 33, 64], [2048] * 16, [0, 0]):
            m = sum(splits)
            dp = -(-(4 * m * -(-wa // 128)) // 256) * 256
            cs = 4 * (_padded_rows(splits) // 128) * w_in
            rht = -(-(dp + cs) // 256) * 256 + 8 * len(splits)
            assert N.act_bwd_workspace_bytes(N.act_params(kind), splits, w_in) == rht
            assert N.quantize_workspace_bytes(splits, wa) == 4 * (_padded_rows(splits) // 128) * wa
    _expect(-2, N.act_bwd_workspace_bytes, N.act_params("swiglu"), [32], 96)
    _expect(-2, N.quantize_workspace_bytes, [32], 40)


def test_size_limits():
    """Quantizing calls reject a group whose padded columnwise matrix reaches 2^31 elements."""
    from moe_grouped_scaled_amd import _native as N
    q = _FakeQ().q
    act = N.act_params("srelu")
    _expect(-2, N.grouped_scaled_act_fwd, act, "mxfp8", [65536], 32768, FAKE, FAKE, out_row=q, stream=0,
            match="2\\^31")
    _expect(-2, N.grouped_scaled_act_bwd, act, "mxfp8", [1, 65536 - 127], 32768, FAKE, FAKE, FAKE, dx=FAKE,
            stream=0, match="2\\^31")


def test_argument_validation_gemm():
    from moe_grouped_scaled_amd import _native as N
    import torch
    q = _FakeQ().q
    c = torch.empty(1, dtype=torch.float32)
    g = N.grouped_gemm_mx
    _expect(-2, g, "fprop", "mxfp8", [32, 32], 63, 64, 64, q, q, c, stream=0, match="split sum")
    _expect(-2, g, "fprop", "mxfp8", [32, 32], 64, 64, 48, q, q, c, stream=0, match="multiple of 32")
    _expect(-2, g, "wgrad", "mxfp8", [32, 32], 64, 64, 63, q, q, c, stream=0, match="split sum")
    _expect(-1, g, "wgrad", "mxfp8", [32, 32], 64, 64, 64, q, q, c, bias=FAKE, stream=0, match="bias")
    cb = torch.empty(1, dtype=torch.bfloat16)
    _expect(-3, g, "fprop", "mxfp8", [32], 32, 64, 64, q, q, cb, accumulate=True, stream=0)
    _expect(-1, g, "fprop", "nvfp4", [32], 32, 64, 64, _FakeQ(gs=False).q, q, c, stream=0)


def test_argument_validation_fprop_act_and_f32_forward():
    from moe_grouped_scaled_amd import _native as N
    import torch
    q = _FakeQ().q
    cb = torch.empty(1, dtype=torch.bfloat16)
    g = N.grouped_gemm_mx_fprop_act
    srelu = N.act_params("srelu")
    _expect(-3, g, [32], 32, 64, 64, q, q, cb, N.act_params("swiglu"), None, q, stream=0, match="gated")
    _expect(-1, g, [32], 32, 64, 64, q, q, None, srelu, None, q, stream=0, match="c_bf16")
    _expect(-1, g, [32], 32, 64, 64, q, q, cb, srelu, None, None, stream=0, match="out_row")
    _expect(-2, g, [32, 32], 63, 64, 64, q, q, cb, srelu, None, q, stream=0, match="split sum")
    _expect(-2, g, [32], 32, 48, 64, q, q, cb, srelu, None, q, stream=0, match="multiple of 32")
    f = N.grouped_scaled_act_fwd_f32
    x = torch.empty(1, dtype=torch.float32)
    _expect(-1, f, srelu, "mxfp8", [32], 64, x, None, stream=0, match="no output")
    _expect(-1, f, srelu, "nvfp4", [32], 64, x, None, q, stream=0, match="group_amax")
    _expect(-2, f, srelu, "mxfp8", [32], 48, x, None, q, stream=0, match="multiple of 32")


def test_argument_validation_rht():
    """The Hadamard transform is for NVFP4 columnwise copies; bit 16 enables it."""
    from moe_grouped_scaled_amd import _native as N
    import torch
    act = N.act_params("srelu")
    x = torch.empty(1, dtype=torch.bfloat16)
    amax = torch.empty(2, dtype=torch.float32)
    col = N.QBuf(FAKE, FAKE, FAKE, N.RHT_ON | 0x1234)
    row = N.QBuf(FAKE, FAKE, FAKE, N.RHT_ON | 0x1234)
    bad = N.QBuf(FAKE, FAKE, FAKE, 0x1234)
    f = N.grouped_scaled_act_fwd
    _expect(-3, f, act, "nvfp4", [32], 64, x, None, out_row=row, group_amax=amax, stream=0, match="columnwise")
    _expect(-3, f, act, "mxfp8", [32], 64, x, None, out_col=col, stream=0, match="NVFP4")
    _expect(-1, f, act, "nvfp4", [32], 64, x, None, out_col=bad, group_amax=amax, stream=0, match="bit 16")
    q = N.grouped_mx_quantize
    _expect(-3, q, "nvfp4", [32], 64, x, out_row=row, group_amax=amax, stream=0, match="columnwise")
    b = N.grouped_scaled_act_bwd
    _expect(-1, b, act, "nvfp4", [32], 64, x, x, None, act_col=col, workspace=None, stream=0, match="workspace")


def test_last_error_is_cleared_on_success():
    from moe_grouped_scaled_amd import _native as N
    with pytest.raises(N.MgsError):
        N.qtensor_nbytes("mxfp8", False, [32], 33, "data")
    assert "multiple of 32" in N.last_error()
    N.qtensor_nbytes("mxfp8", False, [32], 32, "data")
    assert N.last_error() == ""


class _FakeTable:
    def data_ptr(self):
        return FAKE


def _fake_device_groups(e, cap):
    """A DeviceGroups whose device table is a never-dereferenced address (host validation only)."""
    from moe_grouped_scaled_amd import _native as N
    dg = N.DeviceGroups.__new__(N.DeviceGroups)
    dg.num_groups, dg.max_rows, dg.table = e, cap, _FakeTable()
    return dg


def test_device_resident_splits_validation_and_capacity_layouts():
    """With device-resident split sizes the layouts are those of the row capacity: rowwise copies
    hold max_rows rows, columnwise ones the padded bound 128 (ceil(max_rows / 128) + E) rows; the
    GEMMs take m (k for WGRAD) = max_rows; the calls validate their other arguments as with host
    split sizes; the offsets update needs device split sizes and a device table."""
    from moe_grouped_scaled_amd import _native as N
    assert N.LIB.mgs_groups_table_bytes() >= 2 * (2 * 65 + 4) * 4
    e, cap, w = 4, 300, 96
    dg = _fake_device_groups(e, cap)
    assert N.qtensor_nbytes("mxfp8", False, dg, w, "data") == cap * w
    assert N.qtensor_nbytes("mxfp8", True, dg, w, "data") == 128 * (-(-cap // 128) + e) * w
    assert N.qtensor_nbytes("mxfp8", False, dg, w, "scales") >= cap * w // 32
    assert N.act_bwd_workspace_bytes(N.act_params("srelu"), dg, w) >= \
        N.act_bwd_workspace_bytes(N.act_params("srelu"), [cap - 3 * 64 - 1, 64, 64, 64], w)
    q = _FakeQ().q
    act = N.act_params("srelu")
    assert N.qtensor_nbytes("nvfp4", True, dg, w, "data") == 128 * (-(-cap // 128) + e) * w // 2
    _expect(-1, N.grouped_scaled_act_fwd, act, "nvfp4", dg, w, FAKE, FAKE, out_row=q, stream=0,
            match="group_amax")
    _expect(-1, N.grouped_scaled_act_fwd_f32, act, "mxfp8", dg, w, FAKE, FAKE, stream=0, match="no output")
    _expect(-2, N.grouped_col_sum, dg, 12, FAKE, FAKE, stream=0, match="multiple of 8")
    _expect(-1, N.grouped_mx_quantize, "nvfp4", dg, w, FAKE, out_row=q, stream=0, match="group_amax")
    import torch
    c = torch.empty(1, dtype=torch.float32)
    _expect(-2, N.grouped_gemm_mx, "fprop", "mxfp8", dg, cap - 1, 64, 64, q, q, c, stream=0, match="split sum")
    _expect(-2, N.grouped_gemm_mx, "wgrad", "mxfp8", dg, 64, 64, cap + 1, q, q, c, stream=0, match="split sum")
    _expect(-2, N.qtensor_nbytes, "mxfp8", False, _fake_device_groups(e, 0), w, "data", match="max_rows")
    g = N._GroupsArg([1, 2, 3, 4])
    assert N.LIB.mgs_groups_update(g.ref, FAKE, None, None) == -1
    assert "host split sizes" in N.last_error()
    g = N._GroupsArg(dg)
    assert N.LIB.mgs_groups_update(g.ref, None, None, None) == -1
    assert "split_sizes_dev" in N.last_error()
    g.struct.dev_table = None
    assert N.LIB.mgs_groups_update(g.ref, FAKE, None, None) == -1


def test_expert_mlp_device_splits_need_capacity_rows():
    """ExpertMLP with device-resident split sizes takes inputs of the capacity's rows and says so
    before any launch."""
    import torch
    from moe_grouped_scaled_amd.expert_mlp import ExpertMLP
    e, h, f = 4, 64, 64
    w1, w2 = torch.zeros(e, f, h, dtype=torch.bfloat16), torch.zeros(e, h, f, dtype=torch.bfloat16)
    mlp = ExpertMLP("srelu", "mxfp8", w1, w2)
    dg = _fake_device_groups(e, 256)
    with pytest.raises(ValueError, match="capacity"):
        mlp.forward(torch.zeros(200, h, dtype=torch.bfloat16), torch.zeros(200), dg)
