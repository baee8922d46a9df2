"""ctypes binding of the C ABI in include/mgs.h (libmgs.so, built in-tree for gfx950).

Argument marshalling only: every step of the path runs in the library's HIP kernels.  Tensors are
torch tensors on the GPU (PyTorch provides device memory and streams); they are passed as raw device
pointers together with the current HIP stream.  There is no fallback: if the library is missing or
does not load, importing this module raises.
"""

import ctypes
import os

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmgs.so")

MGS_OK = 0
ERRORS = {-1: "MGS_ERR_INVALID_ARG", -2: "MGS_ERR_SHAPE", -3: "MGS_ERR_UNSUPPORTED", -4: "MGS_ERR_HIP"}

ACT = {"identity": 0, "srelu": 1, "tanh_srelu": 2, "swiglu": 3, "clamped_swiglu": 4, "gelu": 5, "sigmoid": 6,
       "glu": 7}
FMT = {"mxfp8": 0, "nvfp4": 1}
GEMM_MODE = {"fprop": 0, "dgrad": 1, "wgrad": 2}
DTYPE = {torch.bfloat16: 0, torch.float32: 1}
NBYTES = {"data": 0, "scales": 1, "group_scale": 2}
MAX_GROUPS = 256


class MgsError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("%s (%d): %s" % (ERRORS.get(code, "?"), code, msg))
        self.code = code


class ActParams(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("s", ctypes.c_float), ("limit", ctypes.c_float),
                ("alpha", ctypes.c_float), ("beta", ctypes.c_float)]


class Groups(ctypes.Structure):
    _fields_ = [("num_groups", ctypes.c_int32), ("split_sizes", ctypes.POINTER(ctypes.c_int64)),
                ("max_rows", ctypes.c_int64), ("dev_table", ctypes.c_void_p)]


class QBuf(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("group_scale", ctypes.c_void_p), ("rht", ctypes.c_uint32)]


RHT_ON = 1 << 16  # mgs_qbuf.rht: bit 16 enables the Hadamard transform, bits 0..15 are its signs


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libmgs.so not found at %s: build it with __graft_entry__.build() "
                          "(hipcc, gfx950)" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    pact, pgr, pq = ctypes.POINTER(ActParams), ctypes.POINTER(Groups), ctypes.POINTER(QBuf)
    sig = {
        "mgs_abi_version": (ctypes.c_int, []),
        "mgs_groups_table_bytes": (i64, []),
        "mgs_groups_update": (ctypes.c_int, [pgr, vp, vp, vp]),
        "mgs_last_error": (ctypes.c_char_p, []),
        "mgs_qtensor_nbytes": (i64, [i32, i32, pgr, i64, i32]),
        "mgs_grouped_scaled_act_fwd": (ctypes.c_int, [pact, i32, pgr, i64, vp, vp, pq, pq, vp, vp]),
        "mgs_grouped_scaled_act_fwd_f32": (ctypes.c_int, [pact, i32, pgr, i64, vp, vp, pq, pq, vp, vp, vp]),
        "mgs_grouped_scaled_act_bwd": (ctypes.c_int, [pact, i32, pgr, i64, vp, vp, vp, vp, pq, pq, vp,
                                                      vp, vp, pq, vp, vp, i64, vp]),
        "mgs_grouped_scaled_act_bwd_noalloc": (ctypes.c_int, [pact, i32, pgr, i64, vp, vp, vp, vp, pq, pq,
                                                              vp, vp, vp, pq, vp, vp]),
        "mgs_act_bwd_workspace_bytes": (i64, [pact, pgr, i64]),
        "mgs_grouped_mx_quantize": (ctypes.c_int, [i32, pgr, i64, vp, pq, pq, vp, vp, vp, i64, vp]),
        "mgs_grouped_mx_quantize_workspace_bytes": (i64, [pgr, i64]),
        "mgs_grouped_gemm_mx": (ctypes.c_int, [i32, i32, pgr, i64, i64, i64, pq, pq, vp, i32, vp, i32,
                                               vp]),
        "mgs_grouped_gemm_mx_fprop_act": (ctypes.c_int, [pgr, i64, i64, i64, pq, pq, vp, vp, pact, vp, i32,
                                                         pq, vp]),
        "mgs_grouped_col_sum": (ctypes.c_int, [pgr, i64, vp, vp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = _load()
EXPORTED = ("mgs_abi_version", "mgs_last_error", "mgs_groups_table_bytes", "mgs_groups_update",
            "mgs_qtensor_nbytes", "mgs_grouped_scaled_act_fwd",
            "mgs_grouped_scaled_act_fwd_f32",
            "mgs_grouped_scaled_act_bwd", "mgs_grouped_scaled_act_bwd_noalloc", "mgs_act_bwd_workspace_bytes", "mgs_grouped_mx_quantize",
            "mgs_grouped_mx_quantize_workspace_bytes", "mgs_grouped_gemm_mx", "mgs_grouped_gemm_mx_fprop_act",
            "mgs_grouped_col_sum")


def _check(rc):
    if rc != MGS_OK:
        raise MgsError(rc, LIB.mgs_last_error().decode())
    return rc


def last_error():
    return LIB.mgs_last_error().decode()


def abi_version():
    return LIB.mgs_abi_version()


class DeviceGroups:
    """Device-resident split sizes (graph-safe calls).  `splits` is a device int64 tensor the
    caller fills (copy_ works under graph replay); update() enqueues the offsets computation on the
    stream, and every call given this object afterwards reads them.  Layouts are strided for the row
    capacity `max_rows`; `status` (device int32) turns 1 when the splits are invalid (negative, or
    their sum above the capacity), in which case the calls write no rows."""

    def __init__(self, num_groups, max_rows, device="cuda"):
        self.num_groups, self.max_rows = int(num_groups), int(max_rows)
        self.splits = torch.zeros(self.num_groups, dtype=torch.int64, device=device)
        self.table = torch.empty(int(LIB.mgs_groups_table_bytes()), dtype=torch.uint8, device=device)
        self.status = torch.zeros(1, dtype=torch.int32, device=device)

    def __len__(self):
        return self.num_groups

    def update(self, stream=None):
        g = _GroupsArg(self)
        _check(LIB.mgs_groups_update(g.ref, self.splits.data_ptr(), self.status.data_ptr(), _stream(stream)))


class _GroupsArg:
    """Keeps the int64 split array alive for the duration of a call."""

    def __init__(self, split_sizes):
        if isinstance(split_sizes, DeviceGroups):
            self.arr = None
            self.struct = Groups(split_sizes.num_groups, None, split_sizes.max_rows, split_sizes.table.data_ptr())
            return
        self.arr = np.ascontiguousarray(np.asarray(split_sizes, dtype=np.int64))
        self.struct = Groups(len(self.arr), self.arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), 0, None)

    @property
    def ref(self):
        return ctypes.byref(self.struct)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    """HIP stream handle: an int passes through (0 = null stream), None = torch's current stream."""
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def act_params(kind, s=2.0, limit=7.0, alpha=1.0, beta=0.0):
    return ActParams(ACT[kind], s, limit, alpha, beta)


class QTensor:
    """One orientation (rowwise or columnwise) of a grouped quantized tensor: three torch buffers."""

    def __init__(self, fmt, colwise, split_sizes, width, device="cuda", rht=None):
        """`rht` (NVFP4 columnwise only): 16-bit sign mask of the Hadamard transform of the copy."""
        self.fmt, self.colwise, self.width = fmt, bool(colwise), int(width)
        self.rht = 0 if rht is None else RHT_ON | (int(rht) & 0xFFFF)
        nd = qtensor_nbytes(fmt, colwise, split_sizes, width, "data")
        ns = qtensor_nbytes(fmt, colwise, split_sizes, width, "scales")
        ng = qtensor_nbytes(fmt, colwise, split_sizes, width, "group_scale")
        self.data = torch.empty(max(nd, 1), dtype=torch.uint8, device=device)[:nd]
        self.scales = torch.empty(max(ns, 1), dtype=torch.uint8, device=device)[:ns]
        self.group_scale = torch.empty(ng // 4, dtype=torch.float32, device=device) if ng else None

    def qbuf(self):
        return QBuf(self.data.data_ptr(), self.scales.data_ptr(), _ptr(self.group_scale), self.rht)

    def nbytes(self):
        return self.data.numel() + self.scales.numel() + (self.group_scale.numel() * 4 if self.group_scale is not None else 0)


def _qref(q):
    if q is None:
        return None, None
    qb = q.qbuf() if isinstance(q, QTensor) else q
    return qb, ctypes.byref(qb)


def qtensor_nbytes(fmt, colwise, split_sizes, width, which):
    g = _GroupsArg(split_sizes)
    n = LIB.mgs_qtensor_nbytes(FMT[fmt], int(bool(colwise)), g.ref, int(width), NBYTES[which])
    if n < 0:
        _check(int(n))
    return int(n)


def grouped_scaled_act_fwd(act, fmt, split_sizes, width_in, x, probs, out_row=None, out_col=None,
                           group_amax=None, stream=None):
    g = _GroupsArg(split_sizes)
    _r, rref = _qref(out_row)
    _c, cref = _qref(out_col)
    _check(LIB.mgs_grouped_scaled_act_fwd(ctypes.byref(act), FMT[fmt], g.ref, int(width_in), _ptr(x),
                                          _ptr(probs), rref, cref, _ptr(group_amax), _stream(stream)))


def grouped_scaled_act_fwd_f32(act, fmt, split_sizes, width_in, x, probs, out_row=None, out_col=None,
                               group_amax=None, x_bf16_out=None, stream=None):
    """Forward from an FP32 input `x`; `x_bf16_out` (nullable) receives its BF16 rounding."""
    g = _GroupsArg(split_sizes)
    _r, rref = _qref(out_row)
    _c, cref = _qref(out_col)
    _check(LIB.mgs_grouped_scaled_act_fwd_f32(ctypes.byref(act), FMT[fmt], g.ref, int(width_in), _ptr(x),
                                              _ptr(probs), rref, cref, _ptr(group_amax), _ptr(x_bf16_out),
                                              _stream(stream)))


def act_bwd_workspace_bytes(act, split_sizes, width_in):
    g = _GroupsArg(split_sizes)
    n = LIB.mgs_act_bwd_workspace_bytes(ctypes.byref(act), g.ref, int(width_in))
    if n < 0:
        _check(int(n))
    return int(n)


def grouped_scaled_act_bwd(act, fmt, split_sizes, width_in, x, dy, probs, dx=None, dx_row=None,
                           dx_col=None, dx_group_amax=None, dprobs=None, dx_col_sum=None, act_col=None,
                           saved_group_amax=None, workspace=None, stream=None):
    """`workspace` (a CUDA tensor) is needed with dprobs or dx_col_sum; when it is None one of the
    right size is allocated here for the call."""
    g = _GroupsArg(split_sizes)
    _r, rref = _qref(dx_row)
    _c, cref = _qref(dx_col)
    _a, aref = _qref(act_col)
    if (dprobs is not None or dx_col_sum is not None) and workspace is None:
        workspace = torch.empty(max(act_bwd_workspace_bytes(act, split_sizes, width_in), 1),
                                dtype=torch.uint8, device="cuda")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(LIB.mgs_grouped_scaled_act_bwd(ctypes.byref(act), FMT[fmt], g.ref, int(width_in), _ptr(x),
                                          _ptr(dy), _ptr(probs), _ptr(dx), rref, cref,
                                          _ptr(dx_group_amax), _ptr(dprobs), _ptr(dx_col_sum), aref,
                                          _ptr(saved_group_amax), _ptr(workspace), int(ws_bytes),
                                          _stream(stream)))


def grouped_scaled_act_bwd_noalloc(act, fmt, split_sizes, width_in, x, dy, probs, dx=None, dx_row=None,
                                   dx_col=None, dx_group_amax=None, dprobs=None, dx_col_sum=None,
                                   act_col=None, saved_group_amax=None, stream=None):
    """The backward with the library's static per-device scratch in place of a workspace: nothing is
    allocated here or in the library.  Calls that overlap on one device race on that scratch."""
    g = _GroupsArg(split_sizes)
    _r, rref = _qref(dx_row)
    _c, cref = _qref(dx_col)
    _a, aref = _qref(act_col)
    _check(LIB.mgs_grouped_scaled_act_bwd_noalloc(ctypes.byref(act), FMT[fmt], g.ref, int(width_in), _ptr(x),
                                                  _ptr(dy), _ptr(probs), _ptr(dx), rref, cref,
                                                  _ptr(dx_group_amax), _ptr(dprobs), _ptr(dx_col_sum), aref,
                                                  _ptr(saved_group_amax), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 16 << 20  # MGS_NOALLOC_SCRATCH_BYTES


def quantize_workspace_bytes(split_sizes, width):
    g = _GroupsArg(split_sizes)
    n = LIB.mgs_grouped_mx_quantize_workspace_bytes(g.ref, int(width))
    if n < 0:
        _check(int(n))
    return int(n)


def grouped_mx_quantize(fmt, split_sizes, width, x, out_row=None, out_col=None, group_amax=None,
                        col_sum=None, workspace=None, stream=None):
    """`workspace` (a CUDA tensor) is needed with col_sum; when it is None one of the right size is
    allocated here for the call."""
    g = _GroupsArg(split_sizes)
    _r, rref = _qref(out_row)
    _c, cref = _qref(out_col)
    if col_sum is not None and workspace is None:
        workspace = torch.empty(max(quantize_workspace_bytes(split_sizes, width), 1), dtype=torch.uint8,
                                device="cuda")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(LIB.mgs_grouped_mx_quantize(FMT[fmt], g.ref, int(width), _ptr(x), rref, cref,
                                       _ptr(group_amax), _ptr(col_sum), _ptr(workspace), int(ws_bytes),
                                       _stream(stream)))


def grouped_gemm_mx(mode, fmt, split_sizes, m, n, k, a, b, c, bias=None, accumulate=False,
                    stream=None):
    g = _GroupsArg(split_sizes)
    _a, aref = _qref(a)
    _b, bref = _qref(b)
    _check(LIB.mgs_grouped_gemm_mx(GEMM_MODE[mode], FMT[fmt], g.ref, int(m), int(n), int(k), aref, bref,
                                   _ptr(c), DTYPE[c.dtype], _ptr(bias), int(bool(accumulate)),
                                   _stream(stream)))


def grouped_gemm_mx_fprop_act(split_sizes, m, n, k, a, b, c, act, probs, out_row, bias=None,
                              act_input="bf16", stream=None):
    """MXFP8 FPROP whose epilogue also writes out_row = MXFP8(act(c) * probs); c is BF16."""
    g = _GroupsArg(split_sizes)
    _a, aref = _qref(a)
    _b, bref = _qref(b)
    _o, oref = _qref(out_row)
    _check(LIB.mgs_grouped_gemm_mx_fprop_act(g.ref, int(m), int(n), int(k), aref, bref, _ptr(c), _ptr(bias),
                                             ctypes.byref(act), _ptr(probs),
                                             {"bf16": 0, "fp32": 1}[act_input], oref, _stream(stream)))


def grouped_col_sum(split_sizes, width, x, out, stream=None):
    g = _GroupsArg(split_sizes)
    _check(LIB.mgs_grouped_col_sum(g.ref, int(width), _ptr(x), _ptr(out), _stream(stream)))
