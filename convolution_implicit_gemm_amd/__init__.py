"""Python binding of libconv3d (MI355X / gfx950 fp16 implicit-GEMM conv3d).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libconv3d.so``.  The functions carry the C names of
``include/conv3d.h``.  Tensor arguments may be torch tensors (their
``data_ptr()`` is passed) or raw device addresses (ints); the stream defaults
to torch's current stream on the current device.  There is no CPU fallback:
if the library is missing, importing a function raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libconv3d.so")

CONV3D_OK = 0
CONV3D_ERR_INVALID_ARG = 1
CONV3D_ERR_UNSUPPORTED = 2
CONV3D_ERR_WORKSPACE = 3
CONV3D_ERR_NO_DEVICE = 4
CONV3D_ERR_HIP = 5

CONV3D_TPAD_ZERO = 0
CONV3D_TPAD_REPLICATE = 1

CONV3D_F_BIAS = 1
CONV3D_F_RESIDUAL = 2
CONV3D_F_NO_T1_FASTPATH = 4
CONV3D_F_BF16 = 8
CONV3D_F_CHUNK = 16
CONV3D_F_GN_STATS = 32

CONV3D_PATH_GENERAL = 0
CONV3D_PATH_T1_FOLD = 1
CONV3D_PATH_POINTWISE = 2

EXPORTED = ("conv3d_plan", "conv3d_plan_query", "conv3d_plan_destroy", "conv3d_forward",
            "conv3d_forward_chunk",
            "groupnorm_silu_workspace", "groupnorm_silu", "groupnorm_silu_bf16",
            "groupnorm_silu_from_stats_workspace", "groupnorm_silu_from_stats", "groupnorm_silu_from_stats_bf16",
            "groupnorm_silu_noalloc_max_bytes", "groupnorm_silu_noalloc",
            "conv3d_calibrate_scratch_bytes",
            "conv3d_calibrate_mfma", "conv3d_calibrate_hbm", "conv3d_clock_stamp_bytes",
            "conv3d_clock_stamp", "conv3d_status_str",
            "conv3d_last_error", "conv3d_version", "conv3d_selftest")


class conv3d_desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("n", "t", "h", "w", "c_in", "c_out", "kt", "kh", "kw",
                 "pad_t_front", "pad_t_back", "pad_h", "pad_w", "t_pad_mode")] + \
               [("flags", ctypes.c_uint32)]


class conv3d_plan_info(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("t_out", ctypes.c_int32), ("h_out", ctypes.c_int32),
                ("w_out", ctypes.c_int32), ("gemm_m", ctypes.c_int64), ("gemm_n", ctypes.c_int64),
                ("gemm_k", ctypes.c_int64), ("flops", ctypes.c_double), ("tile_m", ctypes.c_int32),
                ("tile_n", ctypes.c_int32), ("tile_k", ctypes.c_int32), ("stages", ctypes.c_int32),
                ("threads", ctypes.c_int32), ("grid", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_size_t), ("kernel_name", ctypes.c_char * 64),
                ("split_tiles", ctypes.c_int32), ("split_pieces", ctypes.c_int32),
                ("gn_stats_slots", ctypes.c_int32), ("gn_stats_offset", ctypes.c_size_t)]


class Conv3dError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s (status %d): %s" % (_status_name(status), status, message))
        self.status = status


def _status_name(s):
    return {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "WORKSPACE", 4: "NO_DEVICE",
            5: "HIP"}.get(s, "UNKNOWN")


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libconv3d.so (raises OSError if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise OSError("libconv3d.so not built at %s: run python -m convolution_implicit_gemm_amd.build"
                      % path)
    lib = ctypes.CDLL(path)
    vp, sz, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
    lib.conv3d_plan.argtypes = [ctypes.POINTER(conv3d_desc), ctypes.POINTER(vp), ctypes.POINTER(sz)]
    lib.conv3d_plan.restype = ctypes.c_int
    lib.conv3d_plan_query.argtypes = [vp, ctypes.POINTER(conv3d_plan_info)]
    lib.conv3d_plan_query.restype = ctypes.c_int
    lib.conv3d_plan_destroy.argtypes = [vp]
    lib.conv3d_plan_destroy.restype = None
    lib.conv3d_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.conv3d_forward_chunk.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.conv3d_forward_chunk.restype = ctypes.c_int
    lib.conv3d_forward.restype = ctypes.c_int
    lib.groupnorm_silu_workspace.argtypes = [i32, i64, i32, i32]
    lib.groupnorm_silu_workspace.restype = sz
    lib.groupnorm_silu.argtypes = [vp, vp, vp, vp, i32, i64, i32, i32, ctypes.c_float, i32, vp, sz, vp]
    lib.groupnorm_silu_bf16.argtypes = lib.groupnorm_silu.argtypes
    lib.groupnorm_silu_bf16.restype = ctypes.c_int
    lib.groupnorm_silu.restype = ctypes.c_int
    lib.groupnorm_silu_from_stats_workspace.argtypes = [i32, i32, i32]
    lib.groupnorm_silu_from_stats_workspace.restype = sz
    lib.groupnorm_silu_from_stats.argtypes = [vp, vp, vp, vp, i32, i64, i32, i32, ctypes.c_float, i32, vp, i32,
                                              vp, sz, vp]
    lib.groupnorm_silu_from_stats.restype = ctypes.c_int
    lib.groupnorm_silu_from_stats_bf16.argtypes = lib.groupnorm_silu_from_stats.argtypes
    lib.groupnorm_silu_from_stats_bf16.restype = ctypes.c_int
    lib.groupnorm_silu_noalloc_max_bytes.argtypes = []
    lib.groupnorm_silu_noalloc_max_bytes.restype = sz
    lib.groupnorm_silu_noalloc.argtypes = [vp, vp, vp, vp, i32, i64, i32, i32, ctypes.c_float, i32, vp]
    lib.groupnorm_silu_noalloc.restype = ctypes.c_int
    lib.conv3d_status_str.argtypes = [ctypes.c_int]
    lib.conv3d_status_str.restype = ctypes.c_char_p
    lib.conv3d_last_error.argtypes = []
    lib.conv3d_last_error.restype = ctypes.c_char_p
    lib.conv3d_version.argtypes = []
    lib.conv3d_version.restype = i32
    lib.conv3d_selftest.argtypes = []
    lib.conv3d_selftest.restype = i32
    dp = ctypes.POINTER(ctypes.c_double)
    lib.conv3d_calibrate_scratch_bytes.argtypes = []
    lib.conv3d_calibrate_scratch_bytes.restype = sz
    lib.conv3d_calibrate_mfma.argtypes = [vp, sz, dp, dp, vp]
    lib.conv3d_calibrate_mfma.restype = ctypes.c_int
    lib.conv3d_calibrate_hbm.argtypes = [vp, vp, sz, dp, dp, vp]
    lib.conv3d_calibrate_hbm.restype = ctypes.c_int
    lib.conv3d_clock_stamp_bytes.argtypes = []
    lib.conv3d_clock_stamp_bytes.restype = sz
    lib.conv3d_clock_stamp.argtypes = [vp, sz, vp]
    lib.conv3d_clock_stamp.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status):
    if status != CONV3D_OK:
        raise Conv3dError(status, load_library().conv3d_last_error().decode())


def _addr(t, what="tensor", elems=None, dtype=None):
    """Device address of a torch tensor (or an int address, passed as is).

    A tensor must be contiguous and on a GPU; with ``elems`` / ``dtype`` it
    must also hold at least that many elements of that dtype (the C layer
    sees only the address and cannot check any of this).  Raises Conv3dError
    (INVALID_ARG) otherwise, before anything is enqueued.
    """
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise Conv3dError(CONV3D_ERR_INVALID_ARG, "%s is not contiguous (pass .contiguous())" % what)
    if t.device.type != "cuda":
        raise Conv3dError(CONV3D_ERR_INVALID_ARG, "%s is on %s, not on a GPU" % (what, t.device))
    if dtype is not None and t.dtype != dtype:
        raise Conv3dError(CONV3D_ERR_INVALID_ARG, "%s is %s, the plan expects %s" % (what, t.dtype, dtype))
    if elems is not None and t.numel() < elems:
        raise Conv3dError(CONV3D_ERR_INVALID_ARG, "%s holds %d elements, %d needed" % (what, t.numel(), elems))
    return t.data_ptr()


def _elem_dtype(bf16):
    import torch
    return torch.bfloat16 if bf16 else torch.float16


def _conv_sizes(desc, chunk_t=None):
    """(x, x_prev, weight, bias, y) element counts of a plan's descriptor."""
    d = desc
    to = d.t if chunk_t else d.t + d.pad_t_front + d.pad_t_back - d.kt + 1
    ho = d.h + 2 * d.pad_h - d.kh + 1
    wo = d.w + 2 * d.pad_w - d.kw + 1
    return (d.n * d.t * d.h * d.w * d.c_in, d.n * max(d.kt - 1, 0) * d.h * d.w * d.c_in,
            d.c_out * d.kt * d.kh * d.kw * d.c_in, d.c_out, d.n * to * ho * wo * d.c_out)


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Plan:
    """Owns a conv3d_plan_t; destroyed with the object."""

    def __init__(self, handle, workspace_bytes, desc):
        self.handle = handle
        self.workspace_bytes = workspace_bytes
        self.desc = desc

    def info(self) -> conv3d_plan_info:
        return conv3d_plan_query(self)

    def __del__(self):
        if self.handle and _lib is not None:
            _lib.conv3d_plan_destroy(self.handle)
            self.handle = None


def weight_from_ncdhw(weight):
    """A torch Conv3d weight [Cout][Cin][kt][kh][kw] in this library's layout
    [Cout][kt][kh][kw][Cin] (a contiguous copy).  A load-time conversion, done
    once per weight, off the forward path."""
    return weight.permute(0, 2, 3, 4, 1).contiguous()


def make_desc(n, t, h, w, c_in, c_out, kt=3, kh=3, kw=3, pad_t_front=1, pad_t_back=1, pad_h=1,
              pad_w=1, t_pad_mode=CONV3D_TPAD_ZERO, flags=0) -> conv3d_desc:
    return conv3d_desc(n, t, h, w, c_in, c_out, kt, kh, kw, pad_t_front, pad_t_back, pad_h, pad_w,
                       t_pad_mode, flags)


def conv3d_plan(desc: conv3d_desc) -> Plan:
    lib = load_library()
    h = ctypes.c_void_p()
    ws = ctypes.c_size_t()
    _check(lib.conv3d_plan(ctypes.byref(desc), ctypes.byref(h), ctypes.byref(ws)))
    return Plan(h.value, ws.value, desc)


def conv3d_plan_query(plan: Plan) -> conv3d_plan_info:
    info = conv3d_plan_info()
    _check(load_library().conv3d_plan_query(plan.handle, ctypes.byref(info)))
    return info


def conv3d_plan_destroy(plan: Plan) -> None:
    if plan.handle:
        load_library().conv3d_plan_destroy(plan.handle)
        plan.handle = None


def conv3d_forward(plan: Plan, x, weight, bias, residual, y, workspace=None, workspace_bytes=None,
                   stream=None) -> None:
    """Enqueue y = conv3d(x, weight) (+bias) (+residual) on ``stream``."""
    if workspace_bytes is None:
        if workspace is None:
            workspace_bytes = 0
        elif isinstance(workspace, int):
            workspace_bytes = plan.workspace_bytes
        else:
            workspace_bytes = workspace.numel() * workspace.element_size()
    nx, _, nw, nb, ny = _conv_sizes(plan.desc)
    dt = _elem_dtype(plan.desc.flags & CONV3D_F_BF16)
    _check(load_library().conv3d_forward(plan.handle, _addr(x, "x", nx, dt), _addr(weight, "weight", nw, dt),
                                         _addr(bias, "bias", nb, dt), _addr(residual, "residual", ny, dt),
                                         _addr(y, "y", ny, dt), _addr(workspace, "workspace"),
                                         workspace_bytes, _stream(stream)))


def conv3d_forward_chunk(plan: Plan, x_prev, x, weight, bias, residual, y, workspace,
                         workspace_bytes=None, stream=None) -> None:
    """Enqueue one chunk of a chunked causal decode (plan made with CONV3D_F_CHUNK)."""
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    nx, nxp, nw, nb, ny = _conv_sizes(plan.desc, chunk_t=True)
    dt = _elem_dtype(plan.desc.flags & CONV3D_F_BF16)
    _check(load_library().conv3d_forward_chunk(plan.handle, _addr(x_prev, "x_prev", nxp, dt), _addr(x, "x", nx, dt),
                                               _addr(weight, "weight", nw, dt), _addr(bias, "bias", nb, dt),
                                               _addr(residual, "residual", ny, dt), _addr(y, "y", ny, dt),
                                               _addr(workspace, "workspace"),
                                               workspace_bytes, _stream(stream)))


def groupnorm_silu_workspace(n, thw, c, groups) -> int:
    return load_library().groupnorm_silu_workspace(n, thw, c, groups)


def groupnorm_silu(x, gamma, beta, y, n, thw, c, groups, eps, apply_silu, workspace,
                   workspace_bytes=None, stream=None, bf16=False) -> None:
    """Enqueue y = [SiLU](GroupNorm(x)) on ``stream``."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    lib = load_library()
    fn = lib.groupnorm_silu_bf16 if bf16 else lib.groupnorm_silu
    dt, ne = _elem_dtype(bf16), n * thw * c
    _check(fn(_addr(x, "x", ne, dt), _addr(gamma, "gamma", c, dt), _addr(beta, "beta", c, dt), _addr(y, "y", ne, dt),
              n, thw, c, groups, float(eps), 1 if apply_silu else 0, _addr(workspace, "workspace"),
              workspace_bytes, _stream(stream)))


def groupnorm_silu_from_stats_workspace(n, c, groups) -> int:
    return load_library().groupnorm_silu_from_stats_workspace(n, c, groups)


def gn_stats_view(plan: Plan, workspace):
    """(address, slots) of the GroupNorm partials a CONV3D_F_GN_STATS plan's
    forward leaves in ``workspace`` (a device tensor of the planned size)."""
    info = conv3d_plan_query(plan)
    if not info.gn_stats_slots:
        raise Conv3dError(CONV3D_ERR_INVALID_ARG, "the plan was made without CONV3D_F_GN_STATS")
    if workspace.numel() * workspace.element_size() < plan.workspace_bytes:
        raise Conv3dError(CONV3D_ERR_WORKSPACE, "workspace smaller than the plan's")
    return workspace.data_ptr() + info.gn_stats_offset, info.gn_stats_slots


def groupnorm_silu_from_stats(x, gamma, beta, y, n, thw, c, groups, eps, apply_silu, stats, stats_slots,
                              workspace, workspace_bytes=None, stream=None, bf16=False) -> None:
    """Enqueue y = [SiLU](GroupNorm(x)) with x's statistics merged from the partials
    ``stats`` (an address, see gn_stats_view) that the conv producing x wrote."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    lib = load_library()
    fn = lib.groupnorm_silu_from_stats_bf16 if bf16 else lib.groupnorm_silu_from_stats
    dt, ne = _elem_dtype(bf16), n * thw * c
    _check(fn(_addr(x, "x", ne, dt), _addr(gamma, "gamma", c, dt), _addr(beta, "beta", c, dt), _addr(y, "y", ne, dt),
              n, thw, c, groups, float(eps), 1 if apply_silu else 0, _addr(stats, "stats"), int(stats_slots),
              _addr(workspace, "workspace"), workspace_bytes, _stream(stream)))


def groupnorm_silu_noalloc_max_bytes() -> int:
    return load_library().groupnorm_silu_noalloc_max_bytes()


def groupnorm_silu_noalloc(x, gamma, beta, y, n, thw, c, groups, eps, apply_silu, stream=None) -> None:
    """groupnorm_silu (fp16) with the library's static device scratch instead of a workspace."""
    dt, ne = _elem_dtype(False), n * thw * c
    _check(load_library().groupnorm_silu_noalloc(_addr(x, "x", ne, dt), _addr(gamma, "gamma", c, dt),
                                                 _addr(beta, "beta", c, dt), _addr(y, "y", ne, dt), n, thw, c,
                                                 groups, float(eps), 1 if apply_silu else 0, _stream(stream)))


def conv3d_calibrate_scratch_bytes() -> int:
    return load_library().conv3d_calibrate_scratch_bytes()


def conv3d_calibrate_mfma(scratch, scratch_bytes=None, stream=None):
    """(TFLOP/s, shader MHz) of dense fp16 MFMA chains on random operands; synchronises."""
    if scratch_bytes is None:
        scratch_bytes = scratch.numel() * scratch.element_size()
    tf, mhz = ctypes.c_double(), ctypes.c_double()
    _check(load_library().conv3d_calibrate_mfma(_addr(scratch), scratch_bytes, ctypes.byref(tf),
                                                ctypes.byref(mhz), _stream(stream)))
    return tf.value, mhz.value


def conv3d_calibrate_hbm(src, dst, nbytes, stream=None):
    """(read GB/s, copy GB/s, read + write counted) of 16-byte streams; synchronises."""
    rd, cp = ctypes.c_double(), ctypes.c_double()
    _check(load_library().conv3d_calibrate_hbm(_addr(src), _addr(dst), nbytes, ctypes.byref(rd),
                                               ctypes.byref(cp), _stream(stream)))
    return rd.value, cp.value


def conv3d_clock_stamp_bytes() -> int:
    return load_library().conv3d_clock_stamp_bytes()


def conv3d_clock_stamp(out, out_bytes=None, stream=None) -> None:
    """Enqueue a shader-clock stamp into device buffer ``out`` (see conv3d.h)."""
    if out_bytes is None:
        out_bytes = out.numel() * out.element_size()
    _check(load_library().conv3d_clock_stamp(_addr(out), out_bytes, _stream(stream)))


def sclk_between(before, after):
    """Mean shader clock (MHz) per XCD between two stamps (host uint64 arrays
    of conv3d_clock_stamp's layout): {xcd: MHz}.  Stamps are paired by the CU
    they ran on, since the counters of different CUs are not aligned; an XCD's
    figure is the median over its CUs stamped both times."""
    import numpy as np
    b = np.asarray(before, dtype=np.uint64).reshape(-1, 3)
    a = np.asarray(after, dtype=np.uint64).reshape(-1, 3)
    per_xcd = {}
    for loc in sorted(set(b[:, 2].tolist()) & set(a[:, 2].tolist())):
        bb, aa = b[b[:, 2] == loc], a[a[:, 2] == loc]
        dc = aa[:, 0].astype(np.float64).mean() - bb[:, 0].astype(np.float64).mean()
        dr = aa[:, 1].astype(np.float64).mean() - bb[:, 1].astype(np.float64).mean()
        if dr > 0:
            per_xcd.setdefault(int(loc) & 0xF, []).append(100.0 * dc / dr)
    return {x: float(np.median(v)) for x, v in sorted(per_xcd.items())}


def groupnorm_silu_bf16(x, gamma, beta, y, n, thw, c, groups, eps, apply_silu, workspace,
                        workspace_bytes=None, stream=None) -> None:
    """groupnorm_silu with bf16 x, gamma, beta and y."""
    groupnorm_silu(x, gamma, beta, y, n, thw, c, groups, eps, apply_silu, workspace, workspace_bytes,
                   stream, bf16=True)


def conv3d_status_str(status: int) -> str:
    return load_library().conv3d_status_str(status).decode()


def conv3d_last_error() -> str:
    return load_library().conv3d_last_error().decode()


def conv3d_version() -> int:
    return load_library().conv3d_version()


def conv3d_selftest() -> int:
    """Run the library's start-up self-test on the current device (0 = pass)."""
    return load_library().conv3d_selftest()


def selftest_in_subprocess(timeout: float = 300.0) -> int:
    """conv3d_selftest() in a child process, so that a broken driver or device
    cannot take this process down.  Returns the child's exit status: 0 = pass,
    a conv3d_status or 16 + case number as conv3d_selftest documents,
    negative for a child killed by a signal."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r); import convolution_implicit_gemm_amd as c; "
            "rc = c.conv3d_selftest(); sys.stderr.write(c.conv3d_last_error() + '\\n'); sys.exit(rc)"
            % os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    return subprocess.run([sys.executable, "-c", code], timeout=timeout).returncode
