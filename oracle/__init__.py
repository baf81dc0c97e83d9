"""fp64 CPU oracle for the fp16 conv3d / GroupNorm+SiLU hot path.

TEST INFRASTRUCTURE ONLY: the checker the HIP path is compared against.  Only
the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It never imports the product package
and shares no code with it; the product never imports this.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over output rows).
This module compiles it with gcc, widens the fp16 operands to float64 (exact)
and composes the decoder block.  Definitions and their sources are stated in
``oracle.c``'s header.

Function inventory and pins (tests/test_oracle_*.py):
  conv3d            -- pinned: brute force vs an explicit im2col + numpy matmul;
                       torch.nn.functional.conv3d (fp64, CPU) on the padded
                       tensor; all-ones closed form; delta / shifted delta;
                       1x1x1 == numpy matmul; linearity; causality; the causal
                       identity (3D == sum over temporal taps of 2D) and its
                       T=1 fold; S == conv(|x|, |w|) + |b|.
  conv3d_points     -- pinned: equals conv3d at sampled points.
  groupnorm_silu    -- pinned: torch.nn.functional.group_norm (fp64, CPU) +
                       SiLU; closed forms (constant group, +-a halves);
                       per-sample independence; shift/scale invariance.
  groupnorm_silu_points -- pinned: equals groupnorm_silu (values and
                       statistics) at every element of small tensors, fp16
                       and fp64 inputs.
  bf16_to_f64       -- pinned: every one of the 65,536 patterns against the
                       value sign * 2^(e-127) * (1 + f/128) (normal) or
                       sign * 2^-126 * f/128 (subnormal) built term by term.
  decoder_block     -- a composition of the two above.  Its end-to-end
                       tolerance is not fixed by the pages: parity unpinned
                       beyond the pins of its parts.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

TPAD_ZERO = 0
TPAD_REPLICATE = 1

_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (-O2 -fopenmp, no fast-math, no BLAS)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall", "-Wextra",
             "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        d = ctypes.POINTER(ctypes.c_double)
        i = ctypes.c_int
        lib.oracle_conv3d.argtypes = [d, d, d, d] + [i] * 14 + [d, d]
        lib.oracle_conv3d.restype = i
        vp = ctypes.c_void_p
        lib.oracle_conv3d_points.argtypes = ([vp, i, d, d, vp, i] + [i] * 14 +
                                             [ctypes.POINTER(ctypes.c_int64),
                                              ctypes.POINTER(ctypes.c_int32),
                                              ctypes.c_int64, d, d])
        lib.oracle_conv3d_points.restype = i
        lib.oracle_groupnorm_silu.argtypes = [d, i, ctypes.c_int64, i, i, d, d, ctypes.c_double,
                                              i, d, d, d]
        lib.oracle_groupnorm_silu.restype = i
        lib.oracle_groupnorm_silu_points.argtypes = [vp, i, i, ctypes.c_int64, i, i, d, d, ctypes.c_double, i,
                                                     ctypes.POINTER(ctypes.c_int64),
                                                     ctypes.POINTER(ctypes.c_int32), ctypes.c_int64, d, d, d]
        lib.oracle_groupnorm_silu_points.restype = i
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f64.restype = ctypes.c_double
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = i
        _lib = lib
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle runs on."""
    return _load().oracle_num_threads()


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a), dtype=np.float64)


def _ptr(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def out_shape(x_shape, w_shape, pads):
    n, t, h, w, _ = x_shape
    cout, kt, kh, kw, _ = w_shape
    ptf, ptb, ph, pw = pads
    return (n, t + ptf + ptb - kt + 1, h + 2 * ph - kh + 1, w + 2 * pw - kw + 1, cout)


def conv3d(x, w, b=None, res=None, pads=(1, 1, 1, 1), tmode=TPAD_ZERO, with_mag=True):
    """fp64 conv3d on NDHWC x [N,T,H,W,Cin] and w [Cout,kt,kh,kw,Cin].

    pads = (pad_t_front, pad_t_back, pad_h, pad_w); tmode TPAD_ZERO or
    TPAD_REPLICATE.  Returns (y, S) with S = |b| + sum |w * xhat| (None if
    with_mag is False).
    """
    x, w, b, res = _f64(x), _f64(w), _f64(b), _f64(res)
    n, t, h, wd, cin = x.shape
    cout, kt, kh, kw, cin2 = w.shape
    if cin != cin2:
        raise ValueError("channel mismatch")
    oshape = out_shape(x.shape, w.shape, pads)
    if res is not None and res.shape != oshape:
        raise ValueError("residual shape %s != output %s" % (res.shape, oshape))
    y = np.empty(oshape, np.float64)
    mag = np.empty(oshape, np.float64) if with_mag else None
    rc = _load().oracle_conv3d(_ptr(x), _ptr(w), _ptr(b), _ptr(res), n, t, h, wd, cin, cout,
                               kt, kh, kw, pads[0], pads[1], pads[2], pads[3], tmode,
                               _ptr(y), _ptr(mag))
    if rc != 0:
        raise ValueError("oracle_conv3d rejected the shape")
    return y, mag


def _maybe_f16(a):
    """(pointer, is_f16, keepalive) for an fp16 array passed as raw bits, else fp64."""
    if a is None:
        return None, 0, None
    a = np.asarray(a)
    if a.dtype == np.float16:
        a = np.ascontiguousarray(a)
        return a.ctypes.data_as(ctypes.c_void_p), 1, a
    a = _f64(a)
    return a.ctypes.data_as(ctypes.c_void_p), 0, a


def f16_to_f64(bits: int) -> float:
    """The oracle's exact binary16 decoder (exposed for its pin)."""
    return _load().oracle_f16_to_f64(bits)


def bf16_to_f64(bits):
    """Exact values of bf16 bit patterns (uint16 array) as float64.

    bf16 is the upper half of an IEEE binary32: widening the pattern by 16 zero
    bits gives the binary32 of the same value, which float64 holds exactly.
    """
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns widen to quiet NaNs
        return b.view(np.float32).astype(np.float64)


def conv3d_points(x, w, b, res, pads, tmode, m_idx, co_idx):
    """conv3d at selected outputs: flat voxel index m_idx[i], channel co_idx[i].

    Returns (y[i], S[i]).  x and res (full residual tensor or None) may be
    float16 numpy arrays, read in place and widened exactly in C, so that
    multi-GB activations need no fp64 copy; w and b are widened here.
    """
    xp, xh, xkeep = _maybe_f16(x)
    rp, rh, rkeep = _maybe_f16(res)
    w, b = _f64(w), _f64(b)
    n, t, h, wd, cin = xkeep.shape
    cout, kt, kh, kw, _ = w.shape
    m_idx = np.ascontiguousarray(m_idx, dtype=np.int64)
    co_idx = np.ascontiguousarray(co_idx, dtype=np.int32)
    y = np.empty(m_idx.shape[0], np.float64)
    mag = np.empty(m_idx.shape[0], np.float64)
    rc = _load().oracle_conv3d_points(
        xp, xh, _ptr(w), _ptr(b), rp, rh, n, t, h, wd, cin, cout, kt, kh, kw,
        pads[0], pads[1], pads[2], pads[3], tmode,
        m_idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        co_idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
        m_idx.shape[0], _ptr(y), _ptr(mag))
    del xkeep, rkeep
    if rc != 0:
        raise ValueError("oracle_conv3d_points rejected the input")
    return y, mag


def groupnorm_silu(x, gamma, beta, groups, eps=1e-6, apply_silu=True, return_stats=False):
    """Two-pass fp64 GroupNorm (+SiLU) on channels-last x [N, ..., C]."""
    x = _f64(x)
    shape = x.shape
    n, c = shape[0], shape[-1]
    thw = int(np.prod(shape[1:-1])) if len(shape) > 2 else 1
    g, bt = _f64(gamma), _f64(beta)
    y = np.empty_like(x)
    mean = np.empty((n, groups), np.float64)
    var = np.empty((n, groups), np.float64)
    rc = _load().oracle_groupnorm_silu(_ptr(x), n, thw, c, groups, _ptr(g), _ptr(bt), float(eps),
                                       1 if apply_silu else 0, _ptr(y), _ptr(mean), _ptr(var))
    if rc != 0:
        raise ValueError("oracle_groupnorm_silu rejected the shape")
    if return_stats:
        return y, mean, var
    return y


def groupnorm_silu_points(x, gamma, beta, groups, vox_idx, ch_idx, eps=1e-6, apply_silu=True):
    """GroupNorm (+SiLU) at selected elements: flat voxel vox_idx[i] (over N*THW), channel ch_idx[i].

    x: [N, ..., C]; a float16 array is read in place and widened exactly in C,
    so that multi-GB activations need no fp64 copy.  The statistics are the
    two-pass ones of groupnorm_silu.  Returns (y[i], mean[N, groups], var[N, groups]).
    """
    xp, xh, xkeep = _maybe_f16(x)
    shape = xkeep.shape
    n, c = shape[0], shape[-1]
    thw = int(np.prod(shape[1:-1])) if len(shape) > 2 else 1
    g, bt = _f64(gamma), _f64(beta)
    vox_idx = np.ascontiguousarray(vox_idx, dtype=np.int64)
    ch_idx = np.ascontiguousarray(ch_idx, dtype=np.int32)
    y = np.empty(vox_idx.shape[0], np.float64)
    mean = np.empty((n, groups), np.float64)
    var = np.empty((n, groups), np.float64)
    rc = _load().oracle_groupnorm_silu_points(
        xp, xh, n, thw, c, groups, _ptr(g), _ptr(bt), float(eps), 1 if apply_silu else 0,
        vox_idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        ch_idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), vox_idx.shape[0], _ptr(y), _ptr(mean), _ptr(var))
    del xkeep
    if rc != 0:
        raise ValueError("oracle_groupnorm_silu_points rejected the input")
    return y, mean, var


def decoder_block(x, gn1, conv1, gn2, conv2, groups=32, eps=1e-6, pads=(2, 0, 1, 1),
                  tmode=TPAD_REPLICATE):
    """fp64 3D ResNet decoder block: x + conv2(SiLU(GN2(conv1(SiLU(GN1(x)))))).

    gn* = (gamma, beta); conv* = (w, b).  Everything stays in fp64 (no fp16
    rounding between stages).
    """
    a1 = groupnorm_silu(x, gn1[0], gn1[1], groups, eps)
    c1, _ = conv3d(a1, conv1[0], conv1[1], None, pads, tmode, with_mag=False)
    a2 = groupnorm_silu(c1, gn2[0], gn2[1], groups, eps)
    out, _ = conv3d(a2, conv2[0], conv2[1], _f64(x), pads, tmode, with_mag=False)
    return out
