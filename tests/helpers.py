"""Shared helpers for the GPU parity tests: device I/O, guard bands, bounds.

The acceptance bounds (stated once here, used by every GPU test):
  conv3d:          |gpu - ref| <= 2e-3 * S + ulp16(ref),
                   S = |b| + sum |w * xhat| (the oracle's magnitude), and
                   ulp16(v) = 2^(max(floor(log2|v|), -14) - 10), the fp16
                   spacing at v.  fp32 accumulation over K <= 13,824 terms
                   costs at most K * 2^-24 * S ~ 8.2e-4 S; the final RNE
                   rounding costs half an ulp.
  groupnorm_silu:  |gpu - ref| <= 1e-3 * |ref| + 2^-14 (the absolute floor,
                   the smallest fp16 normal, covers SiLU's zero crossing).
bf16 outputs (8 significant bits): the same with the bf16 ulp in place of the
fp16 one (conv), or added (GroupNorm, whose relative term is below half a bf16
ulp).  The T=1 fold of bf16 weights rounds each summed weight once to bf16:
with 8 significant bits, round-to-nearest-even errs by at most 2^-8 of the
value, so each folded weight carries at most 2^-8 * sum_tau |w_tau| and the
output at most 2^-8 * S more; the fold path of bf16 therefore uses
(2e-3 + 2^-8) * S (BF16_FOLD_REL).  The fp16 fold's one rounding (11
significant bits, 2^-11 * S <= 4.9e-4 * S) stays inside 2e-3 * S.
"""
from __future__ import annotations

import os
from contextlib import contextmanager

import numpy as np
import torch

import convolution_implicit_gemm_amd as c3d

BF16_FOLD_REL = 2e-3 + 2.0 ** -8  # the bf16 T=1 fold path's relative bound (see above)
GUARD = 64  # fp16 elements of guard band on each side of every output
GUARD_BITS = 0x7E5A  # a NaN pattern no kernel writes


def dev(a):
    """numpy fp16 -> torch fp16 on cuda:0; numpy uint16 (bf16 bits) -> torch bfloat16."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(a).to("cuda:0")


def host_bits(t):
    """torch bfloat16 tensor -> numpy uint16 bits on the host."""
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def guarded_empty(shape, dtype=torch.float16):
    """(buffer, view): a 16-bit device tensor with guard bands of a fixed pattern around it."""
    n = int(np.prod(shape))
    buf = torch.empty(n + 2 * GUARD, dtype=torch.int16, device="cuda:0")
    buf.fill_(GUARD_BITS - 65536 if GUARD_BITS > 32767 else GUARD_BITS)
    view = buf[GUARD:GUARD + n].view(dtype).view(shape)
    return buf, view


def check_guards(buf):
    want = np.int16(GUARD_BITS - 65536 if GUARD_BITS > 32767 else GUARD_BITS)
    assert np.all(buf[:GUARD].cpu().numpy() == want), "write before the output tensor"
    assert np.all(buf[-GUARD:].cpu().numpy() == want), "write past the output tensor"


@contextmanager
def env_var(name, value):
    old = os.environ.get(name)
    if value is None:
        os.environ.pop(name, None)
    else:
        os.environ[name] = value
    try:
        yield
    finally:
        if old is None:
            os.environ.pop(name, None)
        else:
            os.environ[name] = old


def workspace_for(plan):
    """Device workspace of the planned size (None when the plan needs none)."""
    if not plan.workspace_bytes:
        return None
    return torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda:0")


@contextmanager
def forced_tile(name):
    old = os.environ.get("CONV3D_TILE")
    if name:
        os.environ["CONV3D_TILE"] = name
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("CONV3D_TILE", None)
        else:
            os.environ["CONV3D_TILE"] = old


def tile_names():
    """Tile configurations compiled into the library (by forcing each name in turn)."""
    names = ["m256n256k64s2w4", "m256n256k32s4w4", "m256n256k64s2w8", "m256n256k64s2a3w8",
             "m256n256k64s2a3w4", "m256n128k64s2a3w4", "m128n128k64s2a3w4", "m128n64k64s2w4",
             "m128n32k32s2w4"]
    return names


def conv_desc(shape, flags=0):
    return c3d.make_desc(shape.n, shape.t, shape.h, shape.w, shape.cin, shape.cout, shape.kt,
                         shape.kh, shape.kw, shape.pad_t_front, shape.pad_t_back, shape.pad_h,
                         shape.pad_w, shape.tmode, flags)


def out_dims(shape):
    return (shape.n, shape.t + shape.pad_t_front + shape.pad_t_back - shape.kt + 1,
            shape.h + 2 * shape.pad_h - shape.kh + 1, shape.w + 2 * shape.pad_w - shape.kw + 1,
            shape.cout)


def run_conv(shape, x, w, b=None, res=None, flags=0, tile=None, keep_device=False, split=None):
    """Run the HIP conv through the C ABI; returns (y numpy or device tensor, plan info).

    fp16 inputs give an fp16 result; uint16 inputs are bf16 bits (the plan gets
    CONV3D_F_BF16) and the result is uint16 bits too.
    split: None lets the planner decide on K-splitting; "0" forbids it, "1" forces it.
    """
    bf16 = (x.dtype == torch.bfloat16) if isinstance(x, torch.Tensor) else (np.asarray(x).dtype == np.uint16)
    if bf16:
        flags |= c3d.CONV3D_F_BF16
    if b is not None:
        flags |= c3d.CONV3D_F_BIAS
    if res is not None:
        flags |= c3d.CONV3D_F_RESIDUAL
    with forced_tile(tile), env_var("CONV3D_STREAMK", split):
        plan = c3d.conv3d_plan(conv_desc(shape, flags))
    info = plan.info()
    xd = x if isinstance(x, torch.Tensor) else dev(x)
    wd = w if isinstance(w, torch.Tensor) else dev(w)
    bd = None if b is None else (b if isinstance(b, torch.Tensor) else dev(b))
    rd = None if res is None else (res if isinstance(res, torch.Tensor) else dev(res))
    buf, y = guarded_empty(out_dims(shape), torch.bfloat16 if bf16 else torch.float16)
    c3d.conv3d_forward(plan, xd, wd, bd, rd, y, workspace_for(plan))
    torch.cuda.synchronize()
    check_guards(buf)
    if keep_device:
        return y, info
    return (host_bits(y) if bf16 else y.cpu().numpy()), info


def ulp16(v):
    a = np.abs(np.asarray(v, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.where(a > 0, np.maximum(e, -14), -14)
    return np.exp2(e - 10)


def ulp_bf16(v):
    """bf16 spacing at v: 8 significant bits, normal range down to 2^-126."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.where(a > 0, np.maximum(e, -126), -126)
    return np.exp2(e - 7)


def conv_violations(gpu, ref, mag, rel=2e-3, ulp=None):
    """Indices where the conv bound fails, and the worst ratio err / bound.

    Bound: rel * S + one ulp of the output format at ref (fp16 unless ulp is given).
    """
    g = np.asarray(gpu, dtype=np.float64)
    err = np.abs(g - ref)
    bound = rel * mag + (ulp16(ref) if ulp is None else ulp(ref))
    bad = ~(err <= bound)  # NaN counts as a failure
    ratio = float(np.max(err / bound)) if err.size else 0.0
    return np.flatnonzero(bad.reshape(-1)), ratio


def assert_conv_close(gpu, ref, mag, what="", rel=2e-3, ulp=None):
    bad, ratio = conv_violations(gpu, ref, mag, rel, ulp)
    if bad.size:
        g = np.asarray(gpu, dtype=np.float64).reshape(-1)
        i = bad[0]
        raise AssertionError("%s: %d of %d outside bound (worst err/bound %.3g); first at %d: "
                             "gpu %r ref %r S %r" % (what, bad.size, g.size, ratio, i, g[i],
                                                     np.asarray(ref).reshape(-1)[i],
                                                     np.asarray(mag).reshape(-1)[i]))
    return ratio


def assert_gn_close(gpu, ref, what="", ulp=None):
    """|gpu - ref| <= 1e-3 |ref| + 2^-14, plus one output ulp at ref when ulp is given (bf16)."""
    g = np.asarray(gpu, dtype=np.float64)
    err = np.abs(g - ref)
    bound = 1e-3 * np.abs(ref) + 2.0 ** -14 + (0.0 if ulp is None else ulp(ref))
    bad = ~(err <= bound)
    if np.any(bad):
        i = np.flatnonzero(bad.reshape(-1))[0]
        raise AssertionError("%s: %d of %d outside bound; first at %d: gpu %r ref %r" % (
            what, int(bad.sum()), g.size, i, g.reshape(-1)[i], np.asarray(ref).reshape(-1)[i]))
    return float(np.max(err / bound)) if err.size else 0.0


def sample_points(m_total, cout, count, seed, extra_m=()):
    """Seeded (m, co) sample: `count` random pairs plus every channel at the voxels in extra_m."""
    rng = np.random.default_rng(seed)
    m = rng.integers(0, m_total, count)
    co = rng.integers(0, cout, count)
    if len(extra_m):
        em = np.repeat(np.asarray(extra_m, dtype=np.int64), cout)
        ec = np.tile(np.arange(cout), len(extra_m))
        m = np.concatenate([m, em])
        co = np.concatenate([co, ec])
    return m, co


def edge_voxels(odims):
    """Flat indices of corner/edge voxels of first, second and last frames."""
    n, t, h, w, _ = odims
    out = []
    for nn in {0, n - 1}:
        for tt in sorted({0, min(1, t - 1), t - 1}):
            for hh in sorted({0, h // 2, h - 1}):
                for ww in sorted({0, w // 2, w - 1}):
                    out.append(((nn * t + tt) * h + hh) * w + ww)
    return out


def frame_voxels(odims, frames):
    """Flat output-voxel indices of every voxel of the given output frames (all samples)."""
    n, t, h, w, _ = odims
    hw = h * w
    out = [np.arange((nn * t + f) * hw, (nn * t + f + 1) * hw, dtype=np.int64)
           for nn in range(n) for f in sorted(set(int(f) % t for f in frames))]
    return np.concatenate(out)


def row_sample(odims, frac, seed):
    """A seeded fraction of all output voxels (at least one), sorted."""
    n, t, h, w, _ = odims
    total = n * t * h * w
    k = max(1, int(round(frac * total)))
    return np.sort(np.random.default_rng(seed).choice(total, k, replace=False)).astype(np.int64)


def check_voxels(shape, x, w, b, y_dev, vox, res=None, what="", rel=2e-3, ulp=None):
    """Every output channel at the voxels `vox`, GPU against the fp64 oracle.

    x, w, b, res are host arrays (x ideally float64: the oracle then reads it
    without decoding fp16 per product); y_dev is the GPU output (device tensor),
    gathered at `vox` on the device so that only the checked rows come back.
    Returns the worst err / bound.
    """
    import oracle
    cout = shape.cout
    vt = torch.from_numpy(np.ascontiguousarray(vox)).to(y_dev.device)
    got = y_dev.reshape(-1, cout).index_select(0, vt)
    got = (host_bits(got) if got.dtype == torch.bfloat16 else got.cpu().numpy())
    m = np.repeat(vox, cout)
    co = np.tile(np.arange(cout, dtype=np.int64), vox.size)
    ref, mag = oracle.conv3d_points(x, w, b, res, shape.pads, shape.tmode, m, co)
    return assert_conv_close(got.reshape(-1), ref, mag, "%s (%d voxels x %d channels)" % (what, vox.size, cout),
                             rel=rel, ulp=ulp)
