"""GPU parity of CONV3D_F_GN_STATS and groupnorm_silu_from_stats, through the C ABI.

A conv planned with CONV3D_F_GN_STATS writes, besides y, GroupNorm partial
statistics of y; groupnorm_silu_from_stats normalises y from them.  Checked:
  * y is bit-identical to the same plan without the flag (the statistics only
    read what the epilogue stores);
  * GroupNorm(+SiLU) of y from those partials is within the GroupNorm bound
    (tests/helpers.py) of the fp64 oracle's GroupNorm of the GPU's y, on whole
    tiles, K-split tiles (the fixup's statistics), the one-workgroup-per-CU
    schedule, several samples, a channel tail (c_out not a multiple of the
    256-channel tile), a Cin tail, a residual, bf16, and at the decoder block's
    full size.
"""
import numpy as np
import pytest
import torch

import convolution_implicit_gemm_amd as c3d
import oracle
import workloads
from workloads import ConvShape

from helpers import (assert_gn_close, check_guards, conv_desc, dev, env_var, guarded_empty, host_bits, out_dims,
                     ulp_bf16, workspace_for)

pytestmark = pytest.mark.gpu


def f64(a):
    a = np.asarray(a)
    return oracle.bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def conv_with_stats(shape, d, res=None, split=None, dynamic=None, bf16=False, extra_flags=0):
    """(y with the flag, y without it, plan, workspace) for one conv."""
    flags = c3d.CONV3D_F_BIAS | (c3d.CONV3D_F_RESIDUAL if res is not None else 0) | \
        (c3d.CONV3D_F_BF16 if bf16 else 0) | extra_flags
    dt = torch.bfloat16 if bf16 else torch.float16
    out = []
    for extra in (c3d.CONV3D_F_GN_STATS, 0):
        # the statistics come from the row-slab tile; the plain plan is held to
        # the same tile so that the two compute y in the same order
        with env_var("CONV3D_STREAMK", split), env_var("CONV3D_DYNAMIC", dynamic), \
                env_var("CONV3D_TILE", None if extra else "m256n256k64ps"):
            plan = c3d.conv3d_plan(conv_desc(shape, flags | extra))
        ws = workspace_for(plan)
        if ws is not None:
            ws.fill_(0xA5)  # stale contents: every statistics slot must be written
        buf, y = guarded_empty(out_dims(shape), dt)
        c3d.conv3d_forward(plan, dev(d["x"]), dev(d["w"]), dev(d["b"]), None if res is None else dev(res), y, ws)
        torch.cuda.synchronize()
        check_guards(buf)
        out.append((y, plan, ws))
    (ys, ps, wss), (yp, pp, _) = out
    assert ps.info().kernel_name == pp.info().kernel_name and ps.info().split_tiles == pp.info().split_tiles
    return ys, yp, ps, wss


def gn_from_stats(y, plan, ws, n, thw, c, groups, gamma, beta, silu=True, bf16=False):
    st, slots = c3d.gn_stats_view(plan, ws)
    gws = torch.empty(c3d.groupnorm_silu_from_stats_workspace(n, c, groups), dtype=torch.uint8, device="cuda:0")
    buf, out = guarded_empty(tuple(y.shape), y.dtype)
    c3d.groupnorm_silu_from_stats(y, dev(gamma), dev(beta), out, n, thw, c, groups, 1e-6, silu, st, slots, gws,
                                  bf16=bf16)
    torch.cuda.synchronize()
    check_guards(buf)
    return out


CASES = [  # (shape, groups, residual, split, dynamic, dtype[, extra flags])
    (ConvShape(1, 2, 16, 32, 64, 256), 32, False, "0", "0", "f16"),     # whole tiles, static schedule
    (ConvShape(1, 2, 16, 32, 64, 256), 32, False, "1", "0", "f16"),     # every tile split: the fixup's statistics
    (ConvShape(1, 4, 16, 64, 64, 256), 32, True, None, "1", "f16"),     # one workgroup per CU, a residual
    (ConvShape(2, 3, 8, 32, 128, 128), 16, False, None, None, "f16"),   # two samples, half the channel tile
    (ConvShape(1, 2, 8, 64, 72, 384), 24, True, "1", "0", "f16"),       # Cin tail, 1.5 channel tiles, split
    (ConvShape(1, 2, 32, 32, 64, 512), 16, False, "0", "1", "f16"),     # 32-channel groups (4 chunks each)
    (ConvShape(1, 2, 16, 32, 64, 256), 32, True, None, None, "bf16"),   # bf16
    # one frame through the general path (the T=1 fold writes no statistics)
    (ConvShape(1, 1, 16, 32, 64, 256), 32, False, None, None, "f16", c3d.CONV3D_F_NO_T1_FASTPATH),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_conv_gn_stats_small(case):
    s, groups, with_res, split, dynamic, dtype = CASES[case][:6]
    extra = CASES[case][6] if len(CASES[case]) > 6 else 0
    bf16 = dtype == "bf16"
    d = workloads.conv_inputs(s, 1500 + case, dtype=dtype)
    od = out_dims(s)
    res = workloads.normal_f16(np.random.SeedSequence(1600 + case), od, dtype=dtype) if with_res else None
    ys, yp, plan, ws = conv_with_stats(s, d, res, split, dynamic, bf16, extra)
    assert torch.equal(ys.view(torch.int16), yp.view(torch.int16)), "the statistics changed y"
    g = workloads.gn_inputs(1, (1, 1, 1), s.cout, 1700 + case, dtype=dtype)
    n, thw = s.n, od[1] * od[2] * od[3]
    out = gn_from_stats(ys, plan, ws, n, thw, s.cout, groups, g["gamma"], g["beta"], bf16=bf16)
    yh = host_bits(ys) if bf16 else ys.cpu().numpy()
    ref = oracle.groupnorm_silu(f64(yh), f64(g["gamma"]), f64(g["beta"]), groups, 1e-6, True)
    got = f64(host_bits(out)) if bf16 else out.cpu().numpy()
    assert_gn_close(got, ref, "GN from conv statistics, case %d" % case, ulp=ulp_bf16 if bf16 else None)


def test_from_stats_without_silu_and_in_place():
    s = ConvShape(1, 2, 16, 32, 64, 128)
    d = workloads.conv_inputs(s, 1520)
    ys, _, plan, ws = conv_with_stats(s, d)
    g = workloads.gn_inputs(1, (1, 1, 1), s.cout, 1720)
    yh = ys.cpu().numpy()
    od = out_dims(s)
    thw = od[1] * od[2] * od[3]
    out = gn_from_stats(ys, plan, ws, 1, thw, s.cout, 8, g["gamma"], g["beta"], silu=False)
    ref = oracle.groupnorm_silu(f64(yh), f64(g["gamma"]), f64(g["beta"]), 8, 1e-6, False)
    assert_gn_close(out.cpu().numpy(), ref, "no SiLU")
    st, slots = c3d.gn_stats_view(plan, ws)
    gws = torch.empty(c3d.groupnorm_silu_from_stats_workspace(1, s.cout, 8), dtype=torch.uint8, device="cuda:0")
    c3d.groupnorm_silu_from_stats(ys, dev(g["gamma"]), dev(g["beta"]), ys, 1, thw, s.cout, 8, 1e-6, True, st, slots,
                                  gws)
    torch.cuda.synchronize()
    ref = oracle.groupnorm_silu(f64(yh), f64(g["gamma"]), f64(g["beta"]), 8, 1e-6, True)
    assert_gn_close(ys.cpu().numpy(), ref, "in place")


def test_decoder_block_conv_gn_stats_full_size():
    # the block's first conv (17 x 128 x 128, 256 -> 256: 1024 whole tiles and
    # 64 split ones) and the block's second GroupNorm from its statistics,
    # every output against the oracle's GroupNorm of the GPU's conv output
    d = workloads.workload_inputs(4)
    s = d["shape"]
    cd = {"x": d["x"], "w": d["w1"], "b": d["b1"]}
    ys, yp, plan, ws = conv_with_stats(s, cd)
    assert plan.info().split_tiles > 0
    assert torch.equal(ys.view(torch.int16), yp.view(torch.int16))
    thw = s.t * s.h * s.w
    out = gn_from_stats(ys, plan, ws, 1, thw, s.cout, 32, d["gamma2"], d["beta2"])
    ref = oracle.groupnorm_silu(ys.cpu().numpy(), d["gamma2"], d["beta2"], 32, 1e-6, True)
    assert_gn_close(out.cpu().numpy(), ref, "GN2 from conv1's statistics, 17x128x128x256")


def test_decoder_block_with_gn2_from_conv1_statistics_end_to_end():
    # GN1+SiLU -> conv1 (with statistics) -> GN2+SiLU from them -> conv2 + x:
    # the second GroupNorm within the GroupNorm bound of the oracle's GroupNorm
    # of the GPU's conv1 output, and the block's output against the all-fp64
    # oracle block under the six-launch block's end-to-end gate (relative L2)
    s = ConvShape(1, 4, 16, 64, 256, 256)
    d = workloads.block_inputs(s, 1410)
    p = {k: dev(d[k]) for k in ("gamma1", "beta1", "w1", "b1", "gamma2", "beta2", "w2", "b2")}
    x = dev(d["x"])
    thw = s.t * s.h * s.w
    flags = c3d.CONV3D_F_BIAS
    p1 = c3d.conv3d_plan(conv_desc(s, flags | c3d.CONV3D_F_GN_STATS))
    p2 = c3d.conv3d_plan(conv_desc(s, flags | c3d.CONV3D_F_RESIDUAL))
    ws1, ws2 = workspace_for(p1), workspace_for(p2)
    gws = torch.empty(c3d.groupnorm_silu_workspace(1, thw, 256, 32), dtype=torch.uint8, device="cuda:0")
    sws = torch.empty(c3d.groupnorm_silu_from_stats_workspace(1, 256, 32), dtype=torch.uint8, device="cuda:0")
    a1, c1, a2, out = (torch.empty_like(x) for _ in range(4))
    st, slots = c3d.gn_stats_view(p1, ws1)
    c3d.groupnorm_silu(x, p["gamma1"], p["beta1"], a1, 1, thw, 256, 32, 1e-6, True, gws)
    c3d.conv3d_forward(p1, a1, p["w1"], p["b1"], None, c1, ws1)
    c3d.groupnorm_silu_from_stats(c1, p["gamma2"], p["beta2"], a2, 1, thw, 256, 32, 1e-6, True, st, slots, sws)
    c3d.conv3d_forward(p2, a2, p["w2"], p["b2"], x, out, ws2)
    torch.cuda.synchronize()
    c1h = c1.cpu().numpy()
    ref2 = oracle.groupnorm_silu(c1h, d["gamma2"], d["beta2"], 32, 1e-6, True)
    assert_gn_close(a2.cpu().numpy(), ref2, "GN2 from conv1's statistics")
    ref = oracle.decoder_block(d["x"], (d["gamma1"], d["beta1"]), (d["w1"], d["b1"]),
                               (d["gamma2"], d["beta2"]), (d["w2"], d["b2"]), groups=32,
                               eps=1e-6, pads=s.pads, tmode=s.tmode)
    o = out.cpu().numpy().astype(np.float64)
    rel = np.linalg.norm(o - ref) / np.linalg.norm(ref)
    print("decoder block (GN2 from conv1's statistics) end-to-end relative L2 error: %.3e" % rel)
    assert rel <= 1e-2
