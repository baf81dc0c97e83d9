"""GPU parity of the bf16 variant (CONV3D_F_BF16, groupnorm_silu_bf16) against the fp64 oracle.

bf16 operands are decoded exactly (oracle.bf16_to_f64) and the oracle runs in
fp64 as for fp16.  Exact cases: every partial sum of a ternary conv is a small
integer, exact in fp32, so the bf16 output is that integer rounded once to
nearest even, computed on the host from the oracle's value.  Other cases use
the bounds of tests/helpers.py with the bf16 ulp: 2e-3*S + ulp_bf16 for the
conv, (2e-3 + 2^-8)*S + ulp_bf16 on the T=1 fold path (the folded bf16 weights
carry one rounding of at most 2^-8 relative), 1e-3|ref| + 2^-14 + ulp_bf16 for
GroupNorm.
"""
import numpy as np
import pytest
import torch

import convolution_implicit_gemm_amd as c3d
import oracle
import workloads
from workloads import ConvShape, TPAD_ZERO as Z

from helpers import (BF16_FOLD_REL, assert_conv_close, assert_gn_close, check_guards, conv_desc, dev, edge_voxels,
                     guarded_empty, host_bits, out_dims, run_conv, sample_points, tile_names,
                     ulp_bf16, workspace_for)

pytestmark = pytest.mark.gpu

f64 = oracle.bf16_to_f64


def ternary_bf16(shape, seed):
    v = np.random.default_rng(seed).integers(-1, 2, size=shape).astype(np.float32)
    return workloads.to_bf16(v)


def oracle_full(shape, x, w, b=None, res=None):
    return oracle.conv3d(f64(x), f64(w), None if b is None else f64(b), None if res is None else f64(res),
                         shape.pads, shape.tmode)


def rounded(ref):
    """The exact (integer) reference rounded once to bf16 bits."""
    return workloads.to_bf16(np.asarray(ref, dtype=np.float32))


EXACT = [
    ConvShape(2, 3, 10, 13, 64, 72),
    ConvShape(2, 3, 10, 13, 40, 72, pad_t_front=1, pad_t_back=1, tmode=Z),
]


@pytest.mark.parametrize("tile", tile_names())
@pytest.mark.parametrize("case", range(len(EXACT)))
def test_bf16_ternary_bit_exact_every_tile(tile, case):
    s = EXACT[case]
    x, w = ternary_bf16(s.x_shape, 110 + case), ternary_bf16(s.w_shape, 120 + case)
    b = workloads.to_bf16(np.random.default_rng(130 + case).integers(-2, 3, s.cout).astype(np.float32))
    y, info = run_conv(s, x, w, b, tile=tile)
    assert info.kernel_name.decode().startswith("conv3d_igemm_" + tile)
    ref, _ = oracle_full(s, x, w, b)
    assert np.array_equal(y, rounded(ref)), tile


RANDOM = [
    ConvShape(2, 3, 5, 7, 8, 8),
    ConvShape(1, 3, 6, 9, 56, 16, pad_t_front=1, pad_t_back=1, tmode=Z),
    ConvShape(1, 6, 17, 23, 128, 136),
    ConvShape(1, 4, 18, 20, 256, 256),
]


@pytest.mark.parametrize("case", range(len(RANDOM)))
def test_bf16_random_shapes_within_bound(case):
    s = RANDOM[case]
    d = workloads.conv_inputs(s, 700 + case, dtype="bf16")
    y, _ = run_conv(s, d["x"], d["w"], d["b"])
    ref, mag = oracle_full(s, d["x"], d["w"], d["b"])
    assert_conv_close(f64(y), ref, mag, "bf16 " + str(s), ulp=ulp_bf16)


@pytest.mark.parametrize("tmode", [workloads.TPAD_REPLICATE, Z])
def test_bf16_first_frame_fold(tmode):
    s = ConvShape(1, 1, 24, 20, 64, 64, pad_t_front=2, pad_t_back=0, tmode=tmode)
    d = workloads.conv_inputs(s, 720 + tmode, dtype="bf16")
    y, info = run_conv(s, d["x"], d["w"], d["b"])
    assert info.path == c3d.CONV3D_PATH_T1_FOLD
    ref, mag = oracle_full(s, d["x"], d["w"], d["b"])
    assert_conv_close(f64(y), ref, mag, "bf16 fold", rel=BF16_FOLD_REL, ulp=ulp_bf16)
    # ternary weights fold exactly (sums of three small integers), so the
    # folded path equals the general one bit for bit
    x, w = ternary_bf16(s.x_shape, 730), ternary_bf16(s.w_shape, 731)
    yf, _ = run_conv(s, x, w)
    yg, ig = run_conv(s, x, w, flags=c3d.CONV3D_F_NO_T1_FASTPATH)
    assert ig.path == c3d.CONV3D_PATH_GENERAL
    assert np.array_equal(yf, yg)


@pytest.mark.parametrize("cin,cout", [(64, 128), (128, 128), (256, 128), (512, 128), (256, 384)])
def test_bf16_pointwise(cin, cout):
    s = ConvShape(2, 3, 9, 10, cin, cout, kt=1, kh=1, kw=1, pad_t_front=0, pad_t_back=0, pad_h=0, pad_w=0,
                  tmode=Z)
    x, w = ternary_bf16(s.x_shape, 740 + cin + cout), ternary_bf16(s.w_shape, 741 + cin + cout)
    y, info = run_conv(s, x, w)
    assert info.kernel_name.decode().startswith("conv1x1_stream")
    ref, _ = oracle_full(s, x, w)
    assert np.array_equal(y, rounded(ref))
    d = workloads.conv_inputs(s, 750 + cin + cout, dtype="bf16")
    res = workloads.normal_f16(np.random.SeedSequence(751 + cin + cout), out_dims(s), dtype="bf16")
    y, _ = run_conv(s, d["x"], d["w"], d["b"], res=res)
    ref, mag = oracle_full(s, d["x"], d["w"], d["b"], res)
    assert_conv_close(f64(y), ref, mag, "bf16 pointwise + residual", ulp=ulp_bf16)


def test_bf16_k_split_matches_whole_tiles():
    s = ConvShape(1, 3, 20, 24, 64, 96)
    x, w = ternary_bf16(s.x_shape, 760), ternary_bf16(s.w_shape, 761)
    y1, i1 = run_conv(s, x, w, tile="m256n256k64s2a3w8", split="1")
    assert i1.split_tiles > 0
    y0, _ = run_conv(s, x, w, tile="m256n256k64s2a3w8", split="0")
    ref, _ = oracle_full(s, x, w)
    assert np.array_equal(y1, rounded(ref)) and np.array_equal(y0, y1)
    d = workloads.conv_inputs(s, 762, dtype="bf16")
    res = workloads.normal_f16(np.random.SeedSequence(763), out_dims(s), dtype="bf16")
    y, info = run_conv(s, d["x"], d["w"], d["b"], res=res, tile="m256n256k64s2a3w8", split="1")
    assert info.split_tiles > 0
    ref, mag = oracle_full(s, d["x"], d["w"], d["b"], res)
    assert_conv_close(f64(y), ref, mag, "bf16 split + residual", ulp=ulp_bf16)


def test_bf16_causal_512_full_size_sampled():
    s = workloads.CAUSAL_512
    d = workloads.conv_inputs(s, 1001, dtype="bf16")
    y, info = run_conv(s, d["x"], d["w"], d["b"])
    od = out_dims(s)
    m, co = sample_points(od[0] * od[1] * od[2] * od[3], s.cout, 4000, 17, edge_voxels(od))
    ref, mag = oracle.conv3d_points(f64(d["x"]), f64(d["w"]), f64(d["b"]), None, s.pads, s.tmode, m, co)
    assert_conv_close(f64(y.reshape(-1, s.cout)[m, co]), ref, mag, "bf16 causal 512", ulp=ulp_bf16)


GN_CASES = [  # (n, thw_shape, c, groups, mean, std)
    (1, (3, 5, 7), 64, 8, 0.0, 1.0),
    (2, (2, 9, 9), 256, 32, 0.0, 1.0),
    (1, (1, 1, 3), 512, 32, 0.0, 1.0),
    (1, (2, 32, 32), 256, 32, 100.0, 1.0),
]


def gn_bf16(x_bits, gamma, beta, groups, silu=True):
    n, c = x_bits.shape[0], x_bits.shape[-1]
    thw = int(np.prod(x_bits.shape[1:-1]))
    ws = torch.empty(c3d.groupnorm_silu_workspace(n, thw, c, groups), dtype=torch.uint8, device="cuda:0")
    buf, y = guarded_empty(tuple(x_bits.shape), torch.bfloat16)
    c3d.groupnorm_silu_bf16(dev(x_bits), dev(gamma), dev(beta), y, n, thw, c, groups, 1e-6, silu, ws)
    torch.cuda.synchronize()
    check_guards(buf)
    return f64(host_bits(y))


@pytest.mark.parametrize("case", range(len(GN_CASES)))
@pytest.mark.parametrize("silu", [True, False])
def test_bf16_groupnorm_silu(case, silu):
    n, thw, c, g, mean, std = GN_CASES[case]
    d = workloads.gn_inputs(n, thw, c, 880 + case, mean, std, dtype="bf16")
    y = gn_bf16(d["x"], d["gamma"], d["beta"], g, silu)
    ref = oracle.groupnorm_silu(f64(d["x"]), f64(d["gamma"]), f64(d["beta"]), g, 1e-6, silu)
    assert_gn_close(y, ref, "bf16 " + str(GN_CASES[case]), ulp=ulp_bf16)


def test_bf16_decoder_block_end_to_end_small():
    s = ConvShape(1, 3, 16, 16, 256, 256)
    d = workloads.block_inputs(s, 1405, dtype="bf16")
    p = {k: dev(d[k]) for k in ("gamma1", "beta1", "w1", "b1", "gamma2", "beta2", "w2", "b2")}
    thw = s.t * s.h * s.w
    p1 = c3d.conv3d_plan(conv_desc(s, c3d.CONV3D_F_BIAS | c3d.CONV3D_F_BF16))
    p2 = c3d.conv3d_plan(conv_desc(s, c3d.CONV3D_F_BIAS | c3d.CONV3D_F_RESIDUAL | c3d.CONV3D_F_BF16))
    ws = torch.empty(c3d.groupnorm_silu_workspace(1, thw, s.cin, 32), dtype=torch.uint8, device="cuda:0")
    x = dev(d["x"])
    a1, c1, a2, out = (torch.empty_like(x) for _ in range(4))
    c3d.groupnorm_silu_bf16(x, p["gamma1"], p["beta1"], a1, 1, thw, s.cin, 32, 1e-6, True, ws)
    c3d.conv3d_forward(p1, a1, p["w1"], p["b1"], None, c1, workspace_for(p1))
    c3d.groupnorm_silu_bf16(c1, p["gamma2"], p["beta2"], a2, 1, thw, s.cout, 32, 1e-6, True, ws)
    c3d.conv3d_forward(p2, a2, p["w2"], p["b2"], x, out, workspace_for(p2))
    torch.cuda.synchronize()
    got = f64(host_bits(out))
    ref = oracle.decoder_block(f64(d["x"]), (f64(d["gamma1"]), f64(d["beta1"])), (f64(d["w1"]), f64(d["b1"])),
                               (f64(d["gamma2"]), f64(d["beta2"])), (f64(d["w2"]), f64(d["b2"])), groups=32,
                               eps=1e-6, pads=s.pads, tmode=s.tmode)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    print("bf16 decoder block end-to-end relative L2 error: %.3e" % rel)
    assert rel <= 2e-2
