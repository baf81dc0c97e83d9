"""GPU parity of the HIP conv3d path against the fp64 oracle, through the C ABI.

Exact cases (ternary inputs, delta kernels) must match bit for bit: every
partial sum there is a small integer, exact in fp32 and in the fp16 output.
Random cases must satisfy |gpu - ref| <= 2e-3*S + ulp16(ref) (tests/helpers.py).
Full-size workloads are checked at every output channel of whole output
frames (the first frames, where the causal front padding acts, and the last)
and of a seeded 1% of all output voxels, which the oracle computes one by one;
the 512-channel workload and the first-frame fold are checked in full.
"""
import dataclasses

import numpy as np
import pytest
import torch

import convolution_implicit_gemm_amd as c3d
import oracle
import workloads
from workloads import ConvShape, TPAD_REPLICATE as R, TPAD_ZERO as Z

from helpers import (assert_conv_close, check_voxels, edge_voxels, frame_voxels, out_dims, row_sample, run_conv,
                     sample_points, tile_names, dev)

pytestmark = pytest.mark.gpu


def ternary(shape, seed):
    return np.random.default_rng(seed).integers(-1, 2, size=shape).astype(np.float16)


def oracle_full(shape, x, w, b=None, res=None):
    return oracle.conv3d(x.astype(np.float64), w.astype(np.float64),
                         None if b is None else b.astype(np.float64),
                         None if res is None else res.astype(np.float64), shape.pads, shape.tmode)


def test_library_loads_on_gpu():
    assert torch.cuda.is_available()
    c3d.load_library()
    assert c3d.conv3d_version() >= 100


EXACT_CASES = [
    ConvShape(2, 3, 10, 13, 64, 72),                                     # causal replicate
    ConvShape(2, 3, 10, 13, 40, 72, pad_t_front=1, pad_t_back=1, tmode=Z),  # zero, channel tail
    # three K-iterations: fewer than the load rings are deep
    ConvShape(1, 2, 7, 9, 64, 40, kt=1, kh=1, kw=3, pad_t_front=0, pad_t_back=0, pad_h=0, pad_w=1,
              tmode=Z),
]


@pytest.mark.parametrize("tile", tile_names())
@pytest.mark.parametrize("case", range(len(EXACT_CASES)))
def test_ternary_bit_exact_every_tile(tile, case):
    s = EXACT_CASES[case]
    x = ternary(s.x_shape, 10 + case)
    w = ternary(s.w_shape, 20 + case)
    b = np.random.default_rng(30 + case).integers(-2, 3, s.cout).astype(np.float16)
    y, info = run_conv(s, x, w, b, tile=tile)
    assert info.kernel_name.decode().startswith("conv3d_igemm_" + tile)
    ref, _ = oracle_full(s, x, w, b)
    assert np.array_equal(y.astype(np.float64), ref), tile


@pytest.mark.parametrize("tile", tile_names())
def test_single_k_iteration_every_tile(tile):
    # a 1x1x1 conv on a forced implicit-GEMM tile (instead of the streaming
    # kernel): one K-iteration, so every prefetch past the first re-reads the
    # frozen last stage
    s = ConvShape(1, 2, 5, 6, 64, 32, kt=1, kh=1, kw=1, pad_t_front=0, pad_t_back=0, pad_h=0,
                  pad_w=0, tmode=Z)
    x = ternary(s.x_shape, 40)
    w = ternary(s.w_shape, 41)
    y, info = run_conv(s, x, w, tile=tile)
    assert info.kernel_name.decode().startswith("conv3d_igemm_" + tile)
    ref, _ = oracle_full(s, x, w)
    assert np.array_equal(y.astype(np.float64), ref), tile


def test_delta_kernels_reproduce_input_exactly():
    rng = np.random.default_rng(1)
    for s in (ConvShape(1, 4, 9, 11, 32, 32),
              ConvShape(1, 4, 9, 11, 32, 32, pad_t_front=1, pad_t_back=1, tmode=Z)):
        x = rng.normal(size=s.x_shape).astype(np.float16)
        w = np.zeros(s.w_shape, np.float16)
        for c in range(32):
            w[c, s.pad_t_front, 1, 1, c] = 1.0
        y, _ = run_conv(s, x, w)
        assert np.array_equal(y, x)
        # shifted delta: tap (r, s) = (0, 0) reads (h-1, w-1); zeros at the border
        w2 = np.zeros(s.w_shape, np.float16)
        for c in range(32):
            w2[c, s.pad_t_front, 0, 0, c] = 1.0
        y2, _ = run_conv(s, x, w2)
        e = np.zeros_like(x)
        e[:, :, 1:, 1:] = x[:, :, :-1, :-1]
        assert np.array_equal(y2, e)
    # causal tap 0 reads frame max(t-2, 0)
    s = ConvShape(1, 5, 6, 7, 16, 16)
    x = rng.normal(size=s.x_shape).astype(np.float16)
    w = np.zeros(s.w_shape, np.float16)
    for c in range(16):
        w[c, 0, 1, 1, c] = 1.0
    y, _ = run_conv(s, x, w)
    for t in range(5):
        assert np.array_equal(y[0, t], x[0, max(t - 2, 0)])


def test_all_ones_closed_form_exact():
    s = ConvShape(1, 4, 7, 9, 512, 64)
    y, _ = run_conv(s, np.ones(s.x_shape, np.float16), np.ones(s.w_shape, np.float16))
    ref, _ = oracle_full(s, np.ones(s.x_shape, np.float16), np.ones(s.w_shape, np.float16))
    assert np.array_equal(y.astype(np.float64), ref)  # interior 27*512 = 13,824


@pytest.mark.parametrize("tmode", [R, Z])
def test_first_frame_fold_path(tmode):
    s = ConvShape(1, 1, 12, 20, 64, 48, tmode=tmode)
    x = ternary(s.x_shape, 40)
    w = ternary(s.w_shape, 41)
    b = np.random.default_rng(42).integers(-2, 3, s.cout).astype(np.float16)
    y, info = run_conv(s, x, w, b)
    assert info.path == c3d.CONV3D_PATH_T1_FOLD
    assert info.gemm_k == 9 * 64
    ref, _ = oracle_full(s, x, w, b)
    assert np.array_equal(y.astype(np.float64), ref)
    yg, info_g = run_conv(s, x, w, b, flags=c3d.CONV3D_F_NO_T1_FASTPATH)
    assert info_g.path == c3d.CONV3D_PATH_GENERAL
    assert np.array_equal(yg, y)


def test_pointwise_path():
    s = ConvShape(2, 3, 9, 10, 256, 128, kt=1, kh=1, kw=1, pad_t_front=0, pad_t_back=0, pad_h=0,
                  pad_w=0, tmode=Z)
    x = ternary(s.x_shape, 50)
    w = ternary(s.w_shape, 51)
    y, info = run_conv(s, x, w)
    assert info.path == c3d.CONV3D_PATH_POINTWISE
    ref, _ = oracle_full(s, x, w)
    assert np.array_equal(y.astype(np.float64), ref)


RANDOM_CASES = [
    ConvShape(2, 3, 5, 7, 8, 8),
    ConvShape(1, 2, 9, 6, 16, 24, tmode=Z),
    ConvShape(2, 1, 11, 4, 24, 40),
    ConvShape(1, 3, 6, 9, 56, 16, pad_t_front=1, pad_t_back=1, tmode=Z),
    ConvShape(1, 4, 8, 8, 32, 32, kt=1, pad_t_front=0, pad_t_back=0),
    ConvShape(1, 5, 7, 7, 32, 48, kh=1, kw=1, pad_h=0, pad_w=0),
    ConvShape(1, 3, 6, 6, 64, 64, pad_t_front=0, pad_t_back=0, pad_h=0, pad_w=0, tmode=Z),
    ConvShape(1, 6, 17, 23, 128, 136),
]


@pytest.mark.parametrize("case", range(len(RANDOM_CASES)))
def test_random_shapes_within_bound(case):
    s = RANDOM_CASES[case]
    d = workloads.conv_inputs(s, 500 + case)
    y, _ = run_conv(s, d["x"], d["w"], d["b"])
    ref, mag = oracle_full(s, d["x"], d["w"], d["b"])
    assert_conv_close(y, ref, mag, str(s))


def test_residual_is_fused_into_the_epilogue():
    s = ConvShape(1, 3, 10, 12, 64, 64)
    d = workloads.conv_inputs(s, 600)
    res = workloads.normal_f16(np.random.SeedSequence(601), out_dims(s))
    y, _ = run_conv(s, d["x"], d["w"], d["b"], res=res)
    ref, mag = oracle_full(s, d["x"], d["w"], d["b"], res)
    assert_conv_close(y, ref, mag, "residual")


def test_repeat_runs_are_bitwise_identical():
    s = ConvShape(1, 3, 16, 16, 256, 256)
    d = workloads.conv_inputs(s, 700)
    y1, _ = run_conv(s, d["x"], d["w"], d["b"])
    y2, _ = run_conv(s, d["x"], d["w"], d["b"])
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))


def test_small_zero_padded_workload_full():
    d = workloads.workload_inputs(0)
    s = d["shape"]
    y, _ = run_conv(s, d["x"], d["w"], d["b"])
    ref, mag = oracle_full(s, d["x"], d["w"], d["b"])
    assert_conv_close(y, ref, mag, "T=5 16x16 32->32 zero padding")


def check_sampled(s, d, y, count=6000, seed=0, w=None, b=None, res=None):
    w = d["w"] if w is None else w
    b = d["b"] if b is None else b
    od = out_dims(s)
    m_total = od[0] * od[1] * od[2] * od[3]
    m, co = sample_points(m_total, s.cout, count, seed, edge_voxels(od))
    ref, mag = oracle.conv3d_points(d["x"], w, b, res, s.pads, s.tmode, m, co)
    got = y.reshape(-1, s.cout)[m, co]
    return assert_conv_close(got, ref, mag, str(s))


def test_causal_512_full_size_every_output():
    # 36,864 voxels x 512 channels: the whole output against the oracle
    d = workloads.workload_inputs(1)
    s = d["shape"]
    y, info = run_conv(s, d["x"], d["w"], d["b"], keep_device=True)
    od = out_dims(s)
    check_voxels(s, d["x"].astype(np.float64), d["w"], d["b"], y, np.arange(od[1] * od[2] * od[3]),
                 what="causal 512, every output")


def test_causal_256_full_size_frames_rows_and_first_frame():
    d = workloads.workload_inputs(2)
    s = d["shape"]
    y, _ = run_conv(s, d["x"], d["w"], d["b"], keep_device=True)
    x64 = d["x"].astype(np.float64)
    od = out_dims(s)
    # the first two output frames (the replicated front), the last, and a seeded 1% of all voxels,
    # every channel
    vox = np.union1d(frame_voxels(od, [0, 1, od[1] - 1]), row_sample(od, 0.01, 12))
    check_voxels(s, x64, d["w"], d["b"], y, vox, what="causal 256, frames 0, 1, T-1 and 1% of voxels")
    check_sampled(s, d, y.cpu().numpy(), seed=12)
    # first-frame case: frame 0 alone, through the fold path; every output
    s1 = dataclasses.replace(s, t=1)
    x1 = np.ascontiguousarray(d["x"][:, :1])
    y1, info = run_conv(s1, x1, d["w"], d["b"], keep_device=True)
    assert info.path == c3d.CONV3D_PATH_T1_FOLD
    check_voxels(s1, x1.astype(np.float64), d["w"], d["b"], y1, np.arange(s.h * s.w), what="first frame, fold")


def test_channel_changing_stage_full_size_frames_and_rows():
    d = workloads.workload_inputs(3)
    s, s2 = d["shape"], d["shape2"]
    y1, _ = run_conv(s, d["x"], d["w"], d["b"], keep_device=True)
    od = out_dims(s)
    x64 = d["x"].astype(np.float64)
    del d["x"]
    # 3x3x3 512->256: frames 0, 1, 2 (the replicated front) and T-1 at every channel, plus a
    # seeded 1% of all output voxels at every channel
    check_voxels(s, x64, d["w"], d["b"], y1, frame_voxels(od, [0, 1, 2, od[1] - 1]),
                 what="3x3x3 512->256 frames 0, 1, 2, T-1")
    check_voxels(s, x64, d["w"], d["b"], y1, row_sample(od, 0.01, 14), what="3x3x3 512->256, 1% of voxels")
    del x64
    # 1x1x1 stage on the GPU's own fp16 output (per-stage parity on identical inputs)
    y2, info = run_conv(s2, y1, d["w2"], d["b2"], keep_device=True)
    assert info.path == c3d.CONV3D_PATH_POINTWISE
    y1h = y1.cpu().numpy().astype(np.float64)
    od2 = out_dims(s2)
    vox = np.union1d(frame_voxels(od2, [0, 1, od2[1] - 1]), row_sample(od2, 0.01, 15))
    check_voxels(s2, y1h, d["w2"], d["b2"], y2, vox, what="1x1x1 256->128, frames 0, 1, T-1 and 1% of voxels")


PW_CASES = [(64, 32), (128, 160), (256, 128), (512, 96), (256, 256), (512, 512), (64, 288)]


@pytest.mark.parametrize("cin,cout", PW_CASES)
def test_streaming_pointwise_exact(cin, cout):
    s = ConvShape(2, 3, 5, 7, cin, cout, kt=1, kh=1, kw=1, pad_t_front=0, pad_t_back=0, pad_h=0,
                  pad_w=0, tmode=Z)  # M = 210 voxels: a ragged last tile
    x = ternary(s.x_shape, 60 + cin)
    w = ternary(s.w_shape, 61 + cout)
    b = np.random.default_rng(62).integers(-2, 3, s.cout).astype(np.float16)
    y, info = run_conv(s, x, w, b)
    assert info.kernel_name.decode() == "conv1x1_stream_cin%d" % cin
    ref, _ = oracle_full(s, x, w, b)
    assert np.array_equal(y.astype(np.float64), ref)
    # the general implicit-GEMM kernel, forced by naming a tile, gives the same bits here
    yg, info_g = run_conv(s, x, w, b, tile="m256n128k64s2a3w4")
    assert info_g.kernel_name.decode().startswith("conv3d_igemm_")
    assert np.array_equal(yg, y)


# Several tiles per persistent block (the input ring wraps) and a ragged last
# tile: M = 3*181*191 = 103713 voxels, above 3 tiles per block for every
# configuration.  (cin, cout, residual): 4- and 8-wave blocks, the 32-row
# tiles at 512 input channels, and the residual epilogue.
PW_RING_CASES = [(64, 64, False), (128, 64, False), (256, 128, False), (256, 128, True), (256, 256, False),
                 (512, 128, True), (512, 256, False)]


@pytest.mark.parametrize("cin,cout,with_res", PW_RING_CASES)
def test_streaming_pointwise_ring_wraps_exact(cin, cout, with_res):
    s = ConvShape(1, 3, 181, 191, cin, cout, kt=1, kh=1, kw=1, pad_t_front=0, pad_t_back=0, pad_h=0,
                  pad_w=0, tmode=Z)
    x = ternary(s.x_shape, 70 + cin)
    w = ternary(s.w_shape, 71 + cout)
    b = np.random.default_rng(72).integers(-2, 3, s.cout).astype(np.float16)
    res = np.random.default_rng(73).integers(-3, 4, out_dims(s)).astype(np.float16) if with_res else None
    y, info = run_conv(s, x, w, b, res=res)
    assert info.kernel_name.decode() == "conv1x1_stream_cin%d" % cin
    m_total = s.n * s.t * s.h * s.w
    assert m_total // info.tile_m > 3 * info.grid
    rows = np.unique(np.concatenate([np.arange(8), np.arange(m_total - 40, m_total),
                                     np.random.default_rng(74).integers(0, m_total, 192)]))
    m = np.repeat(rows, cout)
    co = np.tile(np.arange(cout), rows.size)
    ref, _ = oracle.conv3d_points(x, w, b, res, s.pads, s.tmode, m, co)
    got = y.reshape(-1, cout)[m, co]
    assert np.array_equal(got.astype(np.float64), ref), "%d of %d sampled outputs differ" % (
        int((got.astype(np.float64) != ref).sum()), m.size)


def test_streaming_pointwise_bias_residual_bound():
    s = ConvShape(1, 4, 9, 11, 256, 128, kt=1, kh=1, kw=1, pad_t_front=0, pad_t_back=0, pad_h=0,
                  pad_w=0, tmode=Z)
    d = workloads.conv_inputs(s, 640)
    res = workloads.normal_f16(np.random.SeedSequence(641), out_dims(s))
    y, info = run_conv(s, d["x"], d["w"], d["b"], res=res)
    assert info.kernel_name.decode().startswith("conv1x1_stream")
    ref, mag = oracle_full(s, d["x"], d["w"], d["b"], res)
    assert_conv_close(y, ref, mag, "pointwise + residual")


@pytest.mark.parametrize("tile", ["m256n256k64s2w8", "m256n256k64s2a3w8", "m256n256k64s2a3w4",
                                  "m256n256k64s2w4", "m256n128k64s2a3w4"])
def test_k_split_matches_whole_tiles_exactly(tile):
    s = ConvShape(1, 3, 20, 24, 64, 96)
    x = ternary(s.x_shape, 70)
    w = ternary(s.w_shape, 71)
    b = np.random.default_rng(72).integers(-2, 3, s.cout).astype(np.float16)
    y1, info1 = run_conv(s, x, w, b, tile=tile, split="1")
    assert info1.split_tiles > 0 and info1.split_pieces >= 2
    y0, info0 = run_conv(s, x, w, b, tile=tile, split="0")
    assert info0.split_tiles == 0
    ref, _ = oracle_full(s, x, w, b)
    assert np.array_equal(y1.astype(np.float64), ref)
    assert np.array_equal(y0, y1)


def test_k_split_with_residual_within_bound():
    s = ConvShape(1, 4, 18, 20, 128, 128)
    d = workloads.conv_inputs(s, 650)
    res = workloads.normal_f16(np.random.SeedSequence(651), out_dims(s))
    y, info = run_conv(s, d["x"], d["w"], d["b"], res=res, tile="m256n256k64s2w8", split="1")
    assert info.split_tiles > 0
    ref, mag = oracle_full(s, d["x"], d["w"], d["b"], res)
    assert_conv_close(y, ref, mag, "split K + residual")
