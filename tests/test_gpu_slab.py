"""GPU parity of the row-slab kernel (m256n256k64ps) against the fp64 oracle.

The kernel covers kw = 3 with pw = 1, kt, kh <= 3 and output rows a multiple
of 32 voxels long (tiles of 256 voxels may start inside a row and cross rows,
frames and samples).
Ternary inputs make every partial sum a small integer, so outputs must match
the oracle bit for bit: every row length it takes, both temporal modes, a
channel tail, two samples, an M tail (a last tile past the output), the K
split, bias + residual, bf16, the first-frame fold (kt = 1 after folding), and
the frame-block walk of whole tiles over frame groups and blocks of every
partial size.
"""
import numpy as np
import pytest
import torch

import convolution_implicit_gemm_amd as c3d
import oracle
import workloads
from workloads import ConvShape, TPAD_REPLICATE as R, TPAD_ZERO as Z

from helpers import assert_conv_close, dev, host_bits, out_dims, run_conv

pytestmark = pytest.mark.gpu
TILE = "m256n256k64ps"


def ternary(shape, seed):
    return np.random.default_rng(seed).integers(-1, 2, size=shape).astype(np.float16)


def oracle_full(s, x, w, b=None, res=None):
    f = lambda a: None if a is None else np.asarray(a, dtype=np.float64)
    return oracle.conv3d(f(x), f(w), f(b), f(res), s.pads, s.tmode)


SLAB_CASES = [
    ConvShape(1, 3, 4, 256, 64, 64),                                       # one segment per tile
    ConvShape(1, 3, 6, 128, 64, 96),                                       # two segments, Cout < 256
    ConvShape(2, 3, 8, 64, 72, 64),                                        # four segments, N = 2, channel tail
    ConvShape(1, 2, 8, 32, 40, 264),                                       # eight segments, tail, two column tiles
    ConvShape(1, 3, 4, 512, 16, 32, pad_t_front=1, pad_t_back=1, tmode=Z),  # 256 | W, symmetric zero
    ConvShape(1, 3, 3, 32, 64, 64, pad_t_front=2, tmode=Z),                # M = 288: a partial last tile
    ConvShape(1, 4, 5, 64, 128, 128, kt=1, kh=3, pad_t_front=0),           # kt = 1 (a 2D conv per frame)
    ConvShape(1, 3, 5, 64, 64, 64, kt=2, kh=2, pad_t_front=1, pad_h=1),    # even extents in t and h
    # rows that do not tile 256 voxels: tiles start inside rows, and cross rows,
    # frames and samples
    ConvShape(1, 3, 5, 96, 64, 64),                                        # 96-voxel rows, 480 voxels per frame
    ConvShape(2, 3, 3, 160, 72, 64),                                       # 160-voxel rows, N = 2, channel tail
    ConvShape(1, 2, 4, 320, 64, 128),                                      # 320-voxel rows (longer than a tile)
    ConvShape(1, 2, 3, 224, 64, 64, tmode=Z, pad_t_front=1, pad_t_back=1),  # 224-voxel rows, symmetric zero
]


@pytest.mark.parametrize("case", range(len(SLAB_CASES)))
def test_slab_kernel_ternary_bit_exact(case):
    s = SLAB_CASES[case]
    x = ternary(s.x_shape, 300 + case)
    w = ternary(s.w_shape, 320 + case)
    b = np.random.default_rng(340 + case).integers(-2, 3, s.cout).astype(np.float16)
    y, info = run_conv(s, x, w, b, tile=TILE)
    assert info.kernel_name.decode().startswith("conv3d_igemm_" + TILE)
    ref, _ = oracle_full(s, x, w, b)
    assert np.array_equal(y.astype(np.float64), ref), "%d of %d outputs differ" % (
        int((y.astype(np.float64) != ref).sum()), y.size)


def test_slab_kernel_k_split_exact_and_equal_to_whole_tiles():
    s = ConvShape(1, 3, 8, 128, 64, 96)
    x, w = ternary(s.x_shape, 360), ternary(s.w_shape, 361)
    b = np.random.default_rng(362).integers(-2, 3, s.cout).astype(np.float16)
    y1, i1 = run_conv(s, x, w, b, tile=TILE, split="1")
    assert i1.split_tiles > 0 and i1.split_pieces >= 2
    y0, i0 = run_conv(s, x, w, b, tile=TILE, split="0")
    assert i0.split_tiles == 0
    ref, _ = oracle_full(s, x, w, b)
    assert np.array_equal(y1.astype(np.float64), ref)
    assert np.array_equal(y0, y1)


WALK_CASES = [
    ConvShape(2, 5, 12, 64, 32, 64),      # 3 tiles per frame, 10 frames over two samples: groups of 4, 4, 2 frames
    ConvShape(1, 9, 16, 128, 64, 64),     # 8 tiles per frame, 9 frames: the last group holds one frame
    ConvShape(1, 6, 4, 128, 64, 320),     # 2 tiles per frame and two column tiles: groups of 4, 2 frames
    ConvShape(1, 6, 8, 96, 64, 64),       # 96-voxel rows, 3 tiles per frame: tiles start inside rows
]


@pytest.mark.parametrize("case", range(len(WALK_CASES)))
def test_slab_kernel_frame_block_walk_exact(case):
    # whole tiles only, so every tile goes through the frame-block walk; ternary data, bit-exact
    s = WALK_CASES[case]
    x, w = ternary(s.x_shape, 400 + case), ternary(s.w_shape, 410 + case)
    b = np.random.default_rng(420 + case).integers(-2, 3, s.cout).astype(np.float16)
    y, info = run_conv(s, x, w, b, tile=TILE, split="0")
    assert info.split_tiles == 0
    ref, _ = oracle_full(s, x, w, b)
    assert np.array_equal(y.astype(np.float64), ref), "%d of %d outputs differ" % (
        int((y.astype(np.float64) != ref).sum()), y.size)


DYN_CASES = [
    (ConvShape(1, 9, 16, 128, 64, 64), None),    # whole tiles over 9 frames
    (ConvShape(2, 5, 12, 64, 40, 64), None),     # two samples, channel tail
    (ConvShape(1, 3, 8, 128, 64, 96), "1"),      # every tile split into K-pieces
    (ConvShape(1, 5, 16, 96, 64, 320), None),    # 96-voxel rows, two column tiles
    (ConvShape(1, 9, 64, 128, 64, 64), "0"),     # 288 whole tiles on 256 workgroups: some take two
]


@pytest.mark.parametrize("case", range(len(DYN_CASES)))
def test_slab_kernel_dynamic_schedule_equals_static(case):
    # one workgroup per CU taking tiles (and K-pieces) from counters: the same
    # tiles computed the same way as one workgroup per tile, bit for bit
    from helpers import env_var
    s, split = DYN_CASES[case]
    x, w = ternary(s.x_shape, 430 + case), ternary(s.w_shape, 440 + case)
    b = np.random.default_rng(450 + case).integers(-2, 3, s.cout).astype(np.float16)
    with env_var("CONV3D_DYNAMIC", "1"):
        y1, i1 = run_conv(s, x, w, b, tile=TILE, split=split)
    with env_var("CONV3D_DYNAMIC", "0"):
        y0, i0 = run_conv(s, x, w, b, tile=TILE, split=split)
    assert i1.grid <= 256 and (i1.split_tiles, i1.split_pieces) == (i0.split_tiles, i0.split_pieces)
    ref, _ = oracle_full(s, x, w, b)
    assert np.array_equal(y0.astype(np.float64), ref)
    assert np.array_equal(y1, y0)


def test_slab_kernel_dynamic_schedule_bf16_exact():
    # the bf16 instantiation of the dynamic kernel, whole tiles and K-pieces
    from helpers import env_var
    s = ConvShape(1, 5, 16, 128, 64, 64)
    x = workloads.ternary_f16(np.random.SeedSequence(460), s.x_shape)
    w = workloads.ternary_f16(np.random.SeedSequence(461), s.w_shape)
    to_bf = lambda a: (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    with env_var("CONV3D_DYNAMIC", "1"):
        y1, i1 = run_conv(s, to_bf(x), to_bf(w), tile=TILE, split="1")
    assert i1.grid <= 256 and i1.split_tiles > 0
    ref, _ = oracle_full(s, x, w)
    got = (y1.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(got, ref)


def test_slab_kernel_dynamic_schedule_bias_residual_equals_static():
    # random data with bias and residual: the dynamic schedule computes every
    # tile and K-piece as the static one does, so the outputs agree bit for bit
    from helpers import env_var
    s = ConvShape(1, 9, 16, 128, 128, 64)
    d = workloads.conv_inputs(s, 470)
    res = workloads.normal_f16(np.random.SeedSequence(471), out_dims(s))
    with env_var("CONV3D_DYNAMIC", "1"):
        y1, i1 = run_conv(s, d["x"], d["w"], d["b"], res=res, tile=TILE, split="1")
    with env_var("CONV3D_DYNAMIC", "0"):
        y0, _ = run_conv(s, d["x"], d["w"], d["b"], res=res, tile=TILE, split="1")
    assert i1.grid <= 256
    assert np.array_equal(y1, y0)
    ref, mag = oracle_full(s, d["x"], d["w"], d["b"], res)
    assert_conv_close(y1, ref, mag, "slab kernel, dynamic schedule, bias + residual")


RES_EDGE_CASES = [
    ConvShape(1, 3, 3, 32, 64, 96, pad_t_front=2, tmode=Z),   # M = 288: a last tile of 32 voxels; Cout < 256
    ConvShape(1, 2, 4, 96, 40, 264),                          # tiles inside rows, channel tail, a column tile of 8
]


@pytest.mark.parametrize("case", range(len(RES_EDGE_CASES)))
def test_slab_kernel_residual_edges_exact(case):
    # the epilogue staged through LDS with a residual: rows past the output and
    # channels past Cout are never read or written; ternary data, bit-exact
    s = RES_EDGE_CASES[case]
    x, w = ternary(s.x_shape, 480 + case), ternary(s.w_shape, 482 + case)
    b = np.random.default_rng(484 + case).integers(-2, 3, s.cout).astype(np.float16)
    res = np.random.default_rng(486 + case).integers(-3, 4, out_dims(s)).astype(np.float16)
    y, info = run_conv(s, x, w, b, res=res, tile=TILE, split="0")
    assert info.kernel_name.decode().startswith("conv3d_igemm_" + TILE)
    ref, _ = oracle_full(s, x, w, b, res)
    assert np.array_equal(y.astype(np.float64), ref), "%d of %d outputs differ" % (
        int((y.astype(np.float64) != ref).sum()), y.size)


def test_slab_kernel_random_with_bias_and_residual_within_bound():
    s = ConvShape(1, 5, 16, 128, 256, 256)
    d = workloads.conv_inputs(s, 370)
    res = workloads.normal_f16(np.random.SeedSequence(371), out_dims(s))
    y, info = run_conv(s, d["x"], d["w"], d["b"], res=res, tile=TILE)
    ref, mag = oracle_full(s, d["x"], d["w"], d["b"], res)
    assert_conv_close(y, ref, mag, "slab kernel + residual")
    # the same through a K split: the partials' fixup adds bias and residual
    y2, i2 = run_conv(s, d["x"], d["w"], d["b"], res=res, tile=TILE, split="1")
    assert i2.split_tiles > 0
    assert_conv_close(y2, ref, mag, "slab kernel + residual, K split")


def test_slab_kernel_bf16_ternary_exact():
    s = ConvShape(1, 3, 6, 64, 64, 128)
    x = workloads.ternary_f16(np.random.SeedSequence(380), s.x_shape)
    w = workloads.ternary_f16(np.random.SeedSequence(381), s.w_shape)
    to_bf = lambda a: (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y, info = run_conv(s, to_bf(x), to_bf(w), tile=TILE)
    ref, _ = oracle_full(s, x, w)
    got = (y.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("tmode", [R, Z])
def test_slab_kernel_first_frame_fold_exact(tmode):
    # T = 1: the fold sums the temporal taps and runs a kt = 1 conv, here on the slab kernel
    s = ConvShape(1, 1, 8, 128, 64, 64, tmode=tmode)
    x, w = ternary(s.x_shape, 390 + tmode), ternary(s.w_shape, 392 + tmode)
    y, info = run_conv(s, x, w, tile=TILE)
    assert info.path == c3d.CONV3D_PATH_T1_FOLD
    ref, _ = oracle_full(s, x, w)
    assert np.array_equal(y.astype(np.float64), ref)


def test_slab_kernel_rejects_shapes_it_does_not_cover():
    # rows of 48 voxels are not a multiple of 32: forcing the tile plans nothing
    import os
    from helpers import conv_desc, forced_tile
    with forced_tile(TILE):
        with pytest.raises(c3d.Conv3dError):
            c3d.conv3d_plan(conv_desc(ConvShape(1, 3, 4, 48, 64, 64)))
