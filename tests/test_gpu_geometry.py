"""GPU parity over kernel geometries beyond 3x3x3 and 1x1x1.

Kernels with kt > 3 take the general gather (offsets recomputed per K-iteration,
30-bit window offsets); kt <= 3 the tabulated one.  Covered: kt = 4, 5, 7
(causal replicate, causal zero, symmetric and asymmetric temporal padding),
spatial extents 5 and 7, even extents (one more output row than input rows),
the T=1 fold at kt = 5 in both temporal modes, and the K split on the general
gather.  Ternary data gives exact integer sums (bit-exact against the oracle);
random data is held to the conv bound of tests/helpers.py.
"""
import numpy as np
import pytest

import convolution_implicit_gemm_amd as c3d
import oracle
import workloads
from workloads import ConvShape, TPAD_REPLICATE as R, TPAD_ZERO as Z

from helpers import assert_conv_close, run_conv

pytestmark = pytest.mark.gpu

CASES = [
    ConvShape(1, 6, 9, 11, 64, 48, kt=5, pad_t_front=4, pad_t_back=0, tmode=R),
    ConvShape(2, 5, 8, 10, 40, 72, kt=5, pad_t_front=2, pad_t_back=2, tmode=Z),
    ConvShape(1, 4, 12, 13, 64, 64, kt=4, kh=5, kw=7, pad_t_front=1, pad_t_back=2, pad_h=2, pad_w=3, tmode=Z),
    ConvShape(1, 3, 16, 15, 32, 64, kt=1, kh=7, kw=7, pad_t_front=0, pad_t_back=0, pad_h=3, pad_w=3, tmode=Z),
    ConvShape(1, 9, 6, 7, 64, 32, kt=7, kh=1, kw=1, pad_t_front=6, pad_t_back=0, pad_h=0, pad_w=0, tmode=R),
    ConvShape(1, 4, 10, 12, 64, 64, kt=3, kh=5, kw=5, pad_h=2, pad_w=2),
    ConvShape(1, 5, 9, 9, 48, 40, kt=2, kh=2, kw=2, pad_t_front=1, pad_t_back=0, pad_h=1, pad_w=0, tmode=Z),
    ConvShape(1, 7, 8, 8, 64, 64, kt=6, kh=3, kw=3, pad_t_front=3, pad_t_back=2, tmode=R),
]
TILES = [None, "m256n256k64s2a3w8", "m128n128k64s2a3w4", "m128n32k32s2w4"]


def ternary(shape, seed):
    return workloads.ternary_f16(np.random.SeedSequence(seed), shape)


def small_ints(n, seed):
    return np.random.default_rng(seed).integers(-2, 3, n).astype(np.float16)


def oracle_of(s, x, w, b=None):
    return oracle.conv3d(x.astype(np.float64), w.astype(np.float64), None if b is None else b.astype(np.float64),
                         None, s.pads, s.tmode)


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("case", range(len(CASES)))
def test_geometry_ternary_bit_exact(case, tile):
    s = CASES[case]
    x, w, b = ternary(s.x_shape, 3000 + case), ternary(s.w_shape, 3100 + case), small_ints(s.cout, 3200 + case)
    y, info = run_conv(s, x, w, b, tile=tile)
    assert info.path == c3d.CONV3D_PATH_GENERAL
    ref, _ = oracle_of(s, x, w, b)
    assert np.array_equal(y.astype(np.float64), ref), info.kernel_name


@pytest.mark.parametrize("case", range(len(CASES)))
def test_geometry_random_within_bound(case):
    s = CASES[case]
    d = workloads.conv_inputs(s, 3300 + case)
    y, _ = run_conv(s, d["x"], d["w"], d["b"])
    ref, mag = oracle_of(s, d["x"], d["w"], d["b"])
    assert_conv_close(y, ref, mag, str(s))


@pytest.mark.parametrize("tmode", [R, Z])
def test_first_frame_fold_kt5(tmode):
    s = ConvShape(1, 1, 20, 18, 64, 64, kt=5, pad_t_front=4, pad_t_back=0, tmode=tmode)
    x, w, b = ternary(s.x_shape, 3400 + tmode), ternary(s.w_shape, 3410 + tmode), small_ints(s.cout, 3420)
    yf, info = run_conv(s, x, w, b)
    assert info.path == c3d.CONV3D_PATH_T1_FOLD
    yg, ig = run_conv(s, x, w, b, flags=c3d.CONV3D_F_NO_T1_FASTPATH)
    assert ig.path == c3d.CONV3D_PATH_GENERAL
    ref, _ = oracle_of(s, x, w, b)
    assert np.array_equal(yf.astype(np.float64), ref) and np.array_equal(yg, yf)
    d = workloads.conv_inputs(s, 3430 + tmode)
    y, _ = run_conv(s, d["x"], d["w"], d["b"])
    ref, mag = oracle_of(s, d["x"], d["w"], d["b"])
    assert_conv_close(y, ref, mag, "fold kt=5")


def test_k_split_on_the_general_gather():
    s = CASES[0]
    x, w, b = ternary(s.x_shape, 3500), ternary(s.w_shape, 3501), small_ints(s.cout, 3502)
    y1, i1 = run_conv(s, x, w, b, tile="m256n256k64s2a3w8", split="1")
    assert i1.split_tiles > 0 and i1.split_pieces >= 2
    ref, _ = oracle_of(s, x, w, b)
    assert np.array_equal(y1.astype(np.float64), ref)


DEGENERATE = [
    ConvShape(1, 1, 1, 1, 8, 8),                                   # one voxel (T=1: folded)
    ConvShape(2, 1, 1, 1, 16, 24, tmode=Z),                        # one voxel per sample, zero-causal fold
    ConvShape(1, 5, 1, 37, 16, 8),                                 # one-row frames: only r = 1 reads
    ConvShape(1, 4, 29, 1, 8, 16),                                 # one-column frames
    ConvShape(1, 5, 6, 7, 8, 8),                                   # the fewest channels
    ConvShape(1, 3, 3, 3, 16, 8, pad_t_front=0, pad_t_back=0, pad_h=0, pad_w=0, tmode=Z),  # one output voxel
]


@pytest.mark.parametrize("case", range(len(DEGENERATE)))
def test_degenerate_shapes_bit_exact(case):
    s = DEGENERATE[case]
    x, w, b = ternary(s.x_shape, 3600 + case), ternary(s.w_shape, 3610 + case), small_ints(s.cout, 3620 + case)
    ref, _ = oracle_of(s, x, w, b)
    y, info = run_conv(s, x, w, b)
    assert np.array_equal(y.astype(np.float64), ref), info.kernel_name
    yg, ig = run_conv(s, x, w, b, flags=c3d.CONV3D_F_NO_T1_FASTPATH)
    assert ig.path == c3d.CONV3D_PATH_GENERAL and np.array_equal(yg, y)
