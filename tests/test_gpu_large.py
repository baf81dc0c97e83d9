"""GPU parity at the largest tensors and channel counts the library accepts.

Element offsets beyond 2^31 (byte offsets beyond 4 GiB): a conv whose output
has more than 2^31 elements (8 -> 512 channels), and a 512-channel input of
more than 2^31 elements read by the general conv (512 -> 8), by the streaming
1x1x1 kernel (512 -> 64) and by GroupNorm+SiLU.  Channel limits: Cin = 65536
and Cout = 65536.  Input windows above 1 GiB: a 256-channel causal conv on
1024x1024 frames.

Conv data is ternary (values -1, 0, 1, small integer biases): every partial sum
is an integer below 2^24, exact in fp32, so each fp16 output is the exact sum
rounded once to nearest even.  The oracle's fp64 value rounded the same way on
the host must match bit for bit.  Outputs are sampled at random positions, at
every channel of the edge voxels (which include the last one) and at the last
elements of the tensor.  GroupNorm uses the bound of the other GroupNorm tests.
"""
import numpy as np
import pytest
import torch

import convolution_implicit_gemm_amd as c3d
import oracle
import workloads
from workloads import ConvShape, TPAD_REPLICATE as R

from helpers import (assert_gn_close, check_guards, dev, edge_voxels, guarded_empty, out_dims, run_conv,
                     sample_points)

pytestmark = pytest.mark.gpu

BIG = (1, 17, 512, 512)  # 4,456,448 voxels
TWO31 = 1 << 31


def big_shape(cin, cout, k=3):
    if k == 3:
        return ConvShape(*BIG, cin, cout, tmode=R)
    return ConvShape(*BIG, cin, cout, kt=1, kh=1, kw=1, pad_t_front=0, pad_t_back=0, pad_h=0, pad_w=0, tmode=R)


def ternary(shape, seed):
    return workloads.ternary_f16(np.random.SeedSequence(seed), shape)


def small_ints(n, seed):
    return np.random.default_rng(seed).integers(-2, 3, n).astype(np.float16)


@pytest.fixture(scope="module")
def x512():
    """[1, 17, 512, 512, 512] ternary fp16: 2,281,701,376 elements (4.56 GB), host and device."""
    x = ternary(BIG + (512,), 2100)
    return x, dev(x)


def sampled(shape, count, seed):
    """Sampled (m, co): random pairs, every channel of the edge voxels, and the last 64 elements."""
    od = out_dims(shape)
    mt = od[0] * od[1] * od[2] * od[3]
    m, co = sample_points(mt, shape.cout, count, seed, edge_voxels(od))
    last = np.arange(mt * shape.cout - 64, mt * shape.cout)
    return np.concatenate([m, last // shape.cout]), np.concatenate([co, last % shape.cout])


def check_sampled(shape, x_host, w, b, y_dev, m, co, what):
    got = y_dev.view(-1, shape.cout)[torch.from_numpy(m).cuda(), torch.from_numpy(co).cuda()].cpu().numpy()
    ref, _ = oracle.conv3d_points(x_host, w, b, None, shape.pads, shape.tmode, m, co)
    want = ref.astype(np.float16)
    bad = np.flatnonzero(got.view(np.uint16) != want.view(np.uint16))
    assert bad.size == 0, "%s: %d of %d differ; first at voxel %d channel %d: gpu %r exact %r" % (
        what, bad.size, m.size, m[bad[0]], co[bad[0]], got[bad[0]], ref[bad[0]])


def test_output_beyond_2_31_elements():
    s = big_shape(8, 512)
    x, w, b = ternary(s.x_shape, 2101), ternary(s.w_shape, 2102), small_ints(s.cout, 2103)
    y, info = run_conv(s, x, w, b, keep_device=True)
    assert y.numel() > TWO31 and info.path == c3d.CONV3D_PATH_GENERAL
    m, co = sampled(s, 6000, 2104)
    assert int((m * s.cout + co).max()) >= TWO31
    check_sampled(s, x, w, b, y, m, co, "output > 2^31 elements")


def test_input_beyond_2_31_elements(x512):
    x, xd = x512
    s = big_shape(512, 8)
    w, b = ternary(s.w_shape, 2111), small_ints(s.cout, 2112)
    y, info = run_conv(s, xd, w, b, keep_device=True)
    assert xd.numel() > TWO31 and info.path == c3d.CONV3D_PATH_GENERAL
    m, co = sampled(s, 6000, 2113)
    check_sampled(s, x, w, b, y, m, co, "input > 2^31 elements")


def test_streaming_pointwise_input_beyond_2_31_elements(x512):
    x, xd = x512
    s = big_shape(512, 64, k=1)
    w, b = ternary(s.w_shape, 2121), small_ints(s.cout, 2122)
    y, info = run_conv(s, xd, w, b, keep_device=True)
    assert info.kernel_name.decode() == "conv1x1_stream_cin512"
    m, co = sampled(s, 6000, 2123)
    check_sampled(s, x, w, b, y, m, co, "1x1x1, input > 2^31 elements")


def test_groupnorm_silu_beyond_2_31_elements(x512):
    x, xd = x512
    n, thw, c, groups = 1, int(np.prod(BIG[1:])), 512, 32
    rng = np.random.default_rng(2131)
    gamma = rng.normal(1.0, 0.1, c).astype(np.float16)
    beta = rng.normal(0.0, 0.1, c).astype(np.float16)
    ws = torch.empty(c3d.groupnorm_silu_workspace(n, thw, c, groups), dtype=torch.uint8, device="cuda:0")
    buf, y = guarded_empty(xd.shape)
    c3d.groupnorm_silu(xd, dev(gamma), dev(beta), y, n, thw, c, groups, 1e-6, True, ws)
    torch.cuda.synchronize()
    check_guards(buf)
    rs = np.random.default_rng(2132)
    vox = np.concatenate([rs.integers(0, thw, 6000), np.full(c, thw - 1), np.zeros(c, np.int64)])
    ch = np.concatenate([rs.integers(0, c, 6000), np.arange(c), np.arange(c)])
    got = y.view(-1, c)[torch.from_numpy(vox).cuda(), torch.from_numpy(ch).cuda()].cpu().numpy()
    ref, _, _ = oracle.groupnorm_silu_points(x, gamma, beta, groups, vox, ch, 1e-6, True)
    assert_gn_close(got, ref, "GroupNorm+SiLU, 2^31+ elements")


@pytest.mark.parametrize("cin,cout", [(65536, 64), (8, 65536)])
def test_channel_limits_exact(cin, cout):
    s = ConvShape(1, 2, 4, 5, cin, cout, tmode=R)
    x, w, b = ternary(s.x_shape, 2140 + cin), ternary(s.w_shape, 2141 + cout), small_ints(cout, 2142)
    y, info = run_conv(s, x, w, b)
    ref, _ = oracle.conv3d(x.astype(np.float64), w.astype(np.float64), b.astype(np.float64), None, s.pads,
                           s.tmode, with_mag=False)
    assert np.array_equal(y.view(np.uint16), ref.astype(np.float16).view(np.uint16)), info.kernel_name


def test_input_window_beyond_1_gib():
    # output frame 2 reads frames 0..2: a window of 2 frames + 2 rows + 256
    # voxels of 512 bytes, about 1.075e9 bytes, so gather offsets pass 2^30
    s = ConvShape(1, 3, 1024, 1024, 256, 8, tmode=R)
    x, w, b = ternary(s.x_shape, 2151), ternary(s.w_shape, 2152), small_ints(s.cout, 2153)
    y, info = run_conv(s, x, w, b, keep_device=True)
    assert info.path == c3d.CONV3D_PATH_GENERAL
    m, co = sampled(s, 6000, 2154)
    check_sampled(s, x, w, b, y, m, co, "window > 1 GiB")
