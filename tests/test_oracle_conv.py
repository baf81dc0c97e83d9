"""Pins for the fp64 conv3d oracle (CPU only).

None of these re-types the oracle's loop: each checks it against something
fixed independently -- an explicit im2col + numpy matmul, torch's own conv3d /
conv2d on the CPU in float64, closed forms, and invariants of the definition
(cross-correlation, stride 1, zero or replicate temporal padding).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

Z, R = oracle.TPAD_ZERO, oracle.TPAD_REPLICATE

# (kt, kh, kw, pads=(ptf, ptb, ph, pw), tmode)
GEOMS = [
    (3, 3, 3, (1, 1, 1, 1), Z),   # symmetric zero padding
    (3, 3, 3, (2, 0, 1, 1), R),   # causal, first frame replicated
    (3, 3, 3, (2, 0, 1, 1), Z),   # causal, zeros in front
    (3, 3, 3, (0, 0, 0, 0), Z),   # valid
    (1, 1, 1, (0, 0, 0, 0), Z),   # pointwise
    (1, 3, 3, (0, 0, 1, 1), Z),   # spatial-only
    (3, 1, 1, (2, 0, 0, 0), R),   # temporal-only causal
    (3, 3, 3, (1, 1, 1, 1), R),   # symmetric replicate in time
    (5, 3, 3, (4, 0, 1, 1), R),   # causal kt = 5
    (4, 5, 7, (1, 2, 2, 3), Z),   # mixed extents, asymmetric temporal padding
    (1, 7, 7, (0, 0, 3, 3), Z),   # 7x7 spatial
    (2, 2, 2, (1, 0, 1, 0), Z),   # even extents: one more output row than input rows
]


def rnd(shape, seed, lo=-1.0, hi=1.0):
    return np.random.default_rng(seed).uniform(lo, hi, size=shape)


def im2col_reference(x, w, b, pads, tmode):
    """Independent formulation: materialise the padded tensor, build im2col, matmul."""
    n, t, h, wd, cin = x.shape
    cout, kt, kh, kw, _ = w.shape
    ptf, ptb, ph, pw = pads
    xp = np.pad(x, ((0, 0), (ptf, ptb), (0, 0), (0, 0), (0, 0)),
                mode="edge" if tmode == R else "constant")
    xp = np.pad(xp, ((0, 0), (0, 0), (ph, ph), (pw, pw), (0, 0)), mode="constant")
    to, ho, wo = xp.shape[1] - kt + 1, xp.shape[2] - kh + 1, xp.shape[3] - kw + 1
    cols = []
    for tau in range(kt):
        for r in range(kh):
            for s in range(kw):
                cols.append(xp[:, tau:tau + to, r:r + ho, s:s + wo, :])
    a = np.concatenate(cols, axis=-1).reshape(-1, kt * kh * kw * cin)
    y = a @ w.reshape(cout, -1).T
    if b is not None:
        y = y + b
    return y.reshape(n, to, ho, wo, cout)


def torch_reference(x, w, b, pads, tmode):
    """torch.nn.functional.conv3d on the CPU in float64 (NCDHW)."""
    ptf, ptb, ph, pw = pads
    xt = torch.from_numpy(np.ascontiguousarray(x)).permute(0, 4, 1, 2, 3)
    if ptf or ptb:
        xt = F.pad(xt, (0, 0, 0, 0, ptf, ptb), mode="replicate" if tmode == R else "constant")
    wt = torch.from_numpy(np.ascontiguousarray(w)).permute(0, 4, 1, 2, 3)
    bt = None if b is None else torch.from_numpy(np.asarray(b))
    y = F.conv3d(xt, wt, bt, padding=(0, ph, pw))
    return y.permute(0, 2, 3, 4, 1).numpy()


@pytest.mark.parametrize("geom", GEOMS)
def test_brute_force_im2col(geom):
    kt, kh, kw, pads, tmode = geom
    x = rnd((2, 3, 4, 5, 3), 1)
    w = rnd((2, kt, kh, kw, 3), 2)
    b = rnd((2,), 3)
    y, _ = oracle.conv3d(x, w, b, None, pads, tmode)
    ref = im2col_reference(x, w, b, pads, tmode)
    assert y.shape == ref.shape
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("geom", GEOMS)
def test_library_conv3d(geom):
    kt, kh, kw, pads, tmode = geom
    x = rnd((2, 4, 6, 5, 8), 4)
    w = rnd((5, kt, kh, kw, 8), 5)
    b = rnd((5,), 6)
    y, _ = oracle.conv3d(x, w, b, None, pads, tmode)
    np.testing.assert_allclose(y, torch_reference(x, w, b, pads, tmode), rtol=1e-12, atol=1e-12)


def count_zero(i, n, pad_lo, k):
    """Taps in bounds along one zero-padded axis (closed form for a window of k)."""
    lo = i - pad_lo
    return max(0, min(n, lo + k) - max(0, lo))


@pytest.mark.parametrize("geom", GEOMS)
def test_all_ones_closed_form(geom):
    kt, kh, kw, pads, tmode = geom
    ptf, ptb, ph, pw = pads
    n, t, h, wd, cin = 1, 4, 5, 6, 7
    y, s = oracle.conv3d(np.ones((n, t, h, wd, cin)), np.ones((3, kt, kh, kw, cin)), None, None,
                         pads, tmode)
    to, ho, wo = y.shape[1:4]
    for a in range(to):
        nt = kt if tmode == R else count_zero(a, t, ptf, kt)
        for c in range(ho):
            for d in range(wo):
                expect = cin * nt * count_zero(c, h, ph, kh) * count_zero(d, wd, pw, kw)
                assert np.all(y[0, a, c, d] == expect)
                assert np.all(s[0, a, c, d] == expect)


def test_delta_kernel_reproduces_input():
    x = rnd((2, 4, 5, 6, 4), 7)
    for pads, tmode in (((1, 1, 1, 1), Z), ((2, 0, 1, 1), R), ((2, 0, 1, 1), Z)):
        w = np.zeros((4, 3, 3, 3, 4))
        tc = pads[0]  # the temporal tap that lands on the current frame
        for c in range(4):
            w[c, tc, 1, 1, c] = 1.0
        y, _ = oracle.conv3d(x, w, None, None, pads, tmode)
        assert np.array_equal(y, x)


def test_shifted_delta_is_correlation_not_convolution():
    x = rnd((1, 3, 5, 6, 2), 8)
    w = np.zeros((2, 3, 3, 3, 2))
    w[0, 1, 0, 0, 0] = 1.0  # tap (r, s) = (0, 0): reads (h-1, w-1)
    w[1, 1, 2, 1, 1] = 1.0  # tap (r, s) = (2, 1): reads (h+1, w)
    y, _ = oracle.conv3d(x, w, None, None, (1, 1, 1, 1), Z)
    e0 = np.zeros_like(x[..., 0])
    e0[:, :, 1:, 1:] = x[:, :, :-1, :-1, 0]
    e1 = np.zeros_like(x[..., 1])
    e1[:, :, :-1, :] = x[:, :, 1:, :, 1]
    assert np.array_equal(y[..., 0], e0)
    assert np.array_equal(y[..., 1], e1)


def test_causal_first_tap_reads_clamped_frames():
    x = rnd((1, 5, 3, 3, 2), 9)
    w = np.zeros((2, 3, 3, 3, 2))
    for c in range(2):
        w[c, 0, 1, 1, c] = 1.0  # tau = 0: frame t - 2, clamped to 0
    y, _ = oracle.conv3d(x, w, None, None, (2, 0, 1, 1), R)
    for t in range(5):
        assert np.array_equal(y[0, t], x[0, max(t - 2, 0)])
    yz, _ = oracle.conv3d(x, w, None, None, (2, 0, 1, 1), Z)
    assert np.all(yz[0, :2] == 0)
    assert np.array_equal(yz[0, 2:], x[0, :3])


def test_pointwise_is_matmul():
    x = rnd((2, 3, 4, 5, 16), 10)
    w = rnd((8, 1, 1, 1, 16), 11)
    b = rnd((8,), 12)
    y, _ = oracle.conv3d(x, w, b, None, (0, 0, 0, 0), Z)
    ref = np.matmul(x.reshape(-1, 16), w.reshape(8, 16).T) + b
    np.testing.assert_allclose(y.reshape(-1, 8), ref, rtol=1e-12, atol=1e-13)


def test_linearity_in_x_and_w():
    pads, tmode = (2, 0, 1, 1), R
    x1, x2 = rnd((1, 3, 4, 4, 4), 13), rnd((1, 3, 4, 4, 4), 14)
    w1, w2 = rnd((3, 3, 3, 3, 4), 15), rnd((3, 3, 3, 3, 4), 16)
    a, c = 0.75, -1.5

    def f(x, w):
        return oracle.conv3d(x, w, None, None, pads, tmode, with_mag=False)[0]
    np.testing.assert_allclose(f(a * x1 + c * x2, w1), a * f(x1, w1) + c * f(x2, w1),
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(f(x1, a * w1 + c * w2), a * f(x1, w1) + c * f(x1, w2),
                               rtol=1e-12, atol=1e-12)


def conv2d_frames(frames, w2, ph, pw):
    """torch conv2d (float64, CPU) of frames [F, H, W, Cin] with w2 [Cout, kh, kw, Cin]."""
    xt = torch.from_numpy(np.ascontiguousarray(frames)).permute(0, 3, 1, 2)
    wt = torch.from_numpy(np.ascontiguousarray(w2)).permute(0, 3, 1, 2)
    return F.conv2d(xt, wt, padding=(ph, pw)).permute(0, 2, 3, 1).numpy()


def test_causal_identity_sum_of_2d_over_temporal_taps():
    t = 5
    x = rnd((1, t, 6, 5, 4), 17)
    w = rnd((3, 3, 3, 3, 4), 18)
    b = rnd((3,), 19)
    y, _ = oracle.conv3d(x, w, b, None, (2, 0, 1, 1), R)
    # edge-replicated sequence [x0, x0, x0, x1, ...]
    xr = np.concatenate([x[0, :1], x[0, :1], x[0]], axis=0)
    ref = np.zeros_like(y[0]) + b
    for tau in range(3):
        ref += conv2d_frames(xr[tau:tau + t], w[:, tau], 1, 1)
    np.testing.assert_allclose(y[0], ref, rtol=1e-12, atol=1e-12)


def test_t1_fold_identity():
    x = rnd((1, 1, 6, 7, 8), 20)
    w = rnd((4, 3, 3, 3, 8), 21)
    b = rnd((4,), 22)
    y, _ = oracle.conv3d(x, w, b, None, (2, 0, 1, 1), R)
    ref = conv2d_frames(x[0], w.sum(axis=1), 1, 1) + b
    np.testing.assert_allclose(y[0], ref, rtol=1e-12, atol=1e-12)
    # zero-causal first frame: only the last temporal tap survives
    yz, _ = oracle.conv3d(x, w, b, None, (2, 0, 1, 1), Z)
    np.testing.assert_allclose(yz[0], conv2d_frames(x[0], w[:, 2], 1, 1) + b,
                               rtol=1e-12, atol=1e-12)


def test_causality():
    x = rnd((1, 6, 4, 4, 3), 23)
    w = rnd((2, 3, 3, 3, 3), 24)
    y, _ = oracle.conv3d(x, w, None, None, (2, 0, 1, 1), R)
    for t0 in (1, 3, 5):
        xp = x.copy()
        xp[0, t0] += 10.0
        yp, _ = oracle.conv3d(xp, w, None, None, (2, 0, 1, 1), R)
        assert np.array_equal(yp[0, :t0], y[0, :t0])
        assert not np.array_equal(yp[0, t0], y[0, t0])


@pytest.mark.parametrize("geom", GEOMS[:3])
def test_magnitude_is_conv_of_abs(geom):
    kt, kh, kw, pads, tmode = geom
    x = rnd((1, 3, 4, 5, 6), 25)
    w = rnd((3, kt, kh, kw, 6), 26)
    b = rnd((3,), 27)
    _, s = oracle.conv3d(x, w, b, None, pads, tmode)
    ref = torch_reference(np.abs(x), np.abs(w), np.abs(b), pads, tmode)
    np.testing.assert_allclose(s, ref, rtol=1e-12, atol=1e-12)


def test_residual_is_added_after_bias():
    x = rnd((1, 3, 4, 4, 4), 28)
    w = rnd((4, 3, 3, 3, 4), 29)
    b = rnd((4,), 30)
    res = rnd((1, 3, 4, 4, 4), 31)
    y, s = oracle.conv3d(x, w, b, None, (2, 0, 1, 1), R)
    yr, sr = oracle.conv3d(x, w, b, res, (2, 0, 1, 1), R)
    assert np.array_equal(yr, y + res)
    assert np.array_equal(sr, s)


def test_points_match_full():
    pads, tmode = (2, 0, 1, 1), R
    x = rnd((2, 3, 5, 4, 8), 32)
    w = rnd((6, 3, 3, 3, 8), 33)
    b = rnd((6,), 34)
    res = rnd((2, 3, 5, 4, 6), 35)
    y, s = oracle.conv3d(x, w, b, res, pads, tmode)
    rng = np.random.default_rng(36)
    m = rng.integers(0, y.size // 6, 50)
    co = rng.integers(0, 6, 50)
    yp, sp = oracle.conv3d_points(x, w, b, res, pads, tmode, m, co)
    assert np.array_equal(yp, y.reshape(-1, 6)[m, co])
    assert np.array_equal(sp, s.reshape(-1, 6)[m, co])


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.conv3d(np.ones((1, 1, 2, 2, 2)), np.ones((1, 3, 3, 3, 2)), None, None, (0, 0, 0, 0), Z)
    with pytest.raises(ValueError):
        oracle.conv3d_points(np.ones((1, 3, 3, 3, 2)), np.ones((1, 3, 3, 3, 2)), None, None,
                             (1, 1, 1, 1), Z, [27], [0])


def test_pins_catch_plausible_mistakes():
    """Each mistake a conv implementation plausibly makes changes the pinned result."""
    x = rnd((1, 4, 5, 6, 3), 37)
    w = rnd((2, 3, 3, 3, 3), 38)
    ref = torch_reference(x, w, None, (2, 0, 1, 1), R)
    mistakes = {
        "kernel flipped (convolution instead of correlation)":
            oracle.conv3d(x, w[:, ::-1, ::-1, ::-1], None, None, (2, 0, 1, 1), R)[0],
        "zeros instead of replicated first frame":
            oracle.conv3d(x, w, None, None, (2, 0, 1, 1), Z)[0],
        "symmetric instead of causal temporal padding":
            oracle.conv3d(x, w, None, None, (1, 1, 1, 1), R)[0],
        "input channels read in the wrong order":
            oracle.conv3d(x, w[:, :, :, :, ::-1], None, None, (2, 0, 1, 1), R)[0],
        "temporal taps read in the wrong order":
            oracle.conv3d(x, w[:, ::-1], None, None, (2, 0, 1, 1), R)[0],
        "spatial taps transposed (r <-> s)":
            oracle.conv3d(x, np.swapaxes(w, 2, 3), None, None, (2, 0, 1, 1), R)[0],
    }
    for name, y in mistakes.items():
        assert np.abs(y - ref).max() > 1e-3, name


def test_f16_decoder_is_exact_for_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.isinf(got) & (got > 0), np.isinf(ref) & (ref > 0))
    assert np.array_equal(np.signbit(got[finite]), np.signbit(ref[finite]))


def test_points_read_fp16_inputs_in_place():
    rng = np.random.default_rng(39)
    x16 = rng.normal(size=(1, 3, 5, 4, 8)).astype(np.float16)
    w = rnd((4, 3, 3, 3, 8), 40)
    b = rnd((4,), 41)
    r16 = rng.normal(size=(1, 3, 5, 4, 4)).astype(np.float16)
    y, s = oracle.conv3d(x16.astype(np.float64), w, b, r16.astype(np.float64), (2, 0, 1, 1), R)
    m = rng.integers(0, 60, 40)
    co = rng.integers(0, 4, 40)
    yp, sp = oracle.conv3d_points(x16, w, b, r16, (2, 0, 1, 1), R, m, co)
    assert np.array_equal(yp, y.reshape(-1, 4)[m, co])
    assert np.array_equal(sp, s.reshape(-1, 4)[m, co])
