"""Pins for the fp64 GroupNorm+SiLU oracle and the decoder-block composition (CPU only)."""
import pytest
import numpy as np
import torch
import torch.nn.functional as F

import oracle


def rnd(shape, seed, mean=0.0, std=1.0):
    return np.random.default_rng(seed).normal(mean, std, size=shape)


def torch_gn_silu(x, gamma, beta, groups, eps, silu=True):
    xt = torch.from_numpy(np.ascontiguousarray(x))
    xt = xt.reshape(xt.shape[0], -1, xt.shape[-1]).permute(0, 2, 1)  # N, C, THW
    y = F.group_norm(xt, groups, torch.from_numpy(gamma), torch.from_numpy(beta), eps)
    if silu:
        y = F.silu(y)
    return y.permute(0, 2, 1).reshape(x.shape).numpy()


def test_matches_torch_group_norm():
    x = rnd((2, 3, 4, 5, 32), 1, 0.5, 2.0)
    g, b = rnd((32,), 2, 1.0, 0.1), rnd((32,), 3, 0.0, 0.1)
    for groups in (1, 4, 8, 32):
        for silu in (False, True):
            y = oracle.groupnorm_silu(x, g, b, groups, 1e-6, silu)
            np.testing.assert_allclose(y, torch_gn_silu(x, g, b, groups, 1e-6, silu),
                                       rtol=1e-12, atol=1e-12)


def test_matches_numpy_reshape_mean_var():
    x = rnd((2, 2, 3, 3, 16), 4)
    g, b = rnd((16,), 5, 1.0, 0.1), rnd((16,), 6, 0.0, 0.1)
    y, mean, var = oracle.groupnorm_silu(x, g, b, 4, 1e-5, False, return_stats=True)
    xg = x.reshape(2, -1, 4, 4)  # N, THW, G, C/G
    mu = xg.mean(axis=(1, 3))
    va = xg.var(axis=(1, 3))
    np.testing.assert_allclose(mean, mu, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(var, va, rtol=1e-12)
    ref = (xg - mu[:, None, :, None]) / np.sqrt(va[:, None, :, None] + 1e-5)
    ref = ref.reshape(x.shape) * g + b
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_constant_group_gives_silu_of_beta():
    x = np.full((1, 2, 2, 2, 8), 3.25)
    g, b = rnd((8,), 7, 1.0, 0.1), rnd((8,), 8, 0.0, 0.5)
    y = oracle.groupnorm_silu(x, g, b, 2, 1e-6, True)
    ref = b / (1.0 + np.exp(-b))
    np.testing.assert_allclose(y, np.broadcast_to(ref, y.shape), rtol=1e-14, atol=0)


def test_plus_minus_halves_closed_form():
    a, eps = 1.75, 1e-6
    x = np.empty((1, 4, 1, 1, 4))
    x[:, :2] = a
    x[:, 2:] = -a  # each group: equal halves of +a and -a -> mean 0, var a^2
    g = np.array([1.0, 2.0, 0.5, -1.0])
    b = np.array([0.0, 0.25, -0.5, 1.0])
    y = oracle.groupnorm_silu(x, g, b, 2, eps, False)
    yh = a / np.sqrt(a * a + eps)
    np.testing.assert_allclose(y[0, :2, 0, 0], np.broadcast_to(yh * g + b, (2, 4)), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(y[0, 2:, 0, 0], np.broadcast_to(-yh * g + b, (2, 4)), rtol=1e-14, atol=1e-15)


def test_silu_special_values():
    x = rnd((1, 2, 2, 2, 4), 9)
    zero = oracle.groupnorm_silu(x, np.zeros(4), np.zeros(4), 2, 1e-6, True)
    assert np.all(zero == 0.0)
    one = oracle.groupnorm_silu(x, np.zeros(4), np.ones(4), 2, 1e-6, True)
    np.testing.assert_allclose(one, 1.0 / (1.0 + np.exp(-1.0)), rtol=1e-15)


def test_samples_are_normalised_independently():
    """The batch case that a GROUP_NORM bug once got wrong: each sample on its own."""
    x0 = rnd((1, 3, 3, 3, 16), 10, 0.0, 1.0)
    x1 = rnd((1, 3, 3, 3, 16), 11, 5.0, 3.0)
    g, b = rnd((16,), 12, 1.0, 0.1), rnd((16,), 13, 0.0, 0.1)
    both = oracle.groupnorm_silu(np.concatenate([x0, x1]), g, b, 4, 1e-6, True)
    assert np.array_equal(both[:1], oracle.groupnorm_silu(x0, g, b, 4, 1e-6, True))
    assert np.array_equal(both[1:], oracle.groupnorm_silu(x1, g, b, 4, 1e-6, True))


def test_shift_and_scale_invariance():
    x = rnd((1, 3, 4, 4, 8), 14)
    g, b = rnd((8,), 15, 1.0, 0.1), rnd((8,), 16, 0.0, 0.1)
    y = oracle.groupnorm_silu(x, g, b, 2, 0.0, True)
    y2 = oracle.groupnorm_silu(3.0 * x + 7.0, g, b, 2, 0.0, True)
    np.testing.assert_allclose(y2, y, rtol=1e-12, atol=1e-12)


def test_decoder_block_composition():
    x = rnd((1, 3, 4, 4, 16), 17)
    g1, b1 = rnd((16,), 18, 1.0, 0.1), rnd((16,), 19, 0.0, 0.1)
    g2, b2 = rnd((16,), 20, 1.0, 0.1), rnd((16,), 21, 0.0, 0.1)
    w1, c1 = rnd((16, 3, 3, 3, 16), 22, 0, 0.05), rnd((16,), 23, 0, 0.02)
    w2, c2 = rnd((16, 3, 3, 3, 16), 24, 0, 0.05), rnd((16,), 25, 0, 0.02)
    out = oracle.decoder_block(x, (g1, b1), (w1, c1), (g2, b2), (w2, c2), groups=4)
    # same block through torch on the CPU in float64
    xt = torch.from_numpy(x).permute(0, 4, 1, 2, 3)

    def gn(v, g, b):
        return F.silu(F.group_norm(v, 4, torch.from_numpy(g), torch.from_numpy(b), 1e-6))

    def conv(v, w, c):
        v = F.pad(v, (0, 0, 0, 0, 2, 0), mode="replicate")
        return F.conv3d(v, torch.from_numpy(w).permute(0, 4, 1, 2, 3), torch.from_numpy(c),
                        padding=(0, 1, 1))
    ref = xt + conv(gn(conv(gn(xt, g1, b1), w1, c1), g2, b2), w2, c2)
    np.testing.assert_allclose(out, ref.permute(0, 2, 3, 4, 1).numpy(), rtol=1e-11, atol=1e-12)


def test_points_variant_equals_the_full_oracle_everywhere():
    # fp16 input read in place and fp64 input; several groups per sample, two samples
    rng = np.random.default_rng(31)
    for shape, groups, silu in [((2, 3, 5, 7, 64), 8, True), ((1, 130, 48), 4, False), ((3, 1, 16), 16, True)]:
        x16 = (rng.standard_normal(shape) * 3 + 1).astype(np.float16)
        c = shape[-1]
        gamma, beta = rng.normal(1, 0.1, c), rng.normal(0, 0.1, c)
        ref, mean, var = oracle.groupnorm_silu(x16.astype(np.float64), gamma, beta, groups, 1e-6, silu,
                                               return_stats=True)
        nvox = int(np.prod(shape[:-1]))
        vox = np.repeat(np.arange(nvox), c)
        ch = np.tile(np.arange(c), nvox)
        for xin in (x16, x16.astype(np.float64)):
            y, m, v = oracle.groupnorm_silu_points(xin, gamma, beta, groups, vox, ch, 1e-6, silu)
            np.testing.assert_allclose(y, ref.reshape(-1), rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(m, mean, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(v, var, rtol=1e-12)


def test_points_variant_rejects_out_of_range_elements():
    x = np.zeros((1, 4, 8), np.float16)
    g, b = np.ones(8), np.zeros(8)
    with pytest.raises(ValueError):
        oracle.groupnorm_silu_points(x, g, b, 2, [4], [0])
    with pytest.raises(ValueError):
        oracle.groupnorm_silu_points(x, g, b, 2, [0], [8])
