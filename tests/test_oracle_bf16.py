"""Pins of the bf16 pieces of the test infrastructure (CPU).

bf16_to_f64 (the oracle's decoder of bf16 operands) is checked on all 65,536
bit patterns against the value built term by term from the format's
definition (sign, 8-bit exponent with bias 127, 7-bit fraction).
workloads.to_bf16 (how bf16 inputs are made from float32 draws) is checked
against torch's float32 -> bfloat16 conversion, round-to-nearest-even.
"""
import math

import numpy as np
import torch

import oracle
import workloads


def _by_definition(bits):
    sign = -1.0 if bits >> 15 else 1.0
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    if e == 0xFF:
        return sign * math.inf if f == 0 else math.nan
    if e == 0:
        return sign * math.ldexp(f / 128.0, -126)
    return sign * math.ldexp(1.0 + f / 128.0, e - 127)


def test_bf16_decoder_matches_the_format_definition_on_every_pattern():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.bf16_to_f64(pats)
    want = np.array([_by_definition(int(b)) for b in range(65536)])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_to_bf16_is_round_to_nearest_even():
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.float32([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 0.0, -0.0,
                                    65504.0, 1e-38, 3.0e38])])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(workloads.to_bf16(v), ref)
    # the ties: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 and goes to the even one
    assert oracle.bf16_to_f64(workloads.to_bf16(np.float32([1.0 + 2.0 ** -8])))[0] == 1.0
    assert oracle.bf16_to_f64(workloads.to_bf16(np.float32([1.0 + 3 * 2.0 ** -8])))[0] == 1.0 + 2.0 ** -6


def test_bf16_inputs_share_the_fp16_draws():
    s = workloads.ConvShape(1, 2, 4, 5, 16, 8)
    a = workloads.conv_inputs(s, 77)
    b = workloads.conv_inputs(s, 77, dtype="bf16")
    assert b["x"].dtype == np.uint16 and b["w"].dtype == np.uint16
    # both round the same float32 draws: they agree to bf16 precision
    assert np.allclose(oracle.bf16_to_f64(b["x"]), a["x"].astype(np.float64), rtol=2 ** -8, atol=0)
