"""GPU parity of chunked causal decoding (CONV3D_F_CHUNK, conv3d_forward_chunk).

A chunk's output is the conv of [x_prev; x] along t with no temporal padding,
so the oracle is conv3d over that concatenation (pads (0, 0, ph, pw)).  Decoding
a video in chunks must also reproduce the whole-video causal conv: with ternary
data every sum is exact, so the two agree bit for bit whatever the tiling.
Both ways of running a chunk are checked: one conv over a copy of the
concatenation ("cat") and a head conv plus a conv over the chunk alone
("split"), forced through CONV3D_CHUNK, next to the planner's own choice.
"""
import numpy as np
import pytest
import torch

import convolution_implicit_gemm_amd as c3d
import oracle
import workloads
from workloads import ConvShape, TPAD_REPLICATE as R, TPAD_ZERO as Z

from helpers import (assert_conv_close, check_guards, conv_desc, dev, env_var, guarded_empty, host_bits,
                     out_dims, run_conv, ulp_bf16, workspace_for)

pytestmark = pytest.mark.gpu


STRATEGIES = [None, "cat", "split"]


def chunk(shape, x_prev, x, w, b=None, res=None, bf16=False, strategy=None):
    flags = c3d.CONV3D_F_CHUNK | (c3d.CONV3D_F_BIAS if b is not None else 0) | \
        (c3d.CONV3D_F_RESIDUAL if res is not None else 0) | (c3d.CONV3D_F_BF16 if bf16 else 0)
    with env_var("CONV3D_CHUNK", strategy):
        plan = c3d.conv3d_plan(conv_desc(shape, flags))
    buf, y = guarded_empty(out_dims(shape), torch.bfloat16 if bf16 else torch.float16)
    ws = workspace_for(plan)
    c3d.conv3d_forward_chunk(plan, dev(x_prev), dev(x), dev(w), None if b is None else dev(b),
                             None if res is None else dev(res), y, ws)
    torch.cuda.synchronize()
    check_guards(buf)
    return host_bits(y) if bf16 else y.cpu().numpy()


def widen(a):
    """fp16 numpy -> float64 (exact)."""
    return np.asarray(a, dtype=np.float64)


def concat_oracle(shape, x_prev, x, w, b=None, res=None, dec=widen):
    xc = np.concatenate([dec(x_prev), dec(x)], axis=1)
    return oracle.conv3d(xc, dec(w), None if b is None else dec(b), None if res is None else dec(res),
                         (0, 0, shape.pad_h, shape.pad_w), Z)


CASES = [
    ConvShape(1, 5, 12, 14, 64, 64),
    ConvShape(1, 6, 9, 11, 48, 64, kt=5, pad_t_front=4, pad_t_back=0),   # four history frames (general gather)
    ConvShape(2, 3, 8, 10, 64, 32, kt=2, kh=1, kw=1, pad_t_front=1, pad_t_back=0, pad_h=0, pad_w=0),  # one history frame, 2x1x1 kernel
    ConvShape(2, 4, 9, 10, 40, 48),            # channel tail, two samples
    ConvShape(1, 1, 16, 16, 128, 64),          # one frame: the head conv alone
    ConvShape(1, 2, 8, 8, 32, 32),             # as long as the history: head conv alone
    ConvShape(1, 9, 32, 32, 256, 256),
]


@pytest.mark.parametrize("strategy", STRATEGIES)
@pytest.mark.parametrize("case", range(len(CASES)))
def test_chunk_matches_conv_of_the_concatenation(case, strategy):
    s = CASES[case]
    d = workloads.conv_inputs(s, 900 + case)
    x_prev = workloads.normal_f16(np.random.SeedSequence(950 + case), (s.n, s.kt - 1, s.h, s.w, s.cin))
    res = workloads.normal_f16(np.random.SeedSequence(960 + case), out_dims(s))
    y = chunk(s, x_prev, d["x"], d["w"], d["b"], res, strategy=strategy)
    ref, mag = concat_oracle(s, x_prev, d["x"], d["w"], d["b"], res)
    assert_conv_close(y, ref, mag, "chunk " + str(s))


@pytest.mark.parametrize("strategy", STRATEGIES)
def test_chunked_decode_on_the_dynamic_tile_schedule(strategy):
    # every plan forced onto the row-slab tile and the one-workgroup-per-CU
    # schedule, whose tile counters then sit in each sub-plan's share of the
    # chunk plan's workspace; ternary data, so chunked equals whole bit for bit
    tc = 4
    whole = ConvShape(1, 3 * tc, 8, 64, 64, 64, tmode=R)
    rng = np.random.default_rng(990)
    x = rng.integers(-1, 2, size=whole.x_shape).astype(np.float16)
    w = rng.integers(-1, 2, size=whole.w_shape).astype(np.float16)
    b = rng.integers(-2, 3, whole.cout).astype(np.float16)
    part = ConvShape(1, tc, 8, 64, 64, 64, tmode=R)
    with env_var("CONV3D_TILE", "m256n256k64ps"), env_var("CONV3D_DYNAMIC", "1"):
        y_whole, info = run_conv(whole, x, w, b)
        assert info.grid <= 256
        y0, _ = run_conv(part, x[:, :tc], w, b)
        parts = [y0]
        for k in (1, 2):
            hist = [k * tc - 2, k * tc - 1]
            parts.append(chunk(part, np.ascontiguousarray(x[:, hist]), x[:, k * tc:(k + 1) * tc], w, b,
                               strategy=strategy))
    assert np.array_equal(np.concatenate(parts, axis=1), y_whole)
    ref, _ = oracle.conv3d(widen(x), widen(w), widen(b), None, whole.pads, whole.tmode)
    assert np.array_equal(widen(y_whole), ref)


@pytest.mark.parametrize("strategy", STRATEGIES)
@pytest.mark.parametrize("n,tc", [(1, 6), (2, 3), (1, 1)])
def test_chunked_decode_equals_whole_video_decode(n, tc, strategy):
    # a video of 3 chunks of tc frames: chunk 0 with the causal (replicate)
    # plan, chunks 1 and 2 with their predecessor's last 2 frames as history
    whole = ConvShape(n, 3 * tc, 10, 12, 64, 56, tmode=R)
    rng = np.random.default_rng(970 + n + tc)
    x = rng.integers(-1, 2, size=whole.x_shape).astype(np.float16)
    w = rng.integers(-1, 2, size=whole.w_shape).astype(np.float16)
    b = rng.integers(-2, 3, whole.cout).astype(np.float16)
    y_whole, _ = run_conv(whole, x, w, b)
    part = ConvShape(n, tc, 10, 12, 64, 56, tmode=R)
    y0, _ = run_conv(part, x[:, :tc], w, b)
    parts = [y0]
    for k in (1, 2):
        # chunk k's history: frames k*tc-2 and k*tc-1, clamped at 0 as the
        # whole video's replicate padding clamps them
        hist = [max(k * tc - 2, 0), max(k * tc - 1, 0)]
        parts.append(chunk(part, np.ascontiguousarray(x[:, hist]), x[:, k * tc:(k + 1) * tc], w, b,
                           strategy=strategy))
    assert np.array_equal(np.concatenate(parts, axis=1), y_whole)


@pytest.mark.parametrize("strategy", STRATEGIES)
def test_chunk_bf16(strategy):
    s = ConvShape(2, 4, 12, 10, 64, 64)
    d = workloads.conv_inputs(s, 990, dtype="bf16")
    x_prev = workloads.normal_f16(np.random.SeedSequence(991), (s.n, 2, s.h, s.w, s.cin), dtype="bf16")
    y = chunk(s, x_prev, d["x"], d["w"], d["b"], bf16=True, strategy=strategy)
    ref, mag = concat_oracle(s, x_prev, d["x"], d["w"], d["b"], dec=oracle.bf16_to_f64)
    assert_conv_close(oracle.bf16_to_f64(y), ref, mag, "bf16 chunk", ulp=ulp_bf16)
