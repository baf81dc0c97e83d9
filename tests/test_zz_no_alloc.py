"""groupnorm_silu_noalloc (static device scratch) against groupnorm_silu (caller workspace).

Two calls in a row on one device, the second with a smaller input, each
compared bit for bit with groupnorm_silu on the same data (same kernels and
launch shape, so the same bits) and with the fp64 oracle within the
GroupNorm bound.  Both calls go through the C ABI.
"""
import numpy as np
import pytest
import torch

import convolution_implicit_gemm_amd as c3d
import oracle
import workloads
from helpers import assert_gn_close, check_guards, dev, guarded_empty

pytestmark = pytest.mark.gpu


def _one(n, t, h, w, c, groups, seed, silu=True):
    thw = t * h * w
    g = workloads.gn_inputs(n, (t, h, w), c, seed)
    x, ga, be = dev(g["x"]), dev(g["gamma"]), dev(g["beta"])
    shape = tuple(g["x"].shape)
    ws = torch.zeros(c3d.groupnorm_silu_workspace(n, thw, c, groups), dtype=torch.uint8, device="cuda:0")
    buf_ref, y_ref = guarded_empty(shape)
    c3d.groupnorm_silu(x, ga, be, y_ref, n, thw, c, groups, 1e-6, silu, ws)
    buf, y = guarded_empty(shape)
    c3d.groupnorm_silu_noalloc(x, ga, be, y, n, thw, c, groups, 1e-6, silu)
    torch.cuda.synchronize()
    check_guards(buf)
    check_guards(buf_ref)
    got, want = y.cpu().numpy(), y_ref.cpu().numpy()
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), "noalloc differs from the workspace call"
    ref = oracle.groupnorm_silu(g["x"], g["gamma"], g["beta"], groups, 1e-6, silu)
    assert_gn_close(got, ref, "noalloc n=%d thw=%d c=%d" % (n, thw, c))


def test_noalloc_matches_workspace_call_twice_second_smaller():
    # the decoder-block shape, then a smaller one: the second call finds the
    # first call's statistics in the shared array and must not use them
    _one(1, 17, 128, 128, 256, 32, 901)
    _one(2, 3, 8, 12, 128, 16, 902)


def test_noalloc_without_silu_and_in_place():
    g = workloads.gn_inputs(1, (4, 16, 16), 320, 903)
    thw = 4 * 16 * 16
    x = dev(g["x"])
    ref = oracle.groupnorm_silu(g["x"], g["gamma"], g["beta"], 40, 1e-6, False)
    c3d.groupnorm_silu_noalloc(x, dev(g["gamma"]), dev(g["beta"]), x, 1, thw, 320, 40, 1e-6, False)
    torch.cuda.synchronize()
    assert_gn_close(x.cpu().numpy(), ref, "noalloc in place, no SiLU")
