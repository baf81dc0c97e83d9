"""GPU parity of groupnorm_silu and of the composed decoder block, through the C ABI.

GroupNorm+SiLU bound: |gpu - ref| <= 1e-3 |ref| + 2^-14 (tests/helpers.py).
The decoder block is checked stage by stage on GPU-fed inputs, each stage
under its own bound; its end-to-end relative L2 error against an all-fp64
oracle block is reported and held to 1e-2 (a gate the pages do not fix:
parity unpinned beyond the per-stage bounds).
"""
import numpy as np
import pytest
import torch

import convolution_implicit_gemm_amd as c3d
import oracle
import workloads
from workloads import ConvShape

from helpers import (assert_conv_close, assert_gn_close, check_guards, check_voxels, dev, edge_voxels,
                     frame_voxels, guarded_empty, out_dims, sample_points, conv_desc, workspace_for)

pytestmark = pytest.mark.gpu


def gn_gpu(x, gamma, beta, groups, eps=1e-6, silu=True, ws=None, in_place=False):
    n, c = x.shape[0], x.shape[-1]
    thw = int(np.prod(x.shape[1:-1]))
    xd = x if isinstance(x, torch.Tensor) else dev(x)
    need = c3d.groupnorm_silu_workspace(n, thw, c, groups)
    assert need > 0
    if ws is None:
        ws = torch.zeros(need, dtype=torch.uint8, device="cuda:0")
    if in_place:
        c3d.groupnorm_silu(xd, dev(gamma), dev(beta), xd, n, thw, c, groups, eps, silu, ws)
        torch.cuda.synchronize()
        return xd
    buf, y = guarded_empty(tuple(x.shape))
    c3d.groupnorm_silu(xd, dev(gamma), dev(beta), y, n, thw, c, groups, eps, silu, ws)
    torch.cuda.synchronize()
    check_guards(buf)
    return y


GN_CASES = [  # (n, thw_shape, c, groups, mean, std)
    (1, (3, 5, 7), 64, 8, 0.0, 1.0),
    (2, (2, 9, 9), 256, 32, 0.0, 1.0),
    (1, (4, 6, 5), 320, 40, 0.5, 2.0),
    (1, (1, 1, 3), 512, 32, 0.0, 1.0),
    (3, (5, 4, 4), 128, 1, 0.0, 1.0),
    (1, (2, 64, 64), 512, 32, 100.0, 1.0),  # large mean: the statistics must not cancel
    (2, (1, 1, 1), 64, 8, 0.0, 1.0),          # one voxel per sample: 8 values per group
    (1, (3, 3, 3), 8, 1, 0.0, 1.0),           # the fewest channels: 8 in one group
    (1, (1, 13, 17), 96, 12, -2.0, 0.5),      # odd voxel count, 8-channel groups
    (1, (1, 2, 3), 8192, 32, 0.0, 1.0),       # the most channels
    (1, (4, 32, 32), 1024, 128, 0.0, 1.0),    # 128 groups: partials beyond one apply block's merge
    (2, (4, 16, 16), 2048, 256, 1.0, 3.0),    # 256 groups of 8 channels, two samples
]


@pytest.mark.parametrize("case", range(len(GN_CASES)))
@pytest.mark.parametrize("silu", [True, False])
@pytest.mark.parametrize("final_kernel", [False, True])
def test_groupnorm_silu_small(case, silu, final_kernel, monkeypatch):
    # final_kernel: CONV3D_GN_FINAL=1 takes the separate final kernel and the
    # plain apply for every shape; otherwise the apply blocks merge the
    # partials themselves wherever they fit (256 KiB), as the library chooses
    monkeypatch.setenv("CONV3D_GN_FINAL", "1" if final_kernel else "0")
    n, thw, c, g, mean, std = GN_CASES[case]
    d = workloads.gn_inputs(n, thw, c, 800 + case, mean, std)
    y = gn_gpu(d["x"], d["gamma"], d["beta"], g, silu=silu).cpu().numpy()
    ref = oracle.groupnorm_silu(d["x"], d["gamma"], d["beta"], g, 1e-6, silu)
    assert_gn_close(y, ref, str(GN_CASES[case]))


def test_samples_of_a_batch_are_normalised_separately():
    a = workloads.gn_inputs(1, (3, 8, 8), 256, 900, 0.0, 1.0)
    b = workloads.gn_inputs(1, (3, 8, 8), 256, 901, 3.0, 5.0)
    x = np.concatenate([a["x"], b["x"]])
    y = gn_gpu(x, a["gamma"], a["beta"], 32).cpu().numpy()
    for i in range(2):
        ref = oracle.groupnorm_silu(x[i:i + 1], a["gamma"], a["beta"], 32, 1e-6, True)
        assert_gn_close(y[i:i + 1], ref, "sample %d" % i)


def test_in_place_and_workspace_reuse():
    d = workloads.gn_inputs(1, (3, 16, 16), 256, 902)
    need = c3d.groupnorm_silu_workspace(1, 3 * 256, 256, 32)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda:0")
    for rep in range(3):  # nothing of an earlier call's workspace may leak into the next
        x = d["x"] * np.float16(1 + rep)
        y = gn_gpu(x, d["gamma"], d["beta"], 32, ws=ws, in_place=(rep == 2)).cpu().numpy()
        ref = oracle.groupnorm_silu(x, d["gamma"], d["beta"], 32, 1e-6, True)
        assert_gn_close(y, ref, "rep %d" % rep)


@pytest.mark.parametrize("final_kernel", [False, True])
def test_decoder_block_groupnorm_full_size(final_kernel, monkeypatch):
    monkeypatch.setenv("CONV3D_GN_FINAL", "1" if final_kernel else "0")
    d = workloads.workload_inputs(4)
    y = gn_gpu(d["x"], d["gamma1"], d["beta1"], 32).cpu().numpy()
    ref = oracle.groupnorm_silu(d["x"], d["gamma1"], d["beta1"], 32, 1e-6, True)
    assert_gn_close(y, ref, "GN(32)+SiLU 17x128x128x256")


class Block:
    """The six-launch decoder block on one stream: GN1, conv1, GN2, conv2 (+x)."""

    def __init__(self, shape, groups=32, eps=1e-6):
        self.s, self.groups, self.eps = shape, groups, eps
        self.p1 = c3d.conv3d_plan(conv_desc(shape, c3d.CONV3D_F_BIAS))
        self.p2 = c3d.conv3d_plan(conv_desc(shape, c3d.CONV3D_F_BIAS | c3d.CONV3D_F_RESIDUAL))
        self.ws1, self.ws2 = workspace_for(self.p1), workspace_for(self.p2)
        self.thw = shape.t * shape.h * shape.w
        need = c3d.groupnorm_silu_workspace(shape.n, self.thw, shape.cin, groups)
        self.ws = torch.zeros(need, dtype=torch.uint8, device="cuda:0")

    def run(self, x, p):
        s = self.s
        a1 = torch.empty_like(x)
        c1 = torch.empty(out_dims(s), dtype=torch.float16, device="cuda:0")
        a2 = torch.empty_like(c1)
        out = torch.empty_like(c1)
        c3d.groupnorm_silu(x, p["gamma1"], p["beta1"], a1, s.n, self.thw, s.cin, self.groups,
                           self.eps, True, self.ws)
        c3d.conv3d_forward(self.p1, a1, p["w1"], p["b1"], None, c1, self.ws1)
        c3d.groupnorm_silu(c1, p["gamma2"], p["beta2"], a2, s.n, self.thw, s.cout, self.groups,
                           self.eps, True, self.ws)
        c3d.conv3d_forward(self.p2, a2, p["w2"], p["b2"], x, out, self.ws2)
        return a1, c1, a2, out


def test_decoder_block_per_stage_full_size():
    d = workloads.workload_inputs(4)
    s = d["shape"]
    p = {k: dev(d[k]) for k in ("gamma1", "beta1", "w1", "b1", "gamma2", "beta2", "w2", "b2")}
    blk = Block(s)
    a1, c1, a2, out = (t.cpu().numpy() for t in blk.run(dev(d["x"]), p))
    torch.cuda.synchronize()
    assert_gn_close(a1, oracle.groupnorm_silu(d["x"], d["gamma1"], d["beta1"], 32), "GN1")
    od = out_dims(s)
    m_total = od[0] * od[1] * od[2] * od[3]
    m, co = sample_points(m_total, s.cout, 6000, 16, edge_voxels(od))
    ref, mag = oracle.conv3d_points(a1, d["w1"], d["b1"], None, s.pads, s.tmode, m, co)
    assert_conv_close(c1.reshape(-1, s.cout)[m, co], ref, mag, "conv1")
    assert_gn_close(a2, oracle.groupnorm_silu(c1, d["gamma2"], d["beta2"], 32), "GN2")
    ref, mag = oracle.conv3d_points(a2, d["w2"], d["b2"], d["x"], s.pads, s.tmode, m, co)
    assert_conv_close(out.reshape(-1, s.cout)[m, co], ref, mag, "conv2 + residual")
    # both convs at every channel of output frames 0, 1 and T-1 (each on the GPU's own input)
    vox = frame_voxels(od, [0, 1, od[1] - 1])
    check_voxels(s, a1.astype(np.float64), d["w1"], d["b1"], torch.from_numpy(c1).to("cuda:0"), vox,
                 what="conv1, frames 0, 1, T-1")
    check_voxels(s, a2.astype(np.float64), d["w2"], d["b2"], torch.from_numpy(out).to("cuda:0"), vox,
                 res=d["x"], what="conv2 + residual, frames 0, 1, T-1")


def test_decoder_block_end_to_end_small():
    s = ConvShape(1, 3, 16, 16, 256, 256)
    d = workloads.block_inputs(s, 1404)
    p = {k: dev(d[k]) for k in ("gamma1", "beta1", "w1", "b1", "gamma2", "beta2", "w2", "b2")}
    out = Block(s).run(dev(d["x"]), p)[3].cpu().numpy().astype(np.float64)
    ref = oracle.decoder_block(d["x"], (d["gamma1"], d["beta1"]), (d["w1"], d["b1"]),
                               (d["gamma2"], d["beta2"]), (d["w2"], d["b2"]), groups=32,
                               eps=1e-6, pads=s.pads, tmode=s.tmode)
    rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    print("decoder block end-to-end relative L2 error: %.3e" % rel)
    assert rel <= 1e-2
