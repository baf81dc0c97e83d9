"""HIP-graph capture of the library's calls (torch.cuda.CUDAGraph, captured on the current stream).

Forward calls enqueue kernels and device-to-device copies only: no memsets, no
allocation, no host synchronisation, so a caller may capture them.  Each graph
below is replayed several times.  Between replays, new input values are copied
into the captured input buffers, and eager work and synchronisations run.  Every
replay must equal an eager run on the same inputs bit for bit (same kernels,
same plans, so the same arithmetic order).
"""
import numpy as np
import pytest
import torch

import convolution_implicit_gemm_amd as c3d
import workloads
from workloads import ConvShape

from helpers import conv_desc, dev, env_var, forced_tile, out_dims, workspace_for

pytestmark = pytest.mark.gpu

REPLAYS = 4


def bits(t):
    return t.view(torch.int16)


def capture(fn):
    """Warm fn up eagerly on a side stream, then capture it into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


class BlockBuffers:
    """Decoder block GN1 -> conv1 -> GN2 -> conv2 (+x) over fixed buffers."""

    def __init__(self, s, p1, p2, params, groups=32):
        self.s, self.p1, self.p2, self.p, self.groups = s, p1, p2, params, groups
        self.thw = s.t * s.h * s.w
        self.x = torch.empty(s.x_shape, dtype=torch.float16, device="cuda:0")
        self.a1 = torch.empty_like(self.x)
        self.c1 = torch.empty(out_dims(s), dtype=torch.float16, device="cuda:0")
        self.a2, self.out = torch.empty_like(self.c1), torch.empty_like(self.c1)
        self.ws1, self.ws2 = workspace_for(p1), workspace_for(p2)
        need = c3d.groupnorm_silu_workspace(s.n, self.thw, s.cin, groups)
        self.gws = torch.empty(need, dtype=torch.uint8, device="cuda:0")

    def run(self):
        s, p = self.s, self.p
        c3d.groupnorm_silu(self.x, p["gamma1"], p["beta1"], self.a1, s.n, self.thw, s.cin, self.groups, 1e-6,
                           True, self.gws)
        c3d.conv3d_forward(self.p1, self.a1, p["w1"], p["b1"], None, self.c1, self.ws1)
        c3d.groupnorm_silu(self.c1, p["gamma2"], p["beta2"], self.a2, s.n, self.thw, s.cout, self.groups, 1e-6,
                           True, self.gws)
        c3d.conv3d_forward(self.p2, self.a2, p["w2"], p["b2"], self.x, self.out, self.ws2)


def test_decoder_block_graph_replays_equal_eager():
    s = ConvShape(1, 3, 20, 24, 256, 256)
    # conv1 forced onto a K-split plan, so the graph holds the fixup kernel too
    with forced_tile("m256n256k64s2a3w8"), env_var("CONV3D_STREAMK", "1"):
        p1 = c3d.conv3d_plan(conv_desc(s, c3d.CONV3D_F_BIAS))
    assert p1.info().split_tiles > 0
    p2 = c3d.conv3d_plan(conv_desc(s, c3d.CONV3D_F_BIAS | c3d.CONV3D_F_RESIDUAL))
    d = workloads.block_inputs(s, 1500)
    params = {k: dev(d[k]) for k in ("gamma1", "beta1", "w1", "b1", "gamma2", "beta2", "w2", "b2")}
    graphed, eager = BlockBuffers(s, p1, p2, params), BlockBuffers(s, p1, p2, params)
    graphed.x.copy_(dev(d["x"]))
    g = capture(graphed.run)
    for k in range(REPLAYS):
        xk = dev(workloads.normal_f16(np.random.SeedSequence(1510 + k), s.x_shape))
        graphed.x.copy_(xk)
        g.replay()
        eager.x.copy_(xk)
        eager.run()  # eager work on the same stream between replays
        torch.cuda.synchronize()
        for name in ("a1", "c1", "a2", "out"):
            assert torch.equal(bits(getattr(graphed, name)), bits(getattr(eager, name))), (k, name)


@pytest.mark.parametrize("strategy", ["cat", "split"])
def test_chunked_forward_graph_replays_equal_eager(strategy):
    s = ConvShape(2, 4, 12, 10, 64, 64)
    with env_var("CONV3D_CHUNK", strategy):
        plan = c3d.conv3d_plan(conv_desc(s, c3d.CONV3D_F_BIAS | c3d.CONV3D_F_CHUNK))
    d = workloads.conv_inputs(s, 1520)
    w, b = dev(d["w"]), dev(d["b"])
    hist_shape = (s.n, s.kt - 1, s.h, s.w, s.cin)
    xp, x = torch.empty(hist_shape, dtype=torch.float16, device="cuda:0"), dev(d["x"])
    y, ws = torch.empty(out_dims(s), dtype=torch.float16, device="cuda:0"), workspace_for(plan)
    xp.copy_(dev(workloads.normal_f16(np.random.SeedSequence(1521), hist_shape)))
    g = capture(lambda: c3d.conv3d_forward_chunk(plan, xp, x, w, b, None, y, ws))
    y_eager, ws_eager = torch.empty_like(y), workspace_for(plan)
    for k in range(REPLAYS):
        xp.copy_(dev(workloads.normal_f16(np.random.SeedSequence(1530 + k), hist_shape)))
        x.copy_(dev(workloads.normal_f16(np.random.SeedSequence(1540 + k), s.x_shape)))
        g.replay()
        c3d.conv3d_forward_chunk(plan, xp, x, w, b, None, y_eager, ws_eager)
        torch.cuda.synchronize()
        assert torch.equal(bits(y), bits(y_eager)), k


def test_bf16_conv_and_fold_graph_replays_equal_eager():
    s = ConvShape(1, 1, 24, 20, 64, 64, pad_t_front=2, pad_t_back=0)  # T=1: fold kernel + conv
    plan = c3d.conv3d_plan(conv_desc(s, c3d.CONV3D_F_BIAS | c3d.CONV3D_F_BF16))
    assert plan.info().path == c3d.CONV3D_PATH_T1_FOLD
    d = workloads.conv_inputs(s, 1550, dtype="bf16")
    x, w, b = dev(d["x"]), dev(d["w"]), dev(d["b"])
    y, ws = torch.empty(out_dims(s), dtype=torch.bfloat16, device="cuda:0"), workspace_for(plan)
    g = capture(lambda: c3d.conv3d_forward(plan, x, w, b, None, y, ws))
    y_eager, ws_eager = torch.empty_like(y), workspace_for(plan)
    for k in range(REPLAYS):
        # new weights too: the fold runs inside the graph on every replay
        w.copy_(dev(workloads.uniform_f16(np.random.SeedSequence(1560 + k), s.w_shape, 0.05, dtype="bf16")))
        x.copy_(dev(workloads.normal_f16(np.random.SeedSequence(1570 + k), s.x_shape, dtype="bf16")))
        g.replay()
        c3d.conv3d_forward(plan, x, w, b, None, y_eager, ws_eager)
        torch.cuda.synchronize()
        assert torch.equal(bits(y), bits(y_eager)), k


def test_dynamic_tile_schedule_graph_replays_equal_eager():
    # the slab kernel's dynamic schedule: a counter-reset kernel, then one
    # workgroup per CU taking tiles; replays must find the counters reset
    s = ConvShape(1, 9, 32, 128, 64, 64)
    with forced_tile("m256n256k64ps"), env_var("CONV3D_DYNAMIC", "1"):
        plan = c3d.conv3d_plan(conv_desc(s, c3d.CONV3D_F_BIAS))
    info = plan.info()
    assert info.kernel_name.decode().startswith("conv3d_igemm_m256n256k64ps") and plan.workspace_bytes > 0
    d = workloads.conv_inputs(s, 1580)
    x, w, b = dev(d["x"]), dev(d["w"]), dev(d["b"])
    y, ws = torch.empty(out_dims(s), dtype=torch.float16, device="cuda:0"), workspace_for(plan)
    g = capture(lambda: c3d.conv3d_forward(plan, x, w, b, None, y, ws))
    y_eager, ws_eager = torch.empty_like(y), workspace_for(plan)
    for k in range(REPLAYS):
        x.copy_(dev(workloads.normal_f16(np.random.SeedSequence(1590 + k), s.x_shape)))
        g.replay()
        c3d.conv3d_forward(plan, x, w, b, None, y_eager, ws_eager)
        torch.cuda.synchronize()
        assert torch.equal(bits(y), bits(y_eager)), k


class StatsBlockBuffers(BlockBuffers):
    """The block with GN2 from conv1's statistics (conv1 planned with CONV3D_F_GN_STATS)."""

    def __init__(self, s, p1, p2, params, groups=32):
        super().__init__(s, p1, p2, params, groups)
        self.stats, self.slots = c3d.gn_stats_view(p1, self.ws1)
        self.sws = torch.empty(c3d.groupnorm_silu_from_stats_workspace(s.n, s.cout, groups), dtype=torch.uint8,
                               device="cuda:0")

    def run(self):
        s, p = self.s, self.p
        c3d.groupnorm_silu(self.x, p["gamma1"], p["beta1"], self.a1, s.n, self.thw, s.cin, self.groups, 1e-6,
                           True, self.gws)
        c3d.conv3d_forward(self.p1, self.a1, p["w1"], p["b1"], None, self.c1, self.ws1)
        c3d.groupnorm_silu_from_stats(self.c1, p["gamma2"], p["beta2"], self.a2, s.n, self.thw, s.cout,
                                      self.groups, 1e-6, True, self.stats, self.slots, self.sws)
        c3d.conv3d_forward(self.p2, self.a2, p["w2"], p["b2"], self.x, self.out, self.ws2)


@pytest.mark.parametrize("dynamic", ["0", "1"])
def test_block_with_gn2_from_conv1_statistics_graph_replays_equal_eager(dynamic):
    # conv1 with statistics, forced onto a K split (the fixup's partials too),
    # on the static or the one-workgroup-per-CU schedule (its counter-clearing kernel)
    s = ConvShape(1, 4, 16, 64, 256, 256)
    with env_var("CONV3D_STREAMK", "1"), env_var("CONV3D_DYNAMIC", dynamic):
        p1 = c3d.conv3d_plan(conv_desc(s, c3d.CONV3D_F_BIAS | c3d.CONV3D_F_GN_STATS))
    assert p1.info().split_tiles > 0 and p1.info().gn_stats_slots > 0
    p2 = c3d.conv3d_plan(conv_desc(s, c3d.CONV3D_F_BIAS | c3d.CONV3D_F_RESIDUAL))
    d = workloads.block_inputs(s, 1550)
    params = {k: dev(d[k]) for k in ("gamma1", "beta1", "w1", "b1", "gamma2", "beta2", "w2", "b2")}
    graphed, eager = StatsBlockBuffers(s, p1, p2, params), StatsBlockBuffers(s, p1, p2, params)
    graphed.x.copy_(dev(d["x"]))
    g = capture(graphed.run)
    for k in range(REPLAYS):
        xk = dev(workloads.normal_f16(np.random.SeedSequence(1560 + k), s.x_shape))
        graphed.x.copy_(xk)
        g.replay()
        eager.x.copy_(xk)
        eager.run()
        torch.cuda.synchronize()
        for name in ("a1", "c1", "a2", "out"):
            assert torch.equal(bits(getattr(graphed, name)), bits(getattr(eager, name))), (k, name)
