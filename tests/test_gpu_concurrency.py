"""One plan shared by two host threads, each with its own stream, workspace and
inputs, issuing calls concurrently (the header's contract: a plan is immutable
and shareable; calls on different streams must not share a workspace).  Every
output must equal a sequential run on the same inputs bit for bit.  The plan
splits K, so both streams also run the fixup kernel over their own partials."""
import threading

import numpy as np
import pytest
import torch

import convolution_implicit_gemm_amd as c3d
import workloads
from workloads import ConvShape

from helpers import conv_desc, dev, env_var, forced_tile, out_dims, workspace_for

pytestmark = pytest.mark.gpu

ROUNDS = 6


def test_shared_plan_on_two_streams_from_two_threads():
    s = ConvShape(1, 3, 20, 24, 128, 128)
    with forced_tile("m256n256k64s2a3w8"), env_var("CONV3D_STREAMK", "1"):
        plan = c3d.conv3d_plan(conv_desc(s, c3d.CONV3D_F_BIAS))
    assert plan.info().split_tiles > 0
    d = workloads.conv_inputs(s, 1600)
    w, b = dev(d["w"]), dev(d["b"])
    xs = [[dev(workloads.normal_f16(np.random.SeedSequence(1610 + 10 * t + r), s.x_shape)) for r in range(ROUNDS)]
          for t in range(2)]
    # sequential reference
    ref = []
    ws = workspace_for(plan)
    for t in range(2):
        row = []
        for r in range(ROUNDS):
            y = torch.empty(out_dims(s), dtype=torch.float16, device="cuda:0")
            c3d.conv3d_forward(plan, xs[t][r], w, b, None, y, ws)
            row.append(y)
        ref.append(row)
    torch.cuda.synchronize()
    # concurrent: thread t enqueues all its rounds on its own stream and workspace
    outs = [[torch.empty(out_dims(s), dtype=torch.float16, device="cuda:0") for _ in range(ROUNDS)]
            for _ in range(2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    spaces = [workspace_for(plan), workspace_for(plan)]
    errors = []
    start = threading.Barrier(2)

    def worker(t):
        try:
            torch.cuda.set_device(0)
            start.wait()
            with torch.cuda.stream(streams[t]):
                for r in range(ROUNDS):
                    c3d.conv3d_forward(plan, xs[t][r], w, b, None, outs[t][r], spaces[t])
        except Exception as e:  # reported in the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=60)
    torch.cuda.synchronize()
    assert not errors, errors
    for t in range(2):
        for r in range(ROUNDS):
            assert torch.equal(outs[t][r].view(torch.int16), ref[t][r].view(torch.int16)), (t, r)
