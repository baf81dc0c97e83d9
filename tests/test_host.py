"""Host-side checks that need no GPU: the benchmark's one-GPU contract, the
seeded input generators and the entry-point module."""
import os
import subprocess
import sys

import numpy as np

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True,
                          text=True, timeout=120, env=e)


def test_bench_refuses_more_than_one_gpu():
    r = run_bench(["--gpus", "2"])
    assert r.returncode == 2 and "one GPU" in r.stderr
    r = run_bench([], env={"WORLD_SIZE": "2"})
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_generators_are_deterministic_and_shaped():
    ss = lambda: np.random.SeedSequence(77)
    a, b = workloads.normal_f16(ss(), (3, 5, 7, 16)), workloads.normal_f16(ss(), (3, 5, 7, 16))
    assert a.dtype == np.float16 and a.shape == (3, 5, 7, 16) and np.array_equal(a.view(np.uint16), b.view(np.uint16))
    t = workloads.ternary_f16(ss(), (4, 1000))
    assert set(np.unique(t).tolist()) == {-1.0, 0.0, 1.0}
    assert np.array_equal(t, workloads.ternary_f16(ss(), (4, 1000)))
    bf = workloads.normal_f16(ss(), (64,), dtype="bf16")
    assert bf.dtype == np.uint16
    # inputs of one workload do not depend on which other tensors were drawn
    d1 = workloads.conv_inputs(workloads.SMALL_ZERO, 5)
    d2 = workloads.conv_inputs(workloads.SMALL_ZERO, 5)
    assert all(np.array_equal(d1[k], d2[k]) for k in ("x", "w", "b"))


def test_entry_module_exposes_build_and_smoke():
    sys.path.insert(0, ROOT)
    import __graft_entry__ as g
    assert callable(g.build) and callable(g.smoke)


def test_bench_parity_gate_passes_the_oracle_and_fails_a_planted_error():
    # the gate's host logic on a small causal conv: an output equal to the oracle's, rounded
    # to fp16, passes; the same output with one wrong element (planted on the CPU) fails
    import torch
    sys.path.insert(0, ROOT)
    import bench
    import oracle
    s = workloads.ConvShape(1, 3, 8, 8, 16, 16)
    d = workloads.conv_inputs(s, 4242)
    x64, w64, b64 = (d[k].astype(np.float64) for k in ("x", "w", "b"))
    ref, _ = oracle.conv3d(x64, w64, b64, None, s.pads, s.tmode)
    y = torch.from_numpy(ref.astype(np.float16))
    gate = bench.parity_gate(s, x64, w64, b64, y, torch, np)
    assert gate["passed"] and gate["outputs_checked"] == gate["voxels"] * s.cout
    bad = y.clone()
    bad.view(-1, s.cout)[0, 3] += 0.5   # voxel 0 is a corner voxel: always in the gate's sample
    assert not bench.parity_gate(s, x64, w64, b64, bad, torch, np)["passed"]
