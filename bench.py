#!/usr/bin/env python3
"""Benchmark of the fp16 implicit-GEMM conv3d on one MI355X.

One step = one conv3d_forward of the largest 3x3x3 workload: the causal conv
N=1, T=33, H=W=256, Cin=512 -> Cout=256, fp16 NDHWC, bias, inputs resident in
HBM.  Before anything is timed, the output of that forward is checked against
the fp64 oracle (every channel at 1024 seeded voxels and the edge voxels of
the first, second and last frames, and at the CPU-baseline slab); if it does
not match, the line carries value null and the script exits 1.

Prints ONE JSON line: value = conv TFLOP/s (2*M*Cout*K / wall time per step),
a roofline object for the conv kernel (HIP events on its launch stream, and
the mean shader clock over the timed steps from clock stamps around them),
the oracle timed on a contiguous slab of the same workload on the host cores
(cpu_baseline, extrapolated to the whole conv), the 3D ResNet decoder-block
time in ms (GN+SiLU, causal conv, GN+SiLU, causal conv + x; N=1, C=256, T=17,
128x128), and per-kernel figures of the other hot-path kernels under
"kernels".

It ends with the machine's own ceilings (conv3d_calibrate_mfma / _hbm: dense
fp16 MFMA on random operands with the shader clock, HBM read and copy), and
each roofline figure is also given as a fraction of those.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--cpu-seconds S]
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP16_TFLOPS = 2516.6   # MI355X dense fp16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
CU_FLOP_PER_CLK = 256 * 4096  # dense fp16 MFMA flop per shader clock over the 256 CUs


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("conv3d_igemm.hip", "conv3d_ps.hip", "igemm_common.h", "c3d_internal.h"):
        with open(os.path.join(ROOT, "convolution_implicit_gemm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel, src_hash, grid):
    """HBM bytes per launch of the headline conv from the committed counter summary, if it
    was taken on this kernel source, kernel configuration and launch size."""
    path = os.path.join(ROOT, "profiles", "conv3d_causal512to256_T33_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"source_sha256_16:\s*([0-9a-f]+)", text)
    m_ker = re.search(r"kernel:\s*(\S+)", text)
    m_grid = re.search(r"grid:\s*(\d+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_src and m_ker and m_b and m_grid) or m_src.group(1) != src_hash or m_ker.group(1) != kernel \
            or int(m_grid.group(1)) != grid:
        return None
    return float(m_b.group(1))


def time_steps(fn, steps, warmup, torch, min_warm_s=0.0, stamps=None):
    """Wall time per call of `steps` calls between device syncs, and per-call HIP-event times (ms).

    Warm-up runs at least `warmup` calls and at least `min_warm_s` seconds of them (the shader
    clock settles under sustained load).  stamps: (c3d, before, after) device buffers for
    conv3d_clock_stamp around the timed calls, on the same stream.  Returns (ms, per, warm_calls).
    """
    stream = torch.cuda.current_stream()
    warm = 0
    t0 = time.perf_counter()
    while warm < warmup or time.perf_counter() - t0 < min_warm_s:
        fn()
        warm += 1
        if warm % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    if stamps:
        stamps[0].conv3d_clock_stamp(stamps[1], stream=stream)
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    if stamps:
        stamps[0].conv3d_clock_stamp(stamps[2], stream=stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [a.elapsed_time(b) for a, b in ev]
    return wall * 1e3 / steps, per, warm


def ws_for(plan, torch, dev):
    if not plan.workspace_bytes:
        return None
    return torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)


def desc_of(c3d, s, flags):
    return c3d.make_desc(s.n, s.t, s.h, s.w, s.cin, s.cout, s.kt, s.kh, s.kw, s.pad_t_front,
                         s.pad_t_back, s.pad_h, s.pad_w, s.tmode, flags)


def out_dims(s):
    return (s.n, s.t + s.pad_t_front + s.pad_t_back - s.kt + 1, s.h + 2 * s.pad_h - s.kh + 1,
            s.w + 2 * s.pad_w - s.kw + 1, s.cout)


def oracle_check(s, x64, w, b, y_dev, vox, torch, np, ref_mag=None):
    """Every channel at output voxels `vox`: (outputs checked, worst err/bound, all within bound).
    ref_mag: the oracle's (values, magnitudes) at those outputs, if already computed."""
    import oracle
    vt = torch.from_numpy(np.ascontiguousarray(vox)).to(y_dev.device)
    got = y_dev.reshape(-1, s.cout).index_select(0, vt).cpu().numpy().astype(np.float64).reshape(-1)
    if ref_mag is None:
        m = np.repeat(vox, s.cout)
        co = np.tile(np.arange(s.cout), vox.size)
        ref_mag = oracle.conv3d_points(x64, w, b, None, s.pads, s.tmode, m, co)
    ref, mag = ref_mag
    a = np.abs(ref)
    ulp = np.exp2(np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -14) - 10)
    bound = 2e-3 * mag + ulp
    err = np.abs(got - ref)
    return int(got.size), float(np.max(err / bound)), bool(np.all(err <= bound))


def parity_gate(s, x64, w, b, y_dev, torch, np):
    """The output of the forward about to be timed against the fp64 oracle, before any timing:
    every channel at 1024 seeded voxels and at the corner/edge voxels of the first, second and
    last output frames."""
    to, ho, wo = s.t + s.pad_t_front + s.pad_t_back - s.kt + 1, s.h, s.w
    m_total = s.n * to * ho * wo
    rng = np.random.default_rng(20260)
    edges = [((n * to + t) * ho + h) * wo + ww for n in {0, s.n - 1} for t in sorted({0, 1, to - 1})
             for h in sorted({0, ho // 2, ho - 1}) for ww in sorted({0, wo // 2, wo - 1})]
    vox = np.union1d(rng.choice(m_total, min(1024, m_total), replace=False), np.asarray(edges, dtype=np.int64))
    n, worst, ok = oracle_check(s, x64, w, b, y_dev, vox, torch, np)
    return {"outputs_checked": n, "voxels": int(vox.size), "worst_err_over_bound": round(worst, 4),
            "bound": "|gpu - oracle| <= 2e-3 * sum|x*w| + 1 fp16 ulp", "passed": ok}


def cpu_baseline_leg(s, x64, w, b, y_dev, info, target_s, torch, np):
    """Time the fp64 oracle on a contiguous slab of output voxels (every channel), sized from a
    probe to about target_s seconds, and extrapolate to the whole conv; the GPU output is
    checked on the same slab.  Per-voxel work is the same everywhere (replicate padding keeps
    every temporal tap inside the input), so scaling the slab time by M / slab is exact up
    to cache effects."""
    import oracle
    to = s.t + s.pad_t_front + s.pad_t_back - s.kt + 1
    m_total = int(info.gemm_m)
    first = (to // 2) * s.h * s.w       # a middle frame

    def run(nvox):
        m = np.repeat(np.arange(first, first + nvox, dtype=np.int64), s.cout)
        co = np.tile(np.arange(s.cout), nvox)
        t0 = time.perf_counter()
        ref_mag = oracle.conv3d_points(x64, w, b, None, s.pads, s.tmode, m, co)
        return time.perf_counter() - t0, ref_mag

    probe = 64
    per_vox = max(run(probe)[0] / probe, 1e-6)
    nvox = int(min(m_total - first, max(256, target_s / per_vox)))
    dt, ref_mag = run(nvox)
    k = s.kt * s.kh * s.kw * s.cin
    flops = 2.0 * k * nvox * s.cout
    n, worst, ok = oracle_check(s, x64, w, b, y_dev, np.arange(first, first + nvox, dtype=np.int64), torch, np,
                                ref_mag)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "extrapolated: a contiguous slab of %d output voxels from the middle frame x all %d "
                      "channels (%.3g GFLOP of %.4g), fp64 seven-loop oracle, %.1f s wall; whole conv "
                      "extrapolated to %.0f s" % (nvox, s.cout, flops / 1e9, info.flops / 1e9, dt,
                                                  dt * info.flops / flops),
            "seconds": dt, "seconds_whole_conv_extrapolated": dt * info.flops / flops,
            "gpu_matches_oracle_on_sample": ok, "sample_worst_err_over_bound": round(worst, 4),
            "host_cpu": cpu_model(), "affinity_cores": len(os.sched_getaffinity(0))}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=5,
                    help="untimed steps first (at least --warm-seconds of them)")
    ap.add_argument("--warm-seconds", type=float, default=1.5,
                    help="least seconds of warm-up load before each timed run: the shader clock "
                         "needs sustained load to settle, whatever --warmup says")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="wall seconds of oracle work for cpu_baseline (0 skips it; the parity "
                         "gate before timing runs regardless)")
    ap.add_argument("--no-kernels", action="store_true", help="skip the per-kernel extras")
    ap.add_argument("--extras", default="all",
                    help="comma list of per-kernel extras to run: conv512 (the 9-frame 64x64 512-channel "
                         "conv), block (the decoder block), conv256, groupnorm, bf16, t1, t1zero (the "
                         "zero-causal first frame), chunk (the block conv decoded in chunks), pointwise "
                         "(the 1x1x1 256->128 on the headline's output), gemm (the vendor GEMM on the "
                         "512-channel conv's M x N x K, for context), or all")
    ap.add_argument("--no-calibration", action="store_true",
                    help="skip the MFMA / HBM ceiling measurements at the end")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="end with one 1 GiB device-to-device copy (scales byte counters in profiles)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import convolution_implicit_gemm_amd as c3d
    import workloads

    c3d.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def T(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    nstamp = c3d.conv3d_clock_stamp_bytes()
    st_before = torch.zeros(nstamp, dtype=torch.uint8, device=dev)
    st_after = torch.zeros_like(st_before)

    def sclk(before, after):
        mhz = c3d.sclk_between(before.cpu().numpy().view(np.uint64), after.cpu().numpy().view(np.uint64))
        vals = list(mhz.values())
        return (sum(vals) / len(vals) if vals else None), mhz

    # ---- headline: causal conv3d 3x3x3, 512 -> 256, T=33, 256x256 (the largest 3x3x3 workload)
    log("generating the 33-frame 256x256 512->256 workload (2.2 GB input)")
    d3 = workloads.workload_inputs(3)
    s3 = d3["shape"]
    plan = c3d.conv3d_plan(desc_of(c3d, s3, c3d.CONV3D_F_BIAS))
    info = plan.info()
    x, w, b = T(d3["x"]), T(d3["w"]), T(d3["b"])
    y = torch.empty(out_dims(s3), dtype=torch.float16, device=dev)
    ws = ws_for(plan, torch, dev)

    def step():
        c3d.conv3d_forward(plan, x, w, b, None, y, ws)

    kname = info.kernel_name.decode()
    src_hash = kernel_source_hash()
    workload = ("causal conv3d 3x3x3 (first frame replicated twice in front, spatial zero pad 1), "
                "N=1 T=33 H=W=256 Cin=512 -> Cout=256, fp16 NDHWC, bias; 5 input channels x50")
    result = {
        "metric": "fp16 conv3d 3x3x3 TFLOP/s on 1 MI355X (% of fp16 MFMA peak); decoder-block ms",
        "value": None, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": None, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic (seeded N(0,1) activations, Kaiming-uniform fp16 weights)",
        "config": {"workload": workload, "gemm_m": int(info.gemm_m), "gemm_n": int(info.gemm_n),
                   "gemm_k": int(info.gemm_k), "kernel": kname, "grid": int(info.grid),
                   "parallelism": "single GPU"},
    }

    # parity gate: the forward about to be timed, against the oracle, before any timing
    log("parity gate: one forward against the fp64 oracle")
    step()
    torch.cuda.synchronize()
    x64 = d3["x"].astype(np.float64)
    w64, b64 = d3["w"].astype(np.float64), d3["b"].astype(np.float64)
    gate = parity_gate(s3, x64, w64, b64, y, torch, np)
    result["parity_gate"] = gate
    if args.cpu_seconds > 0:
        log("cpu baseline: oracle on a contiguous slab of the headline conv")
        cb = cpu_baseline_leg(s3, x64, w64, b64, y, info, args.cpu_seconds, torch, np)
        result["cpu_baseline"] = cb
        gate["passed"] = gate["passed"] and cb["gpu_matches_oracle_on_sample"]
    else:
        result["cpu_baseline"] = None
    del x64, w64, b64
    if not gate["passed"]:
        log("parity gate FAILED: no timing is reported for an output that does not match the oracle")
        print(json.dumps(result), flush=True)
        sys.exit(1)

    log("timing %d steps after at least %d warm-up steps and %.1f s" % (args.steps, args.warmup,
                                                                        args.warm_seconds))
    ms, per, warm = time_steps(step, args.steps, args.warmup, torch, args.warm_seconds,
                               (c3d, st_before, st_after))
    mhz, per_xcd = sclk(st_before, st_after)
    kernel_ms = sum(per) / len(per)
    per_sorted = sorted(per)
    value = info.flops / (ms * 1e-3) / 1e12
    achieved = info.flops / (kernel_ms * 1e-3) / 1e12
    result["value"] = round(value, 2)
    result["ms_per_step"] = round(ms, 4)
    result["warmup_steps_run"] = warm
    result["roofline"] = {
        "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_FP16_TFLOPS, 4),
        "traffic": committed_traffic(kname, src_hash, int(info.grid)),
        "kernel_ms": round(kernel_ms, 4), "source_sha256_16": src_hash,
        "sclk_mhz_timed": None if mhz is None else round(mhz, 1),
        "frac_of_peak_at_timed_sclk": None if mhz is None else round(achieved / (CU_FLOP_PER_CLK * mhz / 1e6), 4)}
    result["timing"] = {"launch_ms_mean": round(kernel_ms, 4),
                        "launch_ms_median": round(per_sorted[len(per) // 2], 4),
                        "launch_ms_min": round(per_sorted[0], 4), "launches": len(per),
                        "clock": "HIP events on the launch stream, one pair per step",
                        "sclk_mhz_per_xcd": {str(k): round(v, 1) for k, v in per_xcd.items()}}

    extras = ({"conv512", "block", "conv256", "groupnorm", "bf16", "t1", "t1zero", "chunk", "pointwise", "gemm"}
              if args.extras == "all" else set(args.extras.split(",")))
    kern = {}

    def conv_extra(name, plan_, fn, steps=20, warmup=5):
        _, p, _ = time_steps(fn, steps, warmup, torch, 0.3, (c3d, st_before, st_after))
        t = sum(p) / len(p)
        f = plan_.info().flops / (t * 1e-3) / 1e12
        mhz_, _ = sclk(st_before, st_after)
        kern[name] = {"ms": round(t, 4), "TFLOP/s": round(f, 1), "frac": round(f / PEAK_FP16_TFLOPS, 4),
                      "sclk_mhz": None if mhz_ is None else round(mhz_, 1),
                      "kernel": plan_.info().kernel_name.decode(), "grid": int(plan_.info().grid)}

    if not args.no_kernels and "pointwise" in extras:
        # 1x1x1 256 -> 128 on the headline's own output (the channel-changing stage's second conv)
        s3b = d3["shape2"]
        p3b = c3d.conv3d_plan(desc_of(c3d, s3b, c3d.CONV3D_F_BIAS))
        w3b, b3b = T(d3["w2"]), T(d3["b2"])
        y3b = torch.empty(out_dims(s3b), dtype=torch.float16, device=dev)

        def st2():
            c3d.conv3d_forward(p3b, y, w3b, b3b, None, y3b)
        _, p, _ = time_steps(st2, 20, 5, torch, 0.3)
        t = sum(p) / len(p)
        pw_bytes = y.numel() * 2 + y3b.numel() * 2 + w3b.numel() * 2
        kern["pointwise_256to128_T33_256x256"] = {"ms": round(t, 4), "GB/s": round(pw_bytes / t / 1e6, 1),
                                                  "frac_of_hbm": round(pw_bytes / t / 1e6 / PEAK_HBM_GBS, 3),
                                                  "kernel": p3b.info().kernel_name.decode()}
        del y3b
    del x, y, d3

    if not args.no_kernels and ("conv512" in extras or "gemm" in extras or "bf16" in extras):
        d1 = workloads.workload_inputs(1)
        s1 = d1["shape"]
        p1 = c3d.conv3d_plan(desc_of(c3d, s1, c3d.CONV3D_F_BIAS))
        x1, w1, b1 = T(d1["x"]), T(d1["w"]), T(d1["b"])
        y1 = torch.empty(out_dims(s1), dtype=torch.float16, device=dev)
        ws1 = ws_for(p1, torch, dev)
        if "conv512" in extras:
            conv_extra("causal_conv_512_T9_64x64", p1,
                       lambda: c3d.conv3d_forward(p1, x1, w1, b1, None, y1, ws1), steps=100, warmup=50)
        if "bf16" in extras:
            d1b = workloads.conv_inputs(s1, 1001, dtype="bf16")
            pb = c3d.conv3d_plan(desc_of(c3d, s1, c3d.CONV3D_F_BIAS | c3d.CONV3D_F_BF16))
            wsb = ws_for(pb, torch, dev)

            def bfT(a):
                return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
            xb, wb, bb = bfT(d1b["x"]), bfT(d1b["w"]), bfT(d1b["b"])
            yb = torch.empty(out_dims(s1), dtype=torch.bfloat16, device=dev)
            conv_extra("causal_conv_512_T9_64x64_bf16", pb,
                       lambda: c3d.conv3d_forward(pb, xb, wb, bb, None, yb, wsb), steps=100, warmup=50)
            del xb, wb, bb, yb, wsb, d1b
        if "gemm" in extras:
            # context only ("FLOPs parity"): the vendor GEMM (torch.matmul on hipBLASLt) on a dense
            # fp16 matrix of the 512-channel conv's im2col shape, M x K times K x N.  The conv never
            # builds such a matrix.
            i1 = p1.info()
            gm, gk, gn = i1.gemm_m, i1.gemm_k, i1.gemm_n
            ga = torch.randn(gm, gk, device=dev, dtype=torch.float16)
            gb = torch.randn(gk, gn, device=dev, dtype=torch.float16)
            gc = torch.empty(gm, gn, device=dev, dtype=torch.float16)
            _, p, _ = time_steps(lambda: torch.matmul(ga, gb, out=gc), 30, 10, torch, 0.3)
            t = sum(p) / len(p)
            kern["vendor_gemm_same_mnk_as_512_T9"] = {
                "ms": round(t, 4), "TFLOP/s": round(2.0 * gm * gn * gk / t / 1e9, 1), "shape_m_k_n": [gm, gk, gn],
                "gemm_ms_over_conv_ms": round(t / kern["causal_conv_512_T9_64x64"]["ms"], 3)
                if "causal_conv_512_T9_64x64" in kern else None}
            del ga, gb, gc
        del x1, y1, ws1, d1

    # ---- decoder block: GN+SiLU -> causal conv -> GN+SiLU -> causal conv + x
    d4 = workloads.workload_inputs(4)
    s4 = d4["shape"]
    thw = s4.t * s4.h * s4.w
    bp1 = c3d.conv3d_plan(desc_of(c3d, s4, c3d.CONV3D_F_BIAS))
    bp2 = c3d.conv3d_plan(desc_of(c3d, s4, c3d.CONV3D_F_BIAS | c3d.CONV3D_F_RESIDUAL))
    bws1, bws2 = ws_for(bp1, torch, dev), ws_for(bp2, torch, dev)
    gws = torch.zeros(c3d.groupnorm_silu_workspace(1, thw, s4.cin, 32), dtype=torch.uint8, device=dev)
    bx = T(d4["x"])
    bt = {k: T(d4[k]) for k in ("gamma1", "beta1", "w1", "b1", "gamma2", "beta2", "w2", "b2")}
    a1, c1, a2, out = (torch.empty_like(bx) for _ in range(4))

    def block():
        c3d.groupnorm_silu(bx, bt["gamma1"], bt["beta1"], a1, 1, thw, s4.cin, 32, 1e-6, True, gws)
        c3d.conv3d_forward(bp1, a1, bt["w1"], bt["b1"], None, c1, bws1)
        c3d.groupnorm_silu(c1, bt["gamma2"], bt["beta2"], a2, 1, thw, s4.cout, 32, 1e-6, True, gws)
        c3d.conv3d_forward(bp2, a2, bt["w2"], bt["b2"], bx, out, bws2)

    if "block" in extras or args.no_kernels:
        # The block as measured: GN2's statistics taken in conv1's epilogue
        # (CONV3D_F_GN_STATS) and GN2 normalising from them; the six-launch
        # form (GN2 with its own statistics pass) is reported beside it.
        bp1s = c3d.conv3d_plan(desc_of(c3d, s4, c3d.CONV3D_F_BIAS | c3d.CONV3D_F_GN_STATS))
        bws1s = ws_for(bp1s, torch, dev)
        sst, sslots = c3d.gn_stats_view(bp1s, bws1s)
        sws = torch.empty(c3d.groupnorm_silu_from_stats_workspace(1, s4.cout, 32), dtype=torch.uint8, device=dev)

        def gn1():
            c3d.groupnorm_silu(bx, bt["gamma1"], bt["beta1"], a1, 1, thw, s4.cin, 32, 1e-6, True, gws)

        def conv1_stats():
            c3d.conv3d_forward(bp1s, a1, bt["w1"], bt["b1"], None, c1, bws1s)

        def gn2_from_stats():
            c3d.groupnorm_silu_from_stats(c1, bt["gamma2"], bt["beta2"], a2, 1, thw, s4.cout, 32, 1e-6, True,
                                          sst, sslots, sws)

        def conv1():
            c3d.conv3d_forward(bp1, a1, bt["w1"], bt["b1"], None, c1, bws1)

        def gn2():
            c3d.groupnorm_silu(c1, bt["gamma2"], bt["beta2"], a2, 1, thw, s4.cout, 32, 1e-6, True, gws)

        def conv2():
            c3d.conv3d_forward(bp2, a2, bt["w2"], bt["b2"], bx, out, bws2)

        def block_stats():
            gn1()
            conv1_stats()
            gn2_from_stats()
            conv2()

        def breakdown(calls):
            # events between the four calls, averaged over 20 blocks
            stream = torch.cuda.current_stream()
            parts = {name: [] for name, _ in calls}
            for _ in range(20):
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
                ev[0].record(stream)
                for k, (_, fn) in enumerate(calls):
                    fn()
                    ev[k + 1].record(stream)
                torch.cuda.synchronize()
                for k, (name, _) in enumerate(calls):
                    parts[name].append(ev[k].elapsed_time(ev[k + 1]))
            return {k: round(sum(v) / len(v), 4) for k, v in parts.items()}

        log("decoder block, GN2 from conv1's statistics")
        _, bper, _ = time_steps(block_stats, 20, 5, torch, args.warm_seconds)
        result["decoder_block_ms"] = round(sum(bper) / len(bper), 4)
        result["decoder_block_breakdown_ms"] = breakdown([("gn1", gn1), ("conv1_with_gn2_stats", conv1_stats),
                                                          ("gn2_from_conv1_stats", gn2_from_stats),
                                                          ("conv2_plus_x", conv2)])
        log("decoder block, six launches")
        _, bper, _ = time_steps(block, 20, 5, torch, args.warm_seconds)
        result["decoder_block_six_launch_ms"] = round(sum(bper) / len(bper), 4)
        result["decoder_block_six_launch_breakdown_ms"] = breakdown([("gn1", gn1), ("conv1", conv1), ("gn2", gn2),
                                                                     ("conv2_plus_x", conv2)])
        result["decoder_block_config"] = ("GN(32, eps 1e-6)+SiLU -> causal conv3d 3x3x3 -> GN+SiLU -> "
                                          "causal conv3d 3x3x3 -> +x; N=1 C=256 T=17 H=W=128 fp16; "
                                          "decoder_block_ms: the second GroupNorm's statistics taken in the first "
                                          "conv's epilogue (CONV3D_F_GN_STATS + groupnorm_silu_from_stats)")

    if not args.no_kernels and "conv256" in extras:
        conv_extra("causal_conv_256_T17_128x128", bp1,
                   lambda: c3d.conv3d_forward(bp1, a1, bt["w1"], bt["b1"], None, c1, bws1), steps=40, warmup=20)

    if not args.no_kernels and "groupnorm" in extras:
        # three input copies in rotation (428 MB > the 256 MB MALL), so no call
        # finds its input already cached by the previous one
        gx = [bx, bx.clone(), bx.clone()]
        gi = [0]

        def gn_only():
            c3d.groupnorm_silu(gx[gi[0] % 3], bt["gamma1"], bt["beta1"], a1, 1, thw, s4.cin, 32,
                               1e-6, True, gws)
            gi[0] += 1
        _, p, _ = time_steps(gn_only, 30, 6, torch, 0.3)
        p = sorted(p)
        t = p[len(p) // 2]
        # the same calls back to back, 60 of them between one pair of events: the
        # time per call without an event pair around each one
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(torch.cuda.current_stream())
        for _ in range(60):
            gn_only()
        e1.record(torch.cuda.current_stream())
        torch.cuda.synchronize()
        tb = e0.elapsed_time(e1) / 60
        sbytes = bx.numel() * 2
        kern["groupnorm_silu_256_T17"] = {"ms_median": round(t, 4), "ms_min": round(p[0], 4),
                                          "GB/s_effective_2S": round(2 * sbytes / t / 1e6, 1),
                                          "GB/s_as_implemented_3S": round(3 * sbytes / t / 1e6, 1),
                                          "frac_of_hbm_2S": round(2 * sbytes / t / 1e6 / PEAK_HBM_GBS, 3),
                                          "frac_of_hbm_3S": round(3 * sbytes / t / 1e6 / PEAK_HBM_GBS, 3),
                                          "ms_back_to_back": round(tb, 4),
                                          "frac_of_hbm_2S_back_to_back": round(2 * sbytes / tb / 1e6 / PEAK_HBM_GBS, 3),
                                          "frac_of_hbm_3S_back_to_back": round(3 * sbytes / tb / 1e6 / PEAK_HBM_GBS, 3),
                                          "inputs": "3 copies in rotation"}
        del gx

    if not args.no_kernels and "t1" in extras:
        s1f = workloads.CAUSAL_256_T1
        pt1 = c3d.conv3d_plan(desc_of(c3d, s1f, c3d.CONV3D_F_BIAS))
        wst = ws_for(pt1, torch, dev)
        xt = bx[:, :1].contiguous()
        yt = torch.empty(out_dims(s1f), dtype=torch.float16, device=dev)
        _, p, _ = time_steps(lambda: c3d.conv3d_forward(pt1, xt, bt["w1"], bt["b1"], None, yt, wst), 50, 10,
                             torch, 0.2)
        t = sum(p) / len(p)
        kern["first_frame_fold_256"] = {"us": round(t * 1e3, 2),
                                        "TFLOP/s_folded": round(pt1.info().flops / t / 1e9, 1),
                                        "path": int(pt1.info().path), "grid": int(pt1.info().grid),
                                        "kernel": pt1.info().kernel_name.decode()}
        del xt, yt, wst

    if not args.no_kernels and "t1zero" in extras:
        # the zero-causal first frame: only the last temporal tap sees data
        s1z = dataclasses.replace(workloads.CAUSAL_256_T1, tmode=workloads.TPAD_ZERO)
        ptz = c3d.conv3d_plan(desc_of(c3d, s1z, c3d.CONV3D_F_BIAS))
        wsz = ws_for(ptz, torch, dev)
        xz = bx[:, :1].contiguous()
        yz = torch.empty(out_dims(s1z), dtype=torch.float16, device=dev)
        _, p, _ = time_steps(lambda: c3d.conv3d_forward(ptz, xz, bt["w1"], bt["b1"], None, yz, wsz), 50, 10,
                             torch, 0.2)
        t = sum(p) / len(p)
        kern["first_frame_zero_causal_256"] = {"us": round(t * 1e3, 2),
                                               "TFLOP/s_one_tap": round(ptz.info().flops / t / 1e9, 1),
                                               "path": int(ptz.info().path)}
        del xz, yz, wsz

    if not args.no_kernels and "chunk" in extras:
        # the 17-frame block conv decoded as chunks of 5, 4, 4 and 4 frames: the
        # first with the causal plan, each later one with the previous chunk's
        # last two input frames as history (the same output as the whole conv)
        sizes = [5, 4, 4, 4]
        cplans, t0 = [], 0
        for k, tc in enumerate(sizes):
            sc = dataclasses.replace(s4, t=tc)
            fl = c3d.CONV3D_F_BIAS | (c3d.CONV3D_F_CHUNK if k else 0)
            pc = c3d.conv3d_plan(desc_of(c3d, sc, fl))
            cplans.append((pc, ws_for(pc, torch, dev), t0, tc))
            t0 += tc

        def chunked():
            for k, (pc, wsc, a, tc) in enumerate(cplans):
                if k == 0:
                    c3d.conv3d_forward(pc, bx[:, a:a + tc], bt["w1"], bt["b1"], None, c1[:, a:a + tc], wsc)
                else:
                    c3d.conv3d_forward_chunk(pc, bx[:, a - 2:a], bx[:, a:a + tc], bt["w1"], bt["b1"], None,
                                             c1[:, a:a + tc], wsc)
        _, p, _ = time_steps(chunked, 10, 2, torch, 0.3)
        t = sum(p) / len(p)
        conv_flops = bp1.info().flops
        kern["chunked_causal_conv_256_T17_as_5_4_4_4"] = {
            "ms": round(t, 4), "TFLOP/s": round(conv_flops / t / 1e9, 1),
            "ms_over_whole_conv": round(t / kern["causal_conv_256_T17_128x128"]["ms"], 3)
            if "causal_conv_256_T17_128x128" in kern else None}
        del cplans
    del a1, c1, a2, out, bx
    if not args.no_kernels:
        result["kernels"] = kern

    if not args.no_calibration:
        log("machine ceilings: MFMA on random operands, HBM read and copy")
        scratch = torch.empty(c3d.conv3d_calibrate_scratch_bytes(), dtype=torch.uint8, device=dev)
        mfma_tf, cal_mhz = c3d.conv3d_calibrate_mfma(scratch)
        del scratch
        nb = 2 << 30
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        src.fill_(1)
        dst = torch.empty_like(src)
        rd, cp = c3d.conv3d_calibrate_hbm(src, dst, nb)
        del src, dst
        result["calibration"] = {"mfma_fp16_tflops_random_operands": round(mfma_tf, 1),
                                 "sclk_mhz_during_mfma": round(cal_mhz, 0),
                                 "hbm_read_gbs": round(rd, 1), "hbm_copy_gbs_read_plus_write": round(cp, 1)}
        rf = result["roofline"]
        rf["frac_of_measured"] = round(rf["achieved"] / mfma_tf, 4)
        k = result.get("kernels", {})
        if "pointwise_256to128_T33_256x256" in k:
            k["pointwise_256to128_T33_256x256"]["frac_of_measured_copy"] = round(
                k["pointwise_256to128_T33_256x256"]["GB/s"] / cp, 3)
        if "groupnorm_silu_256_T17" in k:
            k["groupnorm_silu_256_T17"]["frac_of_measured_copy_3S"] = round(
                k["groupnorm_silu_256_T17"]["GB/s_as_implemented_3S"] / cp, 3)

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        torch.empty_like(a).copy_(a)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = 1 << 30

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
