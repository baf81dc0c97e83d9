#!/usr/bin/env python3
"""Benchmark of the fp16 implicit-GEMM conv3d on one MI355X.

One step = one conv3d_forward of the causal 3x3x3 conv, N=1, T=9, H=W=64,
Cin=Cout=512, fp16 NDHWC, bias, inputs resident in HBM.  Prints ONE JSON line:
value = conv TFLOP/s (2*M*Cout*K / time), a roofline object for the conv
kernel (HIP events on its launch stream), the oracle timed on a bounded
sample of the same workload on the host cores (cpu_baseline), the 3D ResNet
decoder-block time in ms (GN+SiLU, causal conv, GN+SiLU, causal conv + x;
N=1, C=256, T=17, 128x128), and per-kernel figures of the other hot-path
kernels under "kernels".

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


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("conv3d_igemm.hip", "c3d_internal.h"):
        with open(os.path.join(ROOT, "convolution_implicit_gemm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel, src_hash):
    """HBM bytes per launch from the committed counter summary, if it matches this source."""
    path = os.path.join(ROOT, "profiles", "conv3d_causal512_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"source_sha256_16:\s*([0-9a-f]+)", text)
    m_ker = re.search(r"kernel:\s*(\S+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_src and m_ker and m_b) or m_src.group(1) != src_hash or m_ker.group(1) != kernel:
        return None
    return float(m_b.group(1))


def time_steps(fn, steps, warmup, torch):
    """Wall time of `steps` calls between device syncs, and per-call HIP-event times (ms)."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [a.elapsed_time(b) for a, b in ev]
    return wall * 1e3 / steps, per


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


def cpu_baseline_leg(d, y_dev, info, target_s, np):
    """Time the fp64 oracle on a bounded sample of the workload; check the GPU there too."""
    import oracle
    s = d["shape"]
    x64 = d["x"].astype(np.float64)
    w64 = d["w"].astype(np.float64)
    b64 = d["b"].astype(np.float64)
    k = s.kt * s.kh * s.kw * s.cin
    rng = np.random.default_rng(2024)
    m_total = int(info.gemm_m)

    def run(nvox):
        m = np.repeat(np.sort(rng.choice(m_total, nvox, replace=False)), s.cout)
        co = np.tile(np.arange(s.cout), nvox)
        t0 = time.perf_counter()
        ref, mag = oracle.conv3d_points(x64, w64, b64, None, s.pads, s.tmode, m, co)
        return time.perf_counter() - t0, m, co, ref, mag

    # size the sample from a probe large enough that thread start-up does not dominate it
    dt, *_ = run(64)
    per_vox = max(dt / 64, 1e-6)
    nvox = int(min(m_total, max(16, target_s / per_vox)))
    dt, m, co, ref, mag = run(nvox)
    flops = 2.0 * k * m.size
    got = y_dev.reshape(-1, s.cout)[m, co].astype(np.float64)
    a = np.abs(ref)
    ulp = np.exp2(np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -14) - 10)
    ok = bool(np.all(np.abs(got - ref) <= 2e-3 * mag + ulp))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "%d output voxels x all %d channels (%.3g GFLOP of %.3g), fp64 "
                      "seven-loop oracle, %.1f s wall" % (nvox, s.cout, flops / 1e9,
                                                          info.flops / 1e9, dt),
            "seconds": dt, "gpu_matches_oracle_on_sample": ok,
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
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps first; the clocks need ~50 ms of load to settle")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="wall seconds of oracle work for cpu_baseline (0 disables it)")
    ap.add_argument("--no-kernels", action="store_true", help="skip the per-kernel extras")
    ap.add_argument("--extras", default="all",
                    help="comma list of per-kernel extras to run: conv256, groupnorm, bf16, t1, t1zero "
                         "(the zero-causal first frame), chunk (the block conv decoded in chunks), stage "
                         "(the 33-frame 256x256 3x3x3 and 1x1x1 pair), gemm (the vendor GEMM on the "
                         "headline's M x N x K, for context), or all")
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

    # ---- headline: causal conv3d 3x3x3, 512 -> 512, T=9, 64x64
    log("generating the causal 512-channel workload")
    d1 = workloads.workload_inputs(1)
    s1 = d1["shape"]
    plan = c3d.conv3d_plan(desc_of(c3d, s1, c3d.CONV3D_F_BIAS))
    info = plan.info()
    x, w, b = T(d1["x"]), T(d1["w"]), T(d1["b"])
    y = torch.empty(out_dims(s1), dtype=torch.float16, device=dev)
    ws = ws_for(plan, torch, dev)

    def step():
        c3d.conv3d_forward(plan, x, w, b, None, y, ws)

    log("timing %d steps after %d warmup" % (args.steps, args.warmup))
    ms, per = time_steps(step, args.steps, args.warmup, torch)
    kernel_ms = sum(per) / len(per)
    per_sorted = sorted(per)
    value = info.flops / (ms * 1e-3) / 1e12
    achieved = info.flops / (kernel_ms * 1e-3) / 1e12
    kname = info.kernel_name.decode()
    src_hash = kernel_source_hash()
    result = {
        "metric": "fp16 conv3d 3x3x3 TFLOP/s on 1 MI355X (% of fp16 MFMA peak); decoder-block ms",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic (seeded N(0,1) activations, Kaiming-uniform fp16 weights)",
        "config": {"workload": "causal conv3d 3x3x3 (first frame replicated twice in front, "
                               "spatial zero pad 1), N=1 T=9 H=W=64 Cin=Cout=512, fp16 NDHWC",
                   "gemm_m": int(info.gemm_m), "gemm_n": int(info.gemm_n),
                   "gemm_k": int(info.gemm_k), "kernel": kname, "grid": int(info.grid),
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP16_TFLOPS, 4),
                     "traffic": committed_traffic(kname, src_hash),
                     "kernel_ms": round(kernel_ms, 4), "source_sha256_16": src_hash},
        "timing": {"launch_ms_mean": round(kernel_ms, 4),
                   "launch_ms_median": round(per_sorted[len(per) // 2], 4),
                   "launch_ms_min": round(per_sorted[0], 4), "launches": len(per),
                   "clock": "HIP events on the launch stream, one pair per step"},
    }

    # ---- decoder block: GN+SiLU -> causal conv -> GN+SiLU -> causal conv + x
    log("decoder block")
    d4 = workloads.workload_inputs(4)
    s4 = d4["shape"]
    thw = s4.t * s4.h * s4.w
    bp1 = c3d.conv3d_plan(desc_of(c3d, s4, c3d.CONV3D_F_BIAS))
    bp2 = c3d.conv3d_plan(desc_of(c3d, s4, c3d.CONV3D_F_BIAS | c3d.CONV3D_F_RESIDUAL))
    bws1, bws2 = ws_for(bp1, torch, dev), ws_for(bp2, torch, dev)
    gws = torch.zeros(c3d.groupnorm_silu_workspace(1, thw, s4.cin, 32), dtype=torch.uint8,
                      device=dev)
    bx = T(d4["x"])
    bt = {k: T(d4[k]) for k in ("gamma1", "beta1", "w1", "b1", "gamma2", "beta2", "w2", "b2")}
    a1, c1, a2, out = (torch.empty_like(bx) for _ in range(4))

    def block():
        c3d.groupnorm_silu(bx, bt["gamma1"], bt["beta1"], a1, 1, thw, s4.cin, 32, 1e-6, True, gws)
        c3d.conv3d_forward(bp1, a1, bt["w1"], bt["b1"], None, c1, bws1)
        c3d.groupnorm_silu(c1, bt["gamma2"], bt["beta2"], a2, 1, thw, s4.cout, 32, 1e-6, True, gws)
        c3d.conv3d_forward(bp2, a2, bt["w2"], bt["b2"], bx, out, bws2)

    bms, bper = time_steps(block, max(5, args.steps // 2), max(2, args.warmup), torch)
    result["decoder_block_ms"] = round(sum(bper) / len(bper), 4)
    # per-launch breakdown: events between the four calls, averaged over 20 blocks
    stream = torch.cuda.current_stream()
    parts = {"gn1": [], "conv1": [], "gn2": [], "conv2_plus_x": []}
    for _ in range(20):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        ev[0].record(stream)
        c3d.groupnorm_silu(bx, bt["gamma1"], bt["beta1"], a1, 1, thw, s4.cin, 32, 1e-6, True, gws)
        ev[1].record(stream)
        c3d.conv3d_forward(bp1, a1, bt["w1"], bt["b1"], None, c1, bws1)
        ev[2].record(stream)
        c3d.groupnorm_silu(c1, bt["gamma2"], bt["beta2"], a2, 1, thw, s4.cout, 32, 1e-6, True, gws)
        ev[3].record(stream)
        c3d.conv3d_forward(bp2, a2, bt["w2"], bt["b2"], bx, out, bws2)
        ev[4].record(stream)
        torch.cuda.synchronize()
        for k, name in enumerate(parts):
            parts[name].append(ev[k].elapsed_time(ev[k + 1]))
    result["decoder_block_breakdown_ms"] = {k: round(sum(v) / len(v), 4) for k, v in parts.items()}
    result["decoder_block_config"] = ("GN(32, eps 1e-6)+SiLU -> causal conv3d 3x3x3 -> GN+SiLU -> "
                                      "causal conv3d 3x3x3 -> +x; N=1 C=256 T=17 H=W=128 fp16")

    extras = ({"conv256", "groupnorm", "bf16", "t1", "t1zero", "chunk", "stage", "gemm"} if args.extras == "all"
              else set(args.extras.split(",")))
    if not args.no_kernels:
        kern = {}
        conv_flops = bp1.info().flops

    if not args.no_kernels and "conv256" in extras:
        def conv_only():
            c3d.conv3d_forward(bp1, a1, bt["w1"], bt["b1"], None, c1, bws1)
        _, p = time_steps(conv_only, 10, 2, torch)
        t = sum(p) / len(p)
        kern["causal_conv_256_T17"] = {"ms": round(t, 4), "TFLOP/s": round(conv_flops / t / 1e9, 1),
                                       "kernel": bp1.info().kernel_name.decode()}

    if not args.no_kernels and "groupnorm" in extras:
        # three input copies in rotation (428 MB > the 256 MB MALL), so no call
        # finds its input already cached by the previous one
        gx = [bx, bx.clone(), bx.clone()]
        gi = [0]

        def gn_only():
            c3d.groupnorm_silu(gx[gi[0] % 3], bt["gamma1"], bt["beta1"], a1, 1, thw, s4.cin, 32,
                               1e-6, True, gws)
            gi[0] += 1
        _, p = time_steps(gn_only, 30, 6, torch)
        p = sorted(p)
        t = p[len(p) // 2]
        sbytes = bx.numel() * 2
        kern["groupnorm_silu_256_T17"] = {"ms_median": round(t, 4), "ms_min": round(p[0], 4),
                                          "GB/s_effective_2S": round(2 * sbytes / t / 1e6, 1),
                                          "GB/s_as_implemented_3S": round(3 * sbytes / t / 1e6, 1),
                                          "frac_of_hbm_3S": round(3 * sbytes / t / 1e6 / PEAK_HBM_GBS, 3),
                                          "inputs": "3 copies in rotation"}
        del gx

    if not args.no_kernels and "bf16" in extras:
        # the headline conv with bf16 operands (CONV3D_F_BF16)
        d1b = workloads.conv_inputs(s1, 1001, dtype="bf16")
        pb = c3d.conv3d_plan(desc_of(c3d, s1, c3d.CONV3D_F_BIAS | c3d.CONV3D_F_BF16))
        wsb = ws_for(pb, torch, dev)

        def bfT(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        xb, wb, bb = bfT(d1b["x"]), bfT(d1b["w"]), bfT(d1b["b"])
        yb = torch.empty(out_dims(s1), dtype=torch.bfloat16, device=dev)

        def conv_bf16():
            c3d.conv3d_forward(pb, xb, wb, bb, None, yb, wsb)
        _, p = time_steps(conv_bf16, 50, 20, torch)
        t = sum(p) / len(p)
        kern["causal_conv_512_T9_bf16"] = {"ms": round(t, 4), "TFLOP/s": round(pb.info().flops / t / 1e9, 1),
                                           "kernel": pb.info().kernel_name.decode()}
        del xb, wb, bb, yb, wsb, d1b

    if not args.no_kernels and "t1" in extras:
        s1f = workloads.CAUSAL_256_T1
        pt1 = c3d.conv3d_plan(desc_of(c3d, s1f, c3d.CONV3D_F_BIAS))
        ws1 = ws_for(pt1, torch, dev)
        x1 = bx[:, :1].contiguous()
        y1 = torch.empty(out_dims(s1f), dtype=torch.float16, device=dev)

        def t1():
            c3d.conv3d_forward(pt1, x1, bt["w1"], bt["b1"], None, y1, ws1)
        _, p = time_steps(t1, 20, 3, torch)
        t = sum(p) / len(p)
        kern["first_frame_fold_256"] = {"us": round(t * 1e3, 2),
                                        "TFLOP/s_folded": round(pt1.info().flops / t / 1e9, 1),
                                        "path": int(pt1.info().path)}
        del x1, y1, ws1

    if not args.no_kernels and "t1zero" in extras:
        # the zero-causal first frame: only the last temporal tap sees data
        s1z = dataclasses.replace(workloads.CAUSAL_256_T1, tmode=workloads.TPAD_ZERO)
        ptz = c3d.conv3d_plan(desc_of(c3d, s1z, c3d.CONV3D_F_BIAS))
        wsz = ws_for(ptz, torch, dev)
        xz = bx[:, :1].contiguous()
        yz = torch.empty(out_dims(s1z), dtype=torch.float16, device=dev)

        def t1z():
            c3d.conv3d_forward(ptz, xz, bt["w1"], bt["b1"], None, yz, wsz)
        _, p = time_steps(t1z, 20, 3, torch)
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
        _, p = time_steps(chunked, 10, 2, torch)
        t = sum(p) / len(p)
        kern["chunked_causal_conv_256_T17_as_5_4_4_4"] = {
            "ms": round(t, 4), "TFLOP/s": round(conv_flops / t / 1e9, 1),
            "ms_over_whole_conv": round(t / kern["causal_conv_256_T17"]["ms"], 3)
            if "causal_conv_256_T17" in kern else None}
        del cplans
    del a1, c1, a2, out, bx

    if not args.no_kernels and "gemm" in extras:
        # context only ("FLOPs parity"): the vendor GEMM (torch.matmul on
        # hipBLASLt) on a dense fp16 matrix of the headline's im2col shape,
        # M x K times K x N.  The conv never builds such a matrix.
        gm, gk, gn = info.gemm_m, info.gemm_k, info.gemm_n
        ga = torch.randn(gm, gk, device=dev, dtype=torch.float16)
        gb = torch.randn(gk, gn, device=dev, dtype=torch.float16)
        gc = torch.empty(gm, gn, device=dev, dtype=torch.float16)

        def gemm():
            torch.matmul(ga, gb, out=gc)
        _, p = time_steps(gemm, 30, 10, torch)
        t = sum(p) / len(p)
        kern["vendor_gemm_same_mnk"] = {"ms": round(t, 4), "TFLOP/s": round(2.0 * gm * gn * gk / t / 1e9, 1),
                                        "shape_m_k_n": [gm, gk, gn], "gemm_ms_over_conv_ms": round(t / kernel_ms, 3)}
        del ga, gb, gc

    if not args.no_kernels and "stage" in extras:
        log("channel-changing stage (2.2 GB input)")
        d3 = workloads.workload_inputs(3)
        s3, s3b = d3["shape"], d3["shape2"]
        p3 = c3d.conv3d_plan(desc_of(c3d, s3, c3d.CONV3D_F_BIAS))
        p3b = c3d.conv3d_plan(desc_of(c3d, s3b, c3d.CONV3D_F_BIAS))
        x3, w3, b3 = T(d3["x"]), T(d3["w"]), T(d3["b"])
        ws3 = ws_for(p3, torch, dev)
        del d3["x"]
        y3 = torch.empty(out_dims(s3), dtype=torch.float16, device=dev)
        w3b, b3b = T(d3["w2"]), T(d3["b2"])
        y3b = torch.empty(out_dims(s3b), dtype=torch.float16, device=dev)

        def st1():
            c3d.conv3d_forward(p3, x3, w3, b3, None, y3, ws3)
        _, p = time_steps(st1, 3, 1, torch)
        t = sum(p) / len(p)
        kern["causal_conv_512to256_T33_256x256"] = {"ms": round(t, 3),
                                                    "TFLOP/s": round(p3.info().flops / t / 1e9, 1),
                                                    "kernel": p3.info().kernel_name.decode()}

        def st2():
            c3d.conv3d_forward(p3b, y3, w3b, b3b, None, y3b)
        _, p = time_steps(st2, 10, 2, torch)
        t = sum(p) / len(p)
        pw_bytes = y3.numel() * 2 + y3b.numel() * 2 + w3b.numel() * 2
        kern["pointwise_256to128_T33_256x256"] = {"ms": round(t, 4),
                                                  "GB/s": round(pw_bytes / t / 1e6, 1),
                                                  "frac_of_hbm": round(pw_bytes / t / 1e6 / PEAK_HBM_GBS, 3),
                                                  "kernel": p3b.info().kernel_name.decode()}
        del x3, y3, y3b
    if not args.no_kernels:
        result["kernels"] = kern

    if args.cpu_seconds > 0:
        log("cpu baseline: oracle on a bounded sample")
        step()
        torch.cuda.synchronize()
        result["cpu_baseline"] = cpu_baseline_leg(d1, y.cpu().numpy(), info, args.cpu_seconds, np)
    else:
        result["cpu_baseline"] = None

    if not args.no_calibration:
        log("machine ceilings: MFMA on random operands, HBM read and copy")
        scratch = torch.empty(c3d.conv3d_calibrate_scratch_bytes(), dtype=torch.uint8, device=dev)
        mfma_tf, sclk = c3d.conv3d_calibrate_mfma(scratch)
        del scratch
        nb = 2 << 30
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        src.fill_(1)
        dst = torch.empty_like(src)
        rd, cp = c3d.conv3d_calibrate_hbm(src, dst, nb)
        del src, dst
        result["calibration"] = {"mfma_fp16_tflops_random_operands": round(mfma_tf, 1),
                                 "sclk_mhz_during_mfma": round(sclk, 0),
                                 "hbm_read_gbs": round(rd, 1), "hbm_copy_gbs_read_plus_write": round(cp, 1)}
        rf = result["roofline"]
        rf["frac_of_measured"] = round(rf["achieved"] / mfma_tf, 4)
        if "kernels" in result:
            k = result["kernels"]
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
