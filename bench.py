"""Benchmark of the ternary rotated-basis linear on one MI355X.

Default workload (the decode product the headline metric is quoted on): one
17408 x 5120 base-3 ternary linear (g128 fp16 scales, 1.75 bits/weight) at
batch 1; the activation is a bf16 N(0,1) vector with 0.1% outlier channels
x20, rotated by 5 blocks of the 1024-point Walsh-Hadamard basis.  One step is
    y = W (R x)  in one call (tb_linear: the rotation runs in the product's
    prologue).
The separate route (tb_fwht_rotate to fp32, then tb_gemv) is timed too.
The packed weights are replicated into enough distinct copies (> 512 MB) that
consecutive steps never hit the 256 MB Infinity Cache; step i uses copy
i mod copies.  The K timed steps are captured in one HIP graph and replayed.

Also measured, in the same run: the pp512 prefill product (M=512, N=17408,
K=5120; rotate to fp16 then tb_gemm) in TFLOP/s for 2-bit codes and for
base-3 bytes, the rotation alone, and the oracle on the host cores as a
baseline.

Prints one JSON line (rank 0).  `value` is the decode step's packed-weight
stream rate in GB/s (codes + scales per step / step time).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

import fwht_rotation_sqrt_amd as tb  # noqa: E402
import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix, published
CACHE_BYTES = 512 << 20         # weight copies must exceed this (Infinity Cache is 256 MB)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gemm", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (for calibrating HBM byte counters) and exit")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(HERE, "profiles", "tb_gemv_base3_17408x5120_b1_traffic.md")


def gemv_traffic_bytes():
    """HBM bytes per GEMV launch from the committed counter runs, or None when the
    kernel source has changed since they were taken (or they are missing)."""
    import hashlib
    try:
        line = next(l for l in open(TRAFFIC_FILE) if l.startswith("machine-readable:"))
        rec = json.loads(line.split(":", 1)[1])
        src = open(os.path.join(HERE, rec["source"]), "rb").read()
    except (OSError, StopIteration, ValueError, KeyError):
        return None
    if hashlib.sha256(src).hexdigest() != rec["source_sha256"]:
        return None
    return rec["fetch_bytes"] + rec["write_bytes"]


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def time_graph(fn_steps, warmup_fn=None):
    """Capture fn_steps() into a graph, replay once untimed, then once timed; seconds."""
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        if warmup_fn:
            warmup_fn()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn_steps()
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    return time.perf_counter() - t0, g


def event_time(g, reps=1):
    """Average seconds of one replay of graph g, from HIP events on the replay stream."""
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(reps):
        g.replay()
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1) / 1e3 / reps


def decode_setup():
    n, k = synth.FFN, synth.HIDDEN
    li = synth.linear_inputs(1, n, k, 1, "bf16", True)
    trits = dev(li.trits)
    packed0 = tb.tb_pack_base3(trits)
    del trits
    scales0 = dev(li.scales.view(np.float16))
    per_copy = packed0.numel() + 2 * scales0.numel()
    copies = max(2, -(-CACHE_BYTES // per_copy))
    packed = [packed0] + [packed0.clone() for _ in range(copies - 1)]
    scales = [scales0] + [scales0.clone() for _ in range(copies - 1)]
    x = dev(li.x.view(np.int16)).view(torch.bfloat16)
    signs = dev(li.signs.view(np.int32))
    xr = torch.empty((1, k), dtype=torch.float32, device="cuda")
    y = torch.empty((1, n), dtype=torch.float32, device="cuda")
    return dict(n=n, k=k, li=li, packed=packed, scales=scales, x=x, signs=signs, xr=xr, y=y,
                per_copy=per_copy, copies=copies)


def bench_decode(d, steps, warmup):
    packed, scales, copies = d["packed"], d["scales"], d["copies"]

    def step(i):
        tb.tb_linear("base3", packed[i % copies], scales[i % copies], d["x"], d["signs"], y=d["y"])

    def warm():
        for i in range(warmup):
            step(i)

    wall, g_step = time_graph(lambda: [step(i) for i in range(steps)], warm)

    # per-kernel durations: each kernel alone, back to back, in its own graph
    # (the fused product is the only kernel of the step)
    def fused_only():
        for i in range(steps):
            tb.tb_linear("base3", packed[i % copies], scales[i % copies], d["x"], d["signs"], y=d["y"])

    def gemv_only():
        for i in range(steps):
            tb.tb_gemv("base3", packed[i % copies], scales[i % copies], d["xr"], y=d["y"])

    def rot_only():
        for i in range(steps):
            tb.tb_fwht_rotate(d["x"], d["signs"], out=d["xr"])

    _, g_fused = time_graph(fused_only)
    _, g_gemv = time_graph(gemv_only)
    _, g_rot = time_graph(rot_only)
    t_fused = event_time(g_fused) / steps
    t_gemv = event_time(g_gemv) / steps
    t_rot = event_time(g_rot) / steps
    return wall, t_fused, t_gemv, t_rot


def bench_gemm(steps, packing="2bit"):
    m, n, k = 512, synth.FFN, synth.HIDDEN
    li = synth.linear_inputs(3, n, k, m, "bf16", True)
    packed = (tb.tb_pack_2bit if packing == "2bit" else tb.tb_pack_base3)(dev(li.trits))
    scales = dev(li.scales.view(np.float16))
    x = dev(li.x.view(np.int16)).view(torch.bfloat16)
    signs = dev(li.signs.view(np.int32))
    xr = torch.empty((m, k), dtype=torch.float16, device="cuda")
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    reps = max(5, steps // 10)

    def gemm_only():
        for _ in range(reps):
            tb.tb_gemm(packing, packed, scales, xr, y=y)

    def rot_only():
        for _ in range(reps):
            tb.tb_fwht_rotate(x, signs, out=xr)

    tb.tb_fwht_rotate(x, signs, out=xr)
    _, g_gemm = time_graph(gemm_only, gemm_only)
    _, g_rot = time_graph(rot_only)
    t_gemm = event_time(g_gemm) / reps
    t_rot = event_time(g_rot) / reps
    flops = 2.0 * m * n * k
    return dict(m=m, n=n, k=k, us=t_gemm * 1e6, tflops=flops / t_gemm / 1e12,
                frac=flops / t_gemm / 1e12 / FP16_MFMA_PEAK_TFLOPS, rotate_us=t_rot * 1e6,
                tokens_per_s=m / (t_gemm + t_rot))


def cpu_baseline(d, budget_s=15.0):
    """The oracle (fp64 numpy) on the same decode workload: rotate + GEMV, whole rows."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        cores = 1
    li, n, k = d["li"], d["n"], d["k"]
    packed, _ = oracle.pack_base3(li.trits)
    x64 = synth.bf16_bits_to_f64(li.x)
    rows = n
    t0 = time.perf_counter()
    done_bytes = 0
    runs = 0
    while True:
        xr = oracle.rotate(x64, li.signs)
        oracle.gemv("base3", packed[:rows], li.scales[:rows], xr, k)
        done_bytes += packed[:rows].nbytes + li.scales[:rows].nbytes
        runs += 1
        if time.perf_counter() - t0 > budget_s or runs >= 8:
            break
    el = time.perf_counter() - t0
    return {"value": done_bytes / el / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{runs} full passes of rotate+GEMV (17408x5120 base-3, batch 1) in fp64 numpy, {el:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported on this build "
              "(the path would shard W by output rows across GPUs, see the design notes)", file=sys.stderr)
        sys.exit(2)
    torch.cuda.init()
    if args.copy_calibration:
        # a known amount of HBM traffic: 256 MiB read + 256 MiB written per copy
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": src.numel(), "copies": 5}), flush=True)
        return
    tb.library()
    d = decode_setup()
    wall, t_fused, t_gemv, t_rot = bench_decode(d, args.steps, args.warmup)
    ms_per_step = wall / args.steps * 1e3
    per_copy = d["per_copy"]
    value = per_copy / (wall / args.steps) / 1e9
    fused_gbs = per_copy / t_fused / 1e9
    traffic = gemv_traffic_bytes()
    gemm = None if args.no_gemm else bench_gemm(args.steps)
    gemm3 = None if args.no_gemm else bench_gemm(args.steps, "base3")
    cpu = None if args.no_cpu_baseline else cpu_baseline(d)
    rec = {
        "metric": "packed-ternary GEMV HBM GB/s (% peak) + pp512 GEMM TFLOP/s, K=5120",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "gemv_ffn_17408x5120_base3_b1", "n": d["n"], "k": d["k"], "batch": 1,
                   "packing": "base3", "bits_per_weight": 1.75, "bytes_per_step": per_copy,
                   "weight_copies": d["copies"], "step": "tb_linear (rotation of bf16 x fused into the product)",
                   "hip_graph": True, "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": round(fused_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(fused_gbs / HBM_PEAK_GBS, 4),
                     # counter-measured HBM bytes of one launch over the same launch time
                     "traffic": None if traffic is None else round(traffic / t_fused / 1e9, 2),
                     "traffic_bytes_per_launch": traffic,
                     "algorithmic_bytes_per_launch": per_copy,
                     "kernel": "tb_linear base-3 17408x5120 b1 (fused rotation)",
                     "kernel_us": round(t_fused * 1e6, 3)},
        "separate_route_us": {"tb_fwht_rotate_b1_k5120": round(t_rot * 1e6, 3),
                              "tb_gemv_base3_17408x5120_b1": round(t_gemv * 1e6, 3)},
        "tokens_per_s_equiv_this_linear": round(1.0 / (wall / args.steps), 1),
        "cpu_baseline": cpu,
    }
    if gemm:
        rec["pp512_gemm"] = {"tflops": round(gemm["tflops"], 2), "us": round(gemm["us"], 2),
                             "frac_of_fp16_mfma_peak": round(gemm["frac"], 4), "peak_tflops": FP16_MFMA_PEAK_TFLOPS,
                             "rotate_us_512x5120_to_f16": round(gemm["rotate_us"], 2),
                             "tokens_per_s_equiv": round(gemm["tokens_per_s"], 1)}
    if gemm3:
        rec["pp512_gemm_base3"] = {"tflops": round(gemm3["tflops"], 2), "us": round(gemm3["us"], 2),
                                   "frac_of_fp16_mfma_peak": round(gemm3["frac"], 4)}
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
