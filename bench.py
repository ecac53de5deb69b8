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

`--suite OUT.md` instead times every block linear (q/k/v/o 5120x5120,
gate/up 17408x5120, down 5120x17408; both packings; batch 1 and 8), one
decode token through 64 distinct base-3 layers (5.2 GB of weights; q/k/v and
gate/up concatenated, so four calls per layer) with the rotation's share of
the separate route, and plain torch streams, and writes a markdown summary.
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
    ap.add_argument("--no-token", action="store_true", help="skip the 64-layer decode token leg")
    ap.add_argument("--no-stream", action="store_true", help="skip the read-ceiling leg")
    ap.add_argument("--no-smi", action="store_true",
                    help="do not start rocm-smi for the shader clock (for runs under a counter profiler, whose "
                         "preloaded library would make the child's interpreter start an exec after GPU init)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (for calibrating HBM byte counters) and exit")
    ap.add_argument("--gemv-batch", type=int, metavar="B",
                    help="instead of the one-line record: time tb_gemv alone on the FFN gate/up linear "
                         "(base-3 17408x5120) at batch B, cache-cold, and print one JSON line")
    ap.add_argument("--suite", metavar="OUT_MD",
                    help="instead of the one-line record: time the block linears (both packings, batch 1 and 8), "
                         "the 64-layer decode token stream and a 2 GiB read, and write a markdown summary")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(HERE, "profiles", "tb_linear_base3_17408x5120_b1_traffic.md")


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


def bench_decode(d, steps, warmup, smi=True):
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
    # the shader clock while the product runs: about 3 s of replays queued, rocm-smi read meanwhile
    sclk = "not read (--no-smi)"
    if smi:
        for _ in range(max(1, int(3.0 / max(t_fused * steps, 1e-6)))):
            g_fused.replay()
        sclk = shader_clock()
        torch.cuda.synchronize()
    return wall, t_fused, t_gemv, t_rot, sclk


def bench_single_1024(steps):
    """The single 1024x1024 2-bit linear at batch 1 (fp32 x, no outliers): us per call of
    tb_linear (rotation fused), tb_fwht_rotate and tb_gemv, from graphs of back-to-back calls.  Its
    0.28 MB of weights stay in cache, so these are latencies, not HBM rates."""
    n = k = 1024
    li = synth.linear_inputs(0, n, k, 1, "f32", False)
    packed = tb.tb_pack_2bit(dev(li.trits))
    scales = dev(li.scales.view(np.float16))
    x = dev(li.x)
    signs = dev(li.signs.view(np.int32))
    xr = torch.empty((1, k), dtype=torch.float32, device="cuda")
    y = torch.empty((1, n), dtype=torch.float32, device="cuda")
    out = {}
    for name, fn in (("tb_linear_us", lambda: tb.tb_linear("2bit", packed, scales, x, signs, y=y)),
                     ("tb_fwht_rotate_us", lambda: tb.tb_fwht_rotate(x, signs, out=xr)),
                     ("tb_gemv_us", lambda: tb.tb_gemv("2bit", packed, scales, xr, y=y))):
        _, g = time_graph(lambda: [fn() for _ in range(steps)], lambda: [fn() for _ in range(3)])
        out[name] = round(event_time(g) / steps * 1e6, 3)
        del g
    return out


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


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads():
    """The host threads this process may use: its CPU affinity, capped by OMP_NUM_THREADS when set."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    env = os.environ.get("OMP_NUM_THREADS")
    return max(1, min(n, int(env))) if env and env.isdigit() else n


def rotate_k17408_us(steps=200):
    """tb_fwht_rotate of one bf16 row of K = 17408 (17 blocks) to fp32, us per call."""
    k = synth.FFN
    x = dev(synth.activations(synth.rng(1, synth.T_X, 0, 9), 1, k, dtype="bf16").view(np.int16)).view(torch.bfloat16)
    sg = dev(synth.sign_bits(synth.rng(1, synth.T_SIGNS, 0, 9), k).view(np.int32))
    xr = torch.empty((1, k), dtype=torch.float32, device="cuda")

    def rot():
        for _ in range(steps):
            tb.tb_fwht_rotate(x, sg, out=xr)

    _, g = time_graph(rot, rot)
    return event_time(g) / steps * 1e6


def cpu_baseline(d, budget_s=(8.0, 5.0)):
    """The plain C++ oracle (fp64 loops) on the same decode step, rotate + product over all
    17408 rows: single-threaded, then with its output rows split over every host thread."""
    import oracle
    from oracle import cpp_oracle
    li, k = d["li"], d["k"]
    packed, _ = oracle.pack_base3(li.trits)
    x64 = synth.bf16_bits_to_f64(li.x)
    per = packed.nbytes + li.scales.nbytes
    out = {}
    for threads, budget in zip((1, host_threads()), budget_s):
        t0 = time.perf_counter()
        runs = 0
        while runs < 1 or time.perf_counter() - t0 < budget:
            cpp_oracle.linear("base3", packed, li.scales, x64, li.signs, threads)
            runs += 1
        el = time.perf_counter() - t0
        out[threads] = (runs * per / el / 1e9, runs, el)
    cores = host_threads()
    v1, r1, e1 = out[1]
    vn, rn, en = out[cores]
    # the same oracle as a prefill product on a sample of pp512's rows (x' already rotated),
    # all threads: multiply-adds per second (2 flops each)
    rows = 16
    xs = synth.bf16_bits_to_f64(synth.activations(synth.rng(3, synth.T_X), rows, k, dtype="bf16"))
    t0 = time.perf_counter()
    cpp_oracle.linear("base3", packed, li.scales, xs, None, cores)
    eg = time.perf_counter() - t0
    gflops = 2.0 * rows * packed.shape[0] * k / eg / 1e9
    return {"value": round(vn, 5), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "single_thread_value": round(v1, 5), "cpu_model": cpu_model(),
            "gemm_sample_gflops": round(gflops, 3),
            "sample": f"plain C++ fp64 oracle, rotate + product of the full 17408x5120 base-3 step at batch 1: "
                      f"{rn} passes in {en:.1f} s on {cores} threads, {r1} passes in {e1:.1f} s on one; "
                      f"gemm_sample_gflops: {rows} rows of the pp512 product (17408x5120 base-3) on {cores} "
                      f"threads, {eg:.1f} s"}


def stream_ceiling(per_copy, reps=20):
    """The library's read-only stream kernel (tb_stream_read): at the decode step's size, cycling
    through > 512 MB of buffers like the weights, and once over 2 GB; GB/s from HIP events."""
    sink = torch.zeros(tb.TB_STREAM_SINK_WORDS, dtype=torch.int32, device="cuda")
    size = -(-per_copy // 16) * 16
    copies = max(2, -(-CACHE_BYTES // size))
    bufs = [torch.ones(size, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    steps = 4 * copies

    def small():
        for i in range(steps):
            tb.tb_stream_read(bufs[i % copies], sink, per_copy // 16 * 16)

    _, g = time_graph(small, small)
    t_small = event_time(g, 3) / steps
    del g, bufs
    big_bytes = 2_000_000_000
    big = torch.ones(big_bytes, dtype=torch.uint8, device="cuda")

    def large():
        for _ in range(reps // 4):
            tb.tb_stream_read(big, sink)

    _, g = time_graph(large, large)
    t_big = event_time(g, 2) / (reps // 4)
    del g, big
    return {"kernel": "tb_stream_read (16-byte loads, 4 in flight per lane)",
            "gbs_at_step_size": round(per_copy // 16 * 16 / t_small / 1e9, 1), "step_size_bytes": per_copy // 16 * 16,
            "us_at_step_size": round(t_small * 1e6, 3),
            "gbs_at_2GB": round(big_bytes / t_big / 1e9, 1)}


# ---------------------------------------------------------------- --suite
#
# Weights for the suite are drawn on the GPU (torch's Philox generator, seeded
# per tensor) with the same distributions as the seeded host generators: trits
# P(0) = 0.5, P(+1) = P(-1) = 0.25; scales |N(0, 0.02)| + 1e-3 in fp16; bf16
# N(0, 1) activations.  Timing does not depend on the values, and 24 G host
# trits would take far too long to draw.

SUITE_SEED = 0x7B500002


def gpu_trits(n, k, gen):
    r = torch.randint(0, 4, (n, k), dtype=torch.int8, device="cuda", generator=gen)
    return (r == 3).to(torch.int8) - (r == 0).to(torch.int8)


def gpu_scales(n, k, gen):
    return (torch.randn((n, k // 128), device="cuda", generator=gen) * 0.02).abs_().add_(1e-3).half()


def gpu_packed(packing, n, k, gen):
    t = gpu_trits(n, k, gen)
    p = (tb.tb_pack_2bit if packing == "2bit" else tb.tb_pack_base3)(t)
    del t
    return p, gpu_scales(n, k, gen)


def gpu_signs(k):
    return dev(synth.sign_bits(synth.rng(4, synth.T_SIGNS), k).view(np.int32))


def suite_linear(packing, n, k, b, gen, steps=50):
    """One linear at batch b: fused call, rotation alone, product alone; us per call."""
    p0, s0 = gpu_packed(packing, n, k, gen)
    per = p0.numel() + 2 * s0.numel()
    copies = max(2, -(-CACHE_BYTES // per))
    ps = [p0] + [p0.clone() for _ in range(copies - 1)]
    ss = [s0] + [s0.clone() for _ in range(copies - 1)]
    x = torch.randn((b, k), device="cuda", generator=gen).to(torch.bfloat16)
    sg = gpu_signs(k)
    xr = torch.empty((b, k), dtype=torch.float32, device="cuda")
    y = torch.empty((b, n), dtype=torch.float32, device="cuda")

    def fused():
        for i in range(steps):
            tb.tb_linear(packing, ps[i % copies], ss[i % copies], x, sg, y=y)

    def rot():
        for _ in range(steps):
            tb.tb_fwht_rotate(x, sg, out=xr)

    def gemv():
        for i in range(steps):
            tb.tb_gemv(packing, ps[i % copies], ss[i % copies], xr, y=y)

    need = tb.tb_linear_workspace_bytes(packing, b, n, k)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")

    def fused_ws():
        for i in range(steps):
            tb.tb_linear_ws(packing, ps[i % copies], ss[i % copies], x, sg, workspace=ws, y=y)

    out = {}
    for name, fn in (("fused", fused), ("rotate", rot), ("gemv", gemv), ("ws", fused_ws)):
        _, g = time_graph(fn, fn)
        out[name] = event_time(g, 3) / steps * 1e6
        del g
    out["bytes"] = per
    del ps, ss
    return out


def suite_token(gen, layers=64, reps=10, per_call=True):
    """One decode token at batch 1 through 64 layers of base-3 linears, q/k/v and
    gate/up concatenated (4 calls per layer): whole-token graph time, fused and
    separate routes, and the rotation's share of the separate route."""
    H, F = synth.HIDDEN, synth.FFN
    shapes = (("qkv", 3 * H, H), ("o", H, H), ("gate_up", 2 * F, H), ("down", H, F))
    W = []
    total = 0
    for _ in range(layers):
        lw = []
        for _, n, k in shapes:
            p, s = gpu_packed("base3", n, k, gen)
            total += p.numel() + 2 * s.numel()
            x = torch.randn((1, k), device="cuda", generator=gen).to(torch.bfloat16)
            lw.append((p, s, x))
        W.append(lw)
    sg = {H: gpu_signs(H), F: gpu_signs(F)}
    xr = {H: torch.empty((1, H), dtype=torch.float32, device="cuda"),
          F: torch.empty((1, F), dtype=torch.float32, device="cuda")}
    ys = [torch.empty((1, n), dtype=torch.float32, device="cuda") for _, n, _ in shapes]
    # one workspace for every call (down's rows of K = 17408 take it for their partial sums)
    ws = torch.empty(max(16, max(tb.tb_linear_workspace_bytes("base3", 1, n, k) for _, n, k in shapes)),
                     dtype=torch.uint8, device="cuda")

    def lin(p, s, x, signs, y):
        tb.tb_linear_ws("base3", p, s, x, signs, workspace=ws, y=y)

    def fused(only=None):
        for lw in W:
            for j, ((_, n, k), (p, s, x)) in enumerate(zip(shapes, lw)):
                if only is None or only == j:
                    lin(p, s, x, sg[k], ys[j])

    def separate(rot=True, prod=True):
        for lw in W:
            for j, ((_, n, k), (p, s, x)) in enumerate(zip(shapes, lw)):
                if rot:
                    tb.tb_fwht_rotate(x, sg[k], out=xr[k])
                if prod:
                    tb.tb_gemv("base3", p, s, xr[k], y=ys[j])

    # The same layers with true dependencies: each call's input is the previous call's output (the
    # first K values of it), per call (dependent) or with q/k/v -> o -> gate/up in one
    # tb_decode_chain launch and down after it (chained: two launches per layer).
    F3, H3 = 2 * F, 3 * H
    yq = torch.empty((1, H3), dtype=torch.float32, device="cuda")
    yo = torch.empty((1, H), dtype=torch.float32, device="cuda")
    yg = torch.empty((1, F3), dtype=torch.float32, device="cuda")
    yd = torch.empty((1, H), dtype=torch.float32, device="cuda")
    x_first = W[0][0][2]
    sync = torch.zeros(tb.TB_CHAIN_MAX + 2, dtype=torch.int32, device="cuda")

    def dependent():
        x = x_first
        for (pq, sq, _), (po, so, _), (pg, sgg, _), (pd, sd, _) in W:
            lin(pq, sq, x, sg[H], yq)
            lin(po, so, yq[:, :H], sg[H], yo)
            lin(pg, sgg, yo, sg[H], yg)
            lin(pd, sd, yg[:, :F], sg[F], yd)
            x = yd

    def chained():
        x = x_first
        for (pq, sq, _), (po, so, _), (pg, sgg, _), (pd, sd, _) in W:
            tb.tb_decode_chain("base3", [(pq, sq), (po, so), (pg, sgg)], x, sg[H], sync, ys=[yq[0], yo[0], yg[0]])
            lin(pd, sd, yg[:, :F], sg[F], yd)
            x = yd

    res = {"bytes": total, "layers": layers, "calls_fused": 4 * layers,
           "launches_fused": 5 * layers}  # down: the parts' launch and the sum of their partial sums
    for name, fn in (("fused", fused), ("separate", separate),
                     ("rotate_only", lambda: separate(True, False)), ("gemv_only", lambda: separate(False, True)),
                     ("dependent", dependent), ("chained", chained)):
        _, g = time_graph(fn, fn)
        res[name] = event_time(g, reps)
        del g
    for j, (nm, n, k) in enumerate(shapes if per_call else ()):
        _, g = time_graph(lambda j=j: fused(j), lambda j=j: fused(j))
        res["call_" + nm] = (n, k, event_time(g, reps) / layers)
        del g
    del W
    return res


def suite_read_calibration(reps=10):
    """Plain HBM streams through torch's own kernels: a 2 GiB read (sum over
    fp32) and a 1 GiB copy (2 GiB moved).  A lower bound on what the box
    streams; neither kernel is tuned for this."""
    buf = torch.ones(512 << 20, dtype=torch.float32, device="cuda")
    out = torch.empty((), dtype=torch.float32, device="cuda")
    half = buf[: 256 << 20]
    dst = torch.empty_like(half)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        s = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(reps):
            fn()
        e1.record(s)
        e1.synchronize()
        return e0.elapsed_time(e1) / 1e3 / reps

    t_read = timed(lambda: out.copy_(buf.sum()))
    t_copy = timed(lambda: dst.copy_(half))
    del buf, dst
    return {"read_us": t_read * 1e6, "gbs": (2 << 30) / t_read / 1e9,
            "copy_us": t_copy * 1e6, "copy_gbs": (2 << 30) / t_copy / 1e9}


def shader_clock():
    """The current sclk line of rocm-smi (the clock while this is called), or a note that it
    was not available."""
    import subprocess
    try:
        out = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=30).stdout
        lines = [l.strip() for l in out.splitlines() if "sclk" in l.lower()]
        return lines[0] if lines else "not reported"
    except Exception as e:  # noqa: BLE001
        return f"not available ({type(e).__name__})"


def run_suite(path, argv):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(SUITE_SEED)
    lines = []
    cal = suite_read_calibration()
    print(f"read calibration: {cal['gbs']:.0f} GB/s read, {cal['copy_gbs']:.0f} GB/s copy", flush=True)
    rows = []
    for packing in ("2bit", "base3"):
        for b in (1, 8):
            for lin in synth.BLOCK_LINEARS:
                r = suite_linear(packing, lin.n, lin.k, b, gen)
                rows.append((lin, packing, b, r))
                print(f"{lin.name} {lin.n}x{lin.k} {packing} b{b}: fused {r['fused']:.2f} us, "
                      f"rotate {r['rotate']:.2f} + gemv {r['gemv']:.2f} us", flush=True)
    # other batches on the FFN linear (above 8: tb_gemv in one pass, tb_linear
    # in chunks of 8 rows)
    big = []
    gate = synth.BLOCK_LINEARS[4]
    for packing in ("2bit", "base3"):
        for b in (2, 4, 8, 9, 16, 32):
            r = suite_linear(packing, gate.n, gate.k, b, gen, steps=20)
            big.append((packing, b, r))
            print(f"gate {packing} b{b}: fused {r['fused']:.2f} us, ws {r['ws']:.2f} us, gemv {r['gemv']:.2f} us",
                  flush=True)
    tok = suite_token(gen)
    print(f"token: fused {tok['fused'] * 1e3:.3f} ms, separate {tok['separate'] * 1e3:.3f} ms", flush=True)
    sclk = shader_clock() if "--no-smi" not in argv else "not read (--no-smi)"

    pk = HBM_PEAK_GBS
    lines.append("# Block linears and the 64-layer decode token stream (MI355X, one GPU)")
    lines.append("")
    lines.append("Command: `python bench.py " + " ".join(argv) + "`")
    lines.append("")
    lines.append("Graph-replayed calls on cache-cold weights (each linear cycles through > 512 MB of copies; "
                 "the token stream's 64 distinct layers hold "
                 f"{tok['bytes'] / 1e9:.2f} GB). Weights drawn on the GPU (seed {SUITE_SEED:#x}); "
                 "bf16 N(0,1) activations. GB/s counts packed codes + fp16 scales; % is of 8 TB/s.")
    lines.append("")
    lines.append(f"Plain streams through torch's own kernels (a lower bound on the box's rate): 2 GiB read "
                 f"(sum over fp32) {cal['read_us']:.1f} us = {cal['gbs']:.0f} GB/s; 1 GiB copy (2 GiB moved) "
                 f"{cal['copy_us']:.1f} us = {cal['copy_gbs']:.0f} GB/s.")
    lines.append("")
    lines.append("## Block linears (q/k/v/o 5120x5120, gate/up 17408x5120, down 5120x17408)")
    lines.append("")
    lines.append("tb_linear_ws differs from tb_linear at batch 8 (x' rotated into the workspace, then tb_gemv's "
                 "product: one pass over the weights; at 5120 rows the batched product takes K in four parts and "
                 "adds their partial sums) and for base-3 down at batch 1 (four parts of K on separate "
                 "workgroups, then a sum of the partial sums).")
    lines.append("")
    lines.append("| linear | N x K | packing | batch | MB | tb_linear us | GB/s | % peak | tb_linear_ws us | GB/s (ws) | "
                 "rotate us | tb_gemv us |")
    lines.append("|---|---|---|---|---|---|---|---|---|---|---|---|")
    for lin, packing, b, r in rows:
        gbs = r["bytes"] / (r["fused"] * 1e-6) / 1e9
        gws = r["bytes"] / (r["ws"] * 1e-6) / 1e9
        lines.append(f"| {lin.name} | {lin.n}x{lin.k} | {packing} | {b} | {r['bytes'] / 1e6:.2f} | {r['fused']:.2f} | "
                     f"{gbs:.0f} | {100 * gbs / pk:.1f} | {r['ws']:.2f} | {gws:.0f} | {r['rotate']:.2f} | "
                     f"{r['gemv']:.2f} |")
    lines.append("")
    lines.append("## Other batch sizes on gate (17408x5120)")
    lines.append("")
    lines.append("From the measured crossover on (here batch 9 for 2-bit, 8 for base-3), tb_gemv streams the "
                 "weights once (fp16 matrix cores, gemv_wide.hip). tb_linear_ws rotates into the caller's "
                 "workspace and runs tb_gemv's product from batch 6 (2-bit) or 5 (base-3) on at K = 5120, where "
                 "that beats the fused kernel's prologue; tb_linear (no workspace) runs the fused kernel up to 8 "
                 "rows and chunks of 8 rows above, each streaming the weights again.")
    lines.append("")
    lines.append("| packing | batch | tb_linear us | tb_linear_ws us | tb_gemv us | weight GB/s (tb_linear_ws) | "
                 "weight GB/s (tb_gemv) |")
    lines.append("|---|---|---|---|---|---|---|")
    for packing, b, r in big:
        lines.append(f"| {packing} | {b} | {r['fused']:.2f} | {r['ws']:.2f} | {r['gemv']:.2f} | "
                     f"{r['bytes'] / (r['ws'] * 1e-6) / 1e9:.0f} | {r['bytes'] / (r['gemv'] * 1e-6) / 1e9:.0f} |")
    lines.append("")
    lines.append("## Decode token stream: 64 layers, base-3, batch 1 (q/k/v and gate/up concatenated)")
    lines.append("")
    t_f, t_s, t_r, t_g = tok["fused"], tok["separate"], tok["rotate_only"], tok["gemv_only"]
    lines.append(f"- Weight bytes per token: {tok['bytes']:,} ({tok['calls_fused']} product calls, "
                 f"{tok['launches_fused']} launches).")
    lines.append(f"- Fused route (tb_linear_ws, rotation in the prologue; down in four parts of K): "
                 f"{t_f * 1e3:.3f} ms per token = "
                 f"**{1 / t_f:.1f} tokens/s-equivalent**, {tok['bytes'] / t_f / 1e9:.0f} GB/s "
                 f"({100 * tok['bytes'] / t_f / 1e9 / pk:.1f} % of 8 TB/s).")
    lines.append(f"- Separate route (tb_fwht_rotate to fp32, then tb_gemv): {t_s * 1e3:.3f} ms per token = "
                 f"{1 / t_s:.1f} tokens/s-equivalent.")
    lines.append(f"- Rotation alone (256 calls): {t_r * 1e3:.3f} ms; products alone: {t_g * 1e3:.3f} ms; "
                 f"FWHT share of the separate route = {100 * t_r / (t_r + t_g):.1f} %.")
    lines.append(f"- With true dependencies (each call's input = the previous call's output): "
                 f"{tok['dependent'] * 1e3:.3f} ms per token = {1 / tok['dependent']:.1f} tokens/s with 256 "
                 f"tb_linear_ws calls; {tok['chained'] * 1e3:.3f} ms = **{1 / tok['chained']:.1f} tokens/s** with "
                 f"q/k/v -> o -> gate/up in one tb_decode_chain launch per layer "
                 f"({3 * tok['layers']} launches with down's two).")
    lines.append("")
    lines.append("| call | N x K | us per call (fused) | GB/s |")
    lines.append("|---|---|---|---|")
    for nm in ("qkv", "o", "gate_up", "down"):
        n, k, t = tok["call_" + nm]
        byts = n * (tb.tb_packed_row_bytes("base3", k) + 2 * (k // 128))
        lines.append(f"| {nm} | {n}x{k} | {t * 1e6:.2f} | {byts / t / 1e9:.0f} |")
    lines.append("")
    lines.append(f"Shader clock reported by rocm-smi after the run: {sclk}.")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps({"suite": path, "token_ms_fused": round(t_f * 1e3, 4),
                      "tokens_per_s_equiv": round(1 / t_f, 1), "read_calibration_gbs": round(cal["gbs"], 1)}),
          flush=True)


def bench_gemv_batch(b, steps):
    """tb_gemv alone at batch b on gate/up (base-3 17408x5120), weights cycled
    through > 512 MB of copies, fp32 x' ~ N(0,1); us per call from HIP events
    over a graph of `steps` calls."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(SUITE_SEED)
    gate = synth.BLOCK_LINEARS[4]
    n, k = gate.n, gate.k
    p0, s0 = gpu_packed("base3", n, k, gen)
    per = p0.numel() + 2 * s0.numel()
    copies = max(2, -(-CACHE_BYTES // per))
    ps = [p0] + [p0.clone() for _ in range(copies - 1)]
    ss = [s0] + [s0.clone() for _ in range(copies - 1)]
    xr = torch.randn((b, k), device="cuda", generator=gen)
    y = torch.empty((b, n), dtype=torch.float32, device="cuda")

    def gemv():
        for i in range(steps):
            tb.tb_gemv("base3", ps[i % copies], ss[i % copies], xr, y=y)

    _, g = time_graph(gemv, gemv)
    us = event_time(g, 3) / steps * 1e6
    return {"metric": "tb_gemv weight GB/s (codes + scales read once per call)", "value": round(per / us / 1e3, 2),
            "unit": "GB/s", "us_per_call": round(us, 3), "batch": b,
            "kernel": "gemv_wide_kernel (fp16 matrix cores)" if b > tb.TB_GEMV_KERNEL_BATCH else "gemv_mfma_kernel (fp8 limbs)",
            "config": {"workload": f"gemv_gate_{n}x{k}_base3_b{b}", "n": n, "k": k, "packing": "base3",
                       "bytes_per_call": per, "weight_copies": copies, "x_dtype": "f32"}}


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
    if args.suite:
        run_suite(args.suite, sys.argv[1:])
        return
    if args.gemv_batch:
        print(json.dumps(bench_gemv_batch(args.gemv_batch, args.steps)), flush=True)
        return
    d = decode_setup()
    wall, t_fused, t_gemv, t_rot, sclk = bench_decode(d, args.steps, args.warmup, not args.no_smi)
    ms_per_step = wall / args.steps * 1e3
    per_copy = d["per_copy"]
    value = per_copy / (wall / args.steps) / 1e9
    fused_gbs = per_copy / t_fused / 1e9
    traffic = gemv_traffic_bytes()
    gemm = None if args.no_gemm else bench_gemm(args.steps)
    gemm3 = None if args.no_gemm else bench_gemm(args.steps, "base3")
    stream = None if args.no_stream else stream_ceiling(per_copy)
    single = bench_single_1024(args.steps)
    token = None
    if not args.no_token:
        del d["packed"], d["scales"]
        gen = torch.Generator(device="cuda")
        gen.manual_seed(SUITE_SEED)
        token = suite_token(gen, reps=3, per_call=False)
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
        # batch-1 base-3 product: x' in four fp6 (e2m3) limbs with a power-of-two scale per
        # 128-group, trits as fp4 (e2m1) codes, fp32 accumulation; the rotation in fp32
        "dtype": "fp6x4-limb*fp4->f32",
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
                     "kernel_us": round(t_fused * 1e6, 3),
                     "frac_of_measured_ceiling": None if stream is None else
                     round(fused_gbs / stream["gbs_at_step_size"], 4)},
        "stream_ceiling": stream,
        "single_linear_1024x1024_2bit_b1": single,
        "sclk_during_decode": sclk,
        "separate_route_us": {"tb_fwht_rotate_b1_k5120": round(t_rot * 1e6, 3),
                              "tb_fwht_rotate_b1_k17408": round(rotate_k17408_us(), 3),
                              "tb_gemv_base3_17408x5120_b1": round(t_gemv * 1e6, 3)},
        "tokens_per_s_equiv_this_linear": round(1.0 / (wall / args.steps), 1),
        "cpu_baseline": cpu,
    }
    if gemm:
        rec["pp512_gemm"] = {"tflops": round(gemm["tflops"], 2), "us": round(gemm["us"], 2),
                             "frac_of_fp16_mfma_peak": round(gemm["frac"], 4), "peak_tflops": FP16_MFMA_PEAK_TFLOPS,
                             "rotate_us_512x5120_to_f16": round(gemm["rotate_us"], 2),
                             # bf16 in + fp16 out, 512 x 5120 x 2 B each
                             "rotate_gbs_512x5120": round(2 * 512 * 5120 * 2 / (gemm["rotate_us"] * 1e-6) / 1e9, 1),
                             "tokens_per_s_equiv": round(gemm["tokens_per_s"], 1)}
    if gemm3:
        rec["pp512_gemm_base3"] = {"tflops": round(gemm3["tflops"], 2), "us": round(gemm3["us"], 2),
                                   "frac_of_fp16_mfma_peak": round(gemm3["frac"], 4)}
    if token:
        t_f, t_r, t_g = token["fused"], token["rotate_only"], token["gemv_only"]
        rec["decode_token_64_layers"] = {
            "tokens_per_s_equiv": round(1.0 / t_f, 1), "ms_per_token": round(t_f * 1e3, 4),
            "dependent_tokens_per_s": round(1.0 / token["dependent"], 1),
            "chained_tokens_per_s": round(1.0 / token["chained"], 1),
            "chained_launches_per_token": 3 * token["layers"],
            "weight_bytes_per_token": token["bytes"], "gbs": round(token["bytes"] / t_f / 1e9, 1),
            "frac_of_hbm_peak": round(token["bytes"] / t_f / 1e9 / HBM_PEAK_GBS, 4),
            "calls_per_token": token["calls_fused"], "launches_per_token": token["launches_fused"],
            "separate_route_ms": round(token["separate"] * 1e3, 4),
            "fwht_share_of_separate_route": round(t_r / (t_r + t_g), 4),
            "workload": "64 layers x (qkv 15360x5120, o 5120x5120, gate_up 34816x5120, down 5120x17408), "
                        "base-3, batch 1, one HIP graph; tokens_per_s_equiv: tb_linear_ws per call on fixed inputs "
                        "(down's rows of K = 17408 in four parts of K, partial sums in the workspace); "
                        "dependent: each call's input is the previous output; chained: the same with "
                        "qkv -> o -> gate_up in one tb_decode_chain launch per layer"}
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
