#!/usr/bin/env python3
"""Benchmark of C = epilogue(A . B) on one MI355X: prints one JSON line.

A step is one gemm_run of the workload over inputs already resident in HBM
(the planner's plan, split K allowed: a split plan's step is the GEMM and
its reduction).  Launched back to back, the first few hundred GEMMs see the
clock boost, dip and recover as power management reacts; the default 400
warm-up steps put the timed steps in the settled state a sustained caller
sees.
Default workload: bf16 M = N = K = 4096, A, B ~ N(0, 1), relu, bf16 out
(the headline GEMM).  W untimed warm-up steps, then K timed steps between
two device synchronisations; the average launch duration of the kernel is
measured with HIP events recorded on the stream the kernel is launched on.

roofline: the kernel is bound by the MFMA units; achieved = 2*M*N*K flops
per launch / average launch duration, against MI355X's published dense
fp16/bf16 MFMA peak (2516.6 TFLOP/s = 256 CUs x 2.4 GHz x 4096 flop/CU/clk).

Also reported: the shader clock measured over the timed region (a probe
kernel reads the shader-clock and constant-rate counters on every XCD just
before and just after it), and the median, minimum and maximum launch
duration from a separate pass with an event after every launch.

cpu_baseline: the CPU oracle (plain C, fp32, OpenMP) timed on this host's
cores on a bounded sample of the same workload: the first r rows of C
(r x N x K multiply-adds), r chosen so the oracle works about 12 s; then on
one thread (about 6 s); with the CPU model.  This leg is the only part of
the script that runs the oracle; it also checks 64 outputs of the last
timed step against it (timed_output_check).

--mfma-ceiling: the register-only MFMA loop instead of the GEMM (the MFMA
units' sustained rate on N(0, 1) bf16 or FP8 operands and the clock they run
at); --copy-issue-cost: MFMA loops with global->LDS copies in between;
--planner-sweep: the planner's plan, the autotuner's and torch.matmul on a
sweep of shapes; --k-sweep: the headline's tile with 2 to 64 trips, split
into a per-trip and a fixed cost per launch.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X dense MFMA peaks: fp16 / bf16 2516.6 TFLOP/s (256 CUs x 2.4 GHz x
# 4096 flop/CU/clk), FP8 5033.2 (8192 flop/CU/clk)
PEAK_MFMA_TFLOPS = {4: 2516.6, 5: 2516.6, 9: 5033.2}
PEAK_HBM_GBS = 8000.0
METRIC = "GEMM TFLOP/s and % of MI355X dense MFMA peak (bf16 4096^3)"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=400,
                    help="untimed launches first: back to back, the shader clock boosts, dips and "
                         "recovers under power management for about the first 300-400 launches of "
                         "~0.1 ms before it settles")
    ap.add_argument("--workload", default="bf16_4096_relu")
    ap.add_argument("--tile", type=int, default=0, help="force a tile configuration id")
    ap.add_argument("--flags", type=int, default=0, help="plan flags (1: one stage, 2: unstaged)")
    ap.add_argument("--no-split", action="store_true", help="do not let the planner split K")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--rotate", type=int, default=0,
                    help="input/output sets cycled between steps (>1 defeats reuse of the 256 MB "
                         "last-level cache); default 4 for HBM-bound workloads, 1 otherwise")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="before the GEMM, run a plain device copy of this many MiB three "
                         "times (a known-size reference for the HBM byte counters)")
    ap.add_argument("--vs-torch", action="store_true",
                    help="also time torch.matmul (the vendor BLAS) on the same resident inputs, "
                         "the same way, with the activation as a separate op; reported as context")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "hbm_traffic.json"),
                    help="HBM bytes per launch measured with rocprofv3 counters")
    ap.add_argument("--launch-samples", type=int, default=100,
                    help="after the timed region, this many more launches each followed by an "
                         "event, for the median and minimum launch duration")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="instead of the GEMM: the register-only MFMA loop (bf16 32x32x16, operands "
                         "drawn from N(0, 1)) on every CU, timed the same way (the throughput the "
                         "MFMA units sustain on this data with no memory traffic)")
    ap.add_argument("--ceiling-dtype", choices=["bf16", "bf16_16x16x32", "fp8"], default="bf16",
                    help="operand type of the --mfma-ceiling loop (fp8: v_mfma_f32_32x32x64_f8f6f4 "
                         "with E4M3 operands; bf16_16x16x32: the other bf16 shape, "
                         "v_mfma_f32_16x16x32_bf16)")
    ap.add_argument("--ceiling-iters", type=int, default=0,
                    help="rounds of 64 MFMAs per wave in one --mfma-ceiling launch")
    ap.add_argument("--copy-issue-cost", action="store_true",
                    help="instead of the GEMM: MFMA loops with global->LDS copies in between "
                         "(tcg_probe_copy_issue), cycles per MFMA per SIMD for each pattern")
    ap.add_argument("--k-sweep", action="store_true",
                    help="instead of the bench line: the headline's tile on 4096 x 4096 x K for "
                         "K = 128 .. 4096, with a line through time and shader cycles per trip")
    ap.add_argument("--sweep-dtype", choices=["bf16", "fp8"], default="bf16",
                    help="--k-sweep operands: bf16 on tile 1, or FP8 E4M3 on tile 8 (K = 256 .. 8192)")
    ap.add_argument("--planner-sweep", action="store_true",
                    help="instead of the bench line: for a sweep of bf16 relu shapes, time the "
                         "planner's choice, the autotuner's and torch.matmul (one JSON line each)")
    return ap.parse_args()


# Shapes of the planner sweep: square sizes, skinny and deep-K products.
SWEEP = [(512, 512, 512), (1024, 1024, 1024), (2048, 2048, 2048), (2304, 2304, 2304),
         (3000, 3000, 3000), (4096, 4096, 4096), (6144, 6144, 6144), (8192, 8192, 8192),
         (1024, 4096, 4096), (4096, 1024, 4096), (4096, 4096, 1024), (256, 4096, 4096),
         (4096, 256, 4096), (128, 8192, 8192), (512, 8192, 8192), (8192, 1024, 1024),
         (16384, 16384, 1024), (2048, 2048, 8192), (512, 512, 16384), (1024, 1024, 32768),
         (4608, 4608, 4608), (7168, 7168, 7168)]


def planner_sweep():
    """The planner's choice (splits allowed), the autotuner's and torch.matmul
    on each SWEEP shape: bf16 operands from N(0,1), relu, bf16 out; HIP
    events, 30 warm-up launches, best of three runs of 20."""
    import torch

    import tensor_core_gemm_amd as tcg

    def timed(fn):
        for _ in range(30):
            fn()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(20):
                fn()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) / 20 * 1e3)
        return best

    g = torch.Generator(device="cuda").manual_seed(0)
    for M, N, K in SWEEP:
        A = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
        B = torch.randn(K, N, device="cuda", generator=g).to(torch.bfloat16)
        C = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
        tflop = 2.0 * M * N * K / 1e12
        row = {"shape": [M, N, K]}
        desc = tcg.make_desc(M, N, K, tcg.BF16, tcg.BF16, tcg.EPI_RELU, tcg.FLAG_SPLIT_K)
        ws = torch.empty(min(16 * M * N * 4, 1 << 30), dtype=torch.uint8, device="cuda")
        for name, p in (("planner", tcg.gemm_plan(desc)),
                        ("autotune", tcg.gemm_autotune(desc, A, B, C, workspace=ws))):
            i = p.info()
            w = ws if i.workspace_bytes else None
            us = timed(lambda: tcg.gemm_run_ex(p, A, B, C, workspace=w))
            row[name] = {"us": round(us, 2), "tflops": round(tflop / us * 1e6, 1),
                         "tile": i.tile_id, "split": i.split_k}
            if i.tail_rows:
                row[name]["tail"] = [i.tail_rows, i.tail_split]
        us = timed(lambda: torch.matmul(A, B, out=C))
        row["torch_matmul"] = {"us": round(us, 2), "tflops": round(tflop / us * 1e6, 1)}
        print(json.dumps(row), flush=True)
        del A, B, C, ws
        torch.cuda.empty_cache()


# Trips of the K sweep: the headline's 4096 x 4096 output on its own tile,
# with 2 to 64 trips (of 64 for bf16, of 128 for FP8).
KSWEEP_TRIPS = [2, 4, 8, 16, 32, 48, 64]


def k_sweep(args):
    """The headline's plan (tile 1: 256 x 256 x 64, two slots) on 4096 x 4096
    x K for K = 64 x KSWEEP_TRIPS: bf16 operands from N(0, 1), relu, bf16 out
    (with --sweep-dtype fp8: FP8 E4M3 operands on tile 8, 256 x 256 x 128,
    K = 128 x KSWEEP_TRIPS).
    Per K: launches back to back for about a second (the shader clock
    settles), then args.steps timed launches between two events on the
    launch stream, with the clock probe around them.  Least-squares lines
    through (trips, time per launch) and (trips, shader cycles per launch)
    split a launch into a cost per trip and a fixed cost (the prologue, the
    epilogue with its 32 MiB of stores, and the gap between launches)."""
    import numpy as np
    import torch

    import tensor_core_gemm_amd as tcg

    import gemm_workloads as gw

    M = N = 4096
    fp8 = args.sweep_dtype == "fp8"
    in_dtype, tile, bk = (gw.FP8, 8, 128) if fp8 else (gw.BF16, 1, 64)
    g = torch.Generator(device="cuda").manual_seed(3)
    stream = torch.cuda.current_stream()
    clock = make_clock_probe()
    rows = []
    for trips in KSWEEP_TRIPS:
        K = bk * trips
        A = gw.draw((M, K), gw.NORMAL, in_dtype, g)
        B = gw.draw((K, N), gw.NORMAL, in_dtype, g)
        C = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
        plan = tcg.gemm_plan(tcg.make_desc(M, N, K, in_dtype, tcg.BF16, tcg.EPI_RELU, 0, tile=tile))

        def step():
            tcg.gemm_run(plan, A, B, C, stream)

        step()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(20):
            step()
        torch.cuda.synchronize()
        per = (time.perf_counter() - t) / 20
        for _ in range(max(100, int(1.0 / per))):
            step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        clock.mark(0, stream)
        e0.record(stream)
        for _ in range(args.steps):
            step()
        e1.record(stream)
        clock.mark(1, stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / args.steps * 1e3
        mhz = clock.result()["mean_mhz"]
        rows.append({"K": K, "trips": trips, "us": round(us, 3), "clock_mhz": mhz,
                     "kcycles": round(us * mhz / 1e3, 2), "tflops": round(2.0 * M * N * K / us / 1e6, 1)})
        print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
        del A, B, C
    trips = np.array([r["trips"] for r in rows], dtype=np.float64)
    slope_us, fixed_us = np.polyfit(trips, np.array([r["us"] for r in rows]), 1)
    slope_kc, fixed_kc = np.polyfit(trips, np.array([r["kcycles"] for r in rows]), 1)
    print(json.dumps({
        "metric": f"time and shader cycles per launch against trips ({args.sweep_dtype} 4096 x 4096 x K, "
                  f"relu, tile {tile})",
        "steps": args.steps, "points": rows,
        "fit_us": {"per_trip": round(float(slope_us), 4), "fixed": round(float(fixed_us), 3)},
        "fit_kcycles": {"per_trip": round(float(slope_kc), 4), "fixed": round(float(fixed_kc), 3)},
        "mfma_kcycles_per_trip": 2.048,
    }), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(the GEMM would shard along M or N with no exchange step).", file=sys.stderr)
        sys.exit(2)

    import torch

    import gemm_workloads as gw
    import tensor_core_gemm_amd as tcg

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(3)
    tcg.check_runtime()
    if args.planner_sweep:
        planner_sweep()
        return
    if args.k_sweep:
        k_sweep(args)
        return
    if args.mfma_ceiling:
        mfma_ceiling(args)
        return
    if args.copy_issue_cost:
        copy_issue_cost()
        return
    w = gw.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    caps = tcg.gemm_device_caps_query(0)

    if args.copy_mib > 0:
        n = args.copy_mib * 1024 * 1024 // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    A_cpu, B_cpu = gw.make_inputs(w)
    # An HBM-bound workload whose bytes fit the last-level cache would be
    # timed on cached inputs if one set were reused: cycle 4 sets (400 MB
    # for the Swin projection) unless told otherwise.
    ridge = PEAK_MFMA_TFLOPS[w.in_dtype] * 1e12 / (PEAK_HBM_GBS * 1e9)
    if args.rotate <= 0:
        args.rotate = 4 if w.flops / w.algorithmic_bytes < ridge else 1
    sets = []
    for r in range(args.rotate):
        A = A_cpu.to(dev) if r == 0 else A_cpu.to(dev).clone()
        B = B_cpu.to(dev) if r == 0 else B_cpu.to(dev).clone()
        C = torch.empty((w.M, w.N), dtype=gw.TORCH_DTYPE[w.out_dtype], device=dev)
        sets.append((A, B, C))
    flags = args.flags | (0 if args.no_split else tcg.FLAG_SPLIT_K)
    desc = tcg.make_desc(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.epilogue, flags,
                         tile=args.tile)
    plan = tcg.gemm_plan(desc)
    info = plan.info()
    stream = torch.cuda.current_stream()
    ws = (torch.empty(info.workspace_bytes, dtype=torch.uint8, device=dev)
          if info.workspace_bytes else None)

    def step(i):
        A, B, C = sets[i % len(sets)]
        if ws is None:
            tcg.gemm_run(plan, A, B, C, stream)
        else:
            tcg.gemm_run_ex(plan, A, B, C, workspace=ws, stream=stream)

    # made before the warm-up: allocating it between the warm-up and the
    # timed region idled the GPU for milliseconds, which restarts the power
    # manager's boost-dip-settle cycle (measured: ~15 % slower timed launches)
    clock = make_clock_probe()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # One event pair around the K launches on the launch stream: the
    # average launch duration is the region's device time over K (events
    # between launches would add their own overhead to every launch).
    K = args.steps
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    clock.mark(0, stream)
    e_start.record(stream)
    for i in range(K):
        step(i)
    e_end.record(stream)
    clock.mark(1, stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    avg_launch_ms = e_start.elapsed_time(e_end) / K
    ms_per_step = (t1 - t0) * 1e3 / K
    clock_measured = clock.result()
    per_launch = per_launch_times(step, args.launch_samples, stream)

    flops = w.flops
    value = flops / (ms_per_step * 1e-3) / 1e12
    peak_mfma = PEAK_MFMA_TFLOPS[w.in_dtype]
    # The roofline that bounds the workload: MFMA where its arithmetic
    # intensity (flops per algorithmic byte) is above the ridge point
    # (peak flops / HBM bandwidth), HBM below it.
    hbm_bound = w.flops / w.algorithmic_bytes < peak_mfma * 1e12 / (PEAK_HBM_GBS * 1e9)
    if hbm_bound:
        achieved = w.algorithmic_bytes / (avg_launch_ms * 1e-3) / 1e9
        peak, bound, unit = PEAK_HBM_GBS, "hbm", "GB/s"
    else:
        achieved = flops / (avg_launch_ms * 1e-3) / 1e12
        peak, bound, unit = peak_mfma, "mfma", "TFLOP/s"

    # 64 outputs of the last timed step, checked against the oracle in the
    # CPU leg (the only part of this script that runs the oracle)
    _, ii, jj = gw.sample_indices(w.M, w.N, 64, 99)
    timed_sample = (ii, jj, sets[(K - 1) % len(sets)][2].float().cpu().numpy()[ii, jj])

    traffic = None
    try:
        with open(args.traffic) as f:
            t = json.load(f).get(w.name)
        if t and t.get("kernel_source_sha") == kernel_source_sha():
            traffic = t["hbm_bytes_per_launch"]
    except (OSError, ValueError):
        pass

    result = {
        # the headline's metric; another workload's line names that workload
        "metric": METRIC if w.name == "bf16_4096_relu" else f"GEMM TFLOP/s ({w.name})",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": gw.DTYPE_NAME[w.in_dtype],
        "data": "synthetic",
        "config": {
            "workload": w.name, "M": w.M, "N": w.N, "K": w.K,
            "in": gw.DTYPE_NAME[w.in_dtype], "out": gw.DTYPE_NAME[w.out_dtype],
            "epilogue": "relu" if w.epilogue else "none", "accumulate": "f32",
            "plan": plan.describe(), "pct_of_peak": round(100 * value / peak_mfma, 2),
            "device": caps.arch.decode(), "cus": caps.num_cus,
            "peak_clock_mhz": caps.clock_khz // 1000,
            "clock_mhz_measured": clock_measured,
            "input_sets": args.rotate,
        },
        "roofline": {
            "bound": bound,
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": unit,
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
            # context only: the same fraction against the peak at the shader clock measured over the
            # timed region (the MFMA peak scales with the clock; the chip ran below 2.4 GHz)
            "frac_at_measured_clock": (round(achieved / (peak * clock_measured["mean_mhz"] / (caps.clock_khz / 1000)), 4)
                                       if bound == "mfma" and clock_measured.get("mean_mhz") else None),
            "kernel_avg_ms": round(avg_launch_ms, 5),
            "launch_ms": per_launch,
            "flops_per_launch": flops,
            "algorithmic_bytes_per_launch": w.algorithmic_bytes,
        },
    }
    if args.vs_torch:
        result["torch_matmul"] = torch_matmul_time(w, sets[0], args.warmup, K, stream)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, A_cpu, B_cpu, args.cpu_seconds, timed_sample)
    print(json.dumps(result), flush=True)


def make_clock_probe():
    """The clock probe, its kernel launched once: the first launch of a
    kernel loads its code (about a millisecond of host time, measured), which
    inside the timed region would leave the GPU idle and count against every
    step."""
    import torch
    from tensor_core_gemm_amd.probe import ClockProbe
    clock = ClockProbe()
    clock.mark(0)
    torch.cuda.synchronize()
    return clock


def per_launch_times(step, n, stream):
    """n more launches, each followed by an event on the launch stream:
    the median, minimum and maximum of the per-launch durations (a pass of
    its own, after the timed region, so the events do not touch the
    region's average)."""
    import numpy as np
    import torch
    if n <= 0:
        return None
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(n):
        step(i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    d = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(n)])
    return {"n": n, "median": round(float(np.median(d)), 5), "min": round(float(d.min()), 5),
            "max": round(float(d.max()), 5), "mean": round(float(d.mean()), 5)}


def mfma_ceiling(args):
    """The register-only MFMA loop on every CU: the MFMA units' sustained
    rate on N(0, 1) bf16 operands with no memory traffic, LDS or barriers,
    and the shader clock it runs at."""
    import numpy as np
    import torch

    import gemm_workloads as gw
    import tensor_core_gemm_amd as tcg
    from tensor_core_gemm_amd import probe

    caps = tcg.gemm_device_caps_query(0)
    wg = caps.num_cus
    gen = torch.Generator().manual_seed(7)
    fp8 = args.ceiling_dtype == "fp8"
    if fp8:
        ops = gw.draw((16 * 64 * 32,), gw.NORMAL, gw.FP8, gen).view(torch.uint8).cuda()
        kind, iters = probe.MFMA_32x32x64_FP8, args.ceiling_iters or 35
        name = "v_mfma_f32_32x32x64_f8f6f4, E4M3"
    elif args.ceiling_dtype == "bf16_16x16x32":
        # half the flops per instruction: twice the rounds for the same work
        ops = gw.draw((16 * 64 * 8,), gw.NORMAL, gw.BF16, gen).view(torch.int16).cuda()
        kind, iters = probe.MFMA_16x16x32_BF16, args.ceiling_iters or 140
        name = "v_mfma_f32_16x16x32_bf16, bf16"
    else:
        ops = gw.draw((16 * 64 * 8,), gw.NORMAL, gw.BF16, gen).view(torch.int16).cuda()
        kind, iters = probe.MFMA_32x32x16_BF16, args.ceiling_iters or 70
        name = "v_mfma_f32_32x32x16_bf16, bf16"
    sink = torch.empty(wg * 256, dtype=torch.float32, device="cuda")
    ticks = torch.zeros(wg, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i=0):
        return probe.mfma_rate(kind, wg, iters, ops, sink, ticks, stream)

    flops = step()
    clock = make_clock_probe()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    clock.mark(0, stream)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    clock.mark(1, stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    per_launch = per_launch_times(step, args.launch_samples, stream)
    cyc = ticks.cpu().numpy().astype(np.float64)
    mfmas_per_wave = iters * 64
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_MFMA_TFLOPS[gw.FP8 if fp8 else gw.BF16]
    print(json.dumps({
        "metric": f"MFMA-only throughput, register operands ({name} operands from N(0,1))",
        "value": round(tflops, 2), "unit": "TFLOP/s", "frac_of_peak": round(tflops / peak, 4),
        "peak": peak, "steps": args.steps, "warmup": args.warmup, "kernel_avg_ms": round(ms, 5),
        "launch_ms": per_launch, "workgroups": wg, "waves_per_simd": 1,
        "mfma_per_wave": mfmas_per_wave,
        "cycles_per_mfma": round(float(np.median(cyc)) / mfmas_per_wave, 3),
        "clock_mhz_measured": clock.result(), "peak_clock_mhz": caps.clock_khz // 1000,
    }), flush=True)


def copy_issue_cost():
    """Cycles per MFMA per SIMD of a register-only MFMA loop with and without
    global->LDS copies between the MFMAs, with one and two waves per SIMD,
    and for the 32x32x16 and the 16x16x32 bf16 shapes (tcg_probe_copy_issue;
    median over the CUs).  Per pattern: 1000 warm-up launches, then 400
    timed ones with HIP events and the shader clock measured around them,
    so the rate under the power manager is reported beside the cycles."""
    import numpy as np
    import torch

    import gemm_workloads as gw
    import tensor_core_gemm_amd as tcg
    from tensor_core_gemm_amd import probe

    wg = tcg.gemm_device_caps_query(0).num_cus
    gen = torch.Generator().manual_seed(11)
    ops = gw.draw((8 * 64 * 8,), gw.NORMAL, gw.BF16, gen).view(torch.int16).cuda()
    src = torch.zeros(65536 // 4, dtype=torch.int32, device="cuda")
    sink = torch.empty(wg * 512, device="cuda")
    ticks = torch.zeros(wg, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()
    clock = make_clock_probe()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    iters, timed = 400, 400
    out = {}
    for pat, (name, waves, per_round) in probe.COPY_PATTERNS.items():
        mflops = probe.COPY_PATTERN_MFMA_FLOPS[pat]
        for _ in range(1000):
            per_simd = probe.copy_issue(pat, wg, iters, ops, src, sink, ticks, stream)
        torch.cuda.synchronize()
        clock.mark(0, stream)
        e0.record(stream)
        for _ in range(timed):
            probe.copy_issue(pat, wg, iters, ops, src, sink, ticks, stream)
        e1.record(stream)
        clock.mark(1, stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / timed
        cyc = float(np.median(ticks.cpu().numpy().astype(np.float64))) / per_simd
        flops = wg * waves * iters * per_round * mflops
        out[name] = {"cycles_per_mfma": round(cyc, 2),
                     "cycles_per_32768_flops": round(cyc * 32768 / mflops, 2),
                     "us_per_launch": round(ms * 1e3, 2),
                     "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                     "clock_mhz": clock.result()["mean_mhz"]}
    print(json.dumps({"metric": "cycles per MFMA per SIMD (bf16 MFMAs on register operands from N(0,1)), "
                                "with global->LDS copies between the MFMAs",
                      "flops_per_round_per_wave": 32 * 32768, "rounds": iters, "workgroups": wg,
                      "patterns": out}), flush=True)


def torch_matmul_time(w, io, warmup, steps, stream):
    """torch.matmul (the vendor BLAS on ROCm) on the same resident inputs,
    timed like the steps above; relu, where the workload has it, is a
    separate in-place op.  FP8 operands go through torch._scaled_mm with
    unit scales (it wants B column-major: a transposed copy made before
    timing)."""
    import torch
    import gemm_workloads as gw
    A, B, C = io
    A2, B2 = A.view(w.M, w.K), B.view(w.K, w.N)
    same_type = C.dtype == A.dtype
    if w.in_dtype == gw.FP8:
        Bcm = B2.t().contiguous().t()
        one = torch.ones((), dtype=torch.float32, device=A.device)
        try:
            torch._scaled_mm(A2, Bcm, scale_a=one, scale_b=one, out_dtype=C.dtype)
        except Exception as e:  # not every build has an FP8 GEMM for this device
            return {"error": f"{type(e).__name__}: {str(e)[:200]}"}

    def gemm():
        if w.in_dtype == gw.FP8:
            return torch._scaled_mm(A2, Bcm, scale_a=one, scale_b=one, out_dtype=C.dtype)
        if same_type:
            torch.matmul(A2, B2, out=C)
            return C
        return torch.matmul(A2, B2).to(C.dtype)

    def step():
        y = gemm()
        if w.epilogue:
            torch.relu_(y)

    clock = make_clock_probe()

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        clock.mark(0, stream)
        for _ in range(steps):
            fn()
        clock.mark(1, stream)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps, clock.result()["mean_mhz"]

    ms, mhz = timed(step)
    out = {"ms_per_step": round(ms, 5), "tflops": round(w.flops / (ms * 1e-3) / 1e12, 2),
           "with_relu": bool(w.epilogue), "clock_mhz_measured": mhz}
    if w.epilogue:
        # the product alone, without the separate relu
        ms_gemm, mhz_gemm = timed(gemm)
        out["gemm_only_ms"] = round(ms_gemm, 5)
        out["gemm_only_tflops"] = round(w.flops / (ms_gemm * 1e-3) / 1e12, 2)
        out["gemm_only_clock_mhz_measured"] = mhz_gemm
    return out


def kernel_source_sha() -> str:
    """Hash of the code (comments and layout removed) of the GEMM kernels'
    device sources (headers, kernel instantiations and the persistent
    short-K kernel; not the host planner, the probes or the reduction), so
    that counter data taken from other kernel code is not reported."""
    import hashlib
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tensor_core_gemm_amd", "csrc")
    for fn in sorted(os.listdir(csrc)):
        if fn.endswith(".h") or (fn.startswith("tcgemm_inst_") and fn.endswith(".hip")) or \
                fn == "tcgemm_shortk.hip":
            with open(os.path.join(csrc, fn)) as f:
                text = f.read()
            # code only: comments and layout do not change what runs
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
            text = re.sub(r"//[^\n]*", " ", text)
            text = " ".join(text.split())
            h.update(fn.encode() + text.encode())
    return h.hexdigest()[:16]


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_rate(w, A, B, target_s, n_threads):
    """The oracle on the first r rows of C, r scaled so the run takes about
    target_s seconds with n_threads threads (0: every thread OpenMP has)."""
    import oracle
    a = A.reshape(w.M, w.K)
    rows = 1
    t0 = time.perf_counter()
    oracle.gemm(a[:rows].contiguous(), B, rows, w.N, w.K, w.in_dtype, w.out_dtype, w.epilogue,
                n_threads=n_threads)
    dt = time.perf_counter() - t0
    if dt < 0.05:  # one row is too short to time: try 16
        rows = min(w.M, 16)
        t0 = time.perf_counter()
        oracle.gemm(a[:rows].contiguous(), B, rows, w.N, w.K, w.in_dtype, w.out_dtype, w.epilogue,
                    n_threads=n_threads)
        dt = time.perf_counter() - t0
    rows = int(max(1, min(w.M, rows * target_s / max(dt, 1e-6))))
    t0 = time.perf_counter()
    oracle.gemm(a[:rows].contiguous(), B, rows, w.N, w.K, w.in_dtype, w.out_dtype, w.epilogue,
                n_threads=n_threads)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * w.N * w.K
    return flops / dt, rows, flops, dt


def cpu_baseline(w, A, B, target_s, timed_sample=None):
    """The oracle as it is, on this host's cores (all OpenMP threads, then
    one), over the first r rows of C; and, given (rows, columns, values) of
    the last timed step's output, their largest relative error against the
    oracle (floor 0.01 of an output's standard deviation)."""
    import numpy as np

    import oracle
    threads = oracle.threads()
    rate, rows, flops, dt = oracle_rate(w, A, B, target_s, 0)
    rate1, rows1, flops1, dt1 = oracle_rate(w, A, B, target_s * 0.5, 1)
    check = None
    if timed_sample is not None:
        ii, jj, got = timed_sample
        _, y = oracle.gemm_sampled(A, B, w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.epilogue,
                                   np.zeros_like(ii), ii, jj)
        err = np.abs(got - y) / np.maximum(np.abs(y), 0.01 * w.sigma_out())
        check = {"outputs": int(ii.size), "max_rel_err": float(err.max())}
    return {
        "value": round(rate / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"first {rows} of {w.M} rows of C ({rows}x{w.N}x{w.K}, "
                  f"{flops / 1e9:.1f} GFLOP) in {dt:.2f} s on {threads} threads",
        "cpu_model": cpu_model(),
        "logical_cpus": os.cpu_count(),
        "single_core": {"value": round(rate1 / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
                        "sample": f"first {rows1} rows ({flops1 / 1e9:.1f} GFLOP) in {dt1:.2f} s"},
        "timed_output_check": check,
    }


if __name__ == "__main__":
    main()
