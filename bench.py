"""Benchmark: one fused GEMM + reduce-scatter pass per step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama70b]

A step is the whole hot path over one batch: the GEMM + epilogue kernel
(scatter into staging slots, flag publish) and the flag-gated reduce, on
W = 8 virtual ranks at the 70B-like FFN down-projection shard
(A_r[8192,3584] x B_r[3584,8192], bias row, bf16).  Inputs are resident in
HBM before timing starts.  Prints one JSON line.

value = algorithmic FLOPs of the step (W * 2*M*N*K) / wall time per step.
roofline: the GEMM kernel against the bf16 dense MFMA peak, with its
duration from HIP events around each launch inside the timed region.
cpu_baseline: the CPU oracle (fp64, all host threads) on a bounded sample
of the same workload's output rows.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 flop/clk x 2.4 GHz, dense
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBPS = 8000.0
METRIC = ("fused GEMM+RS TFLOP/s & MFMA util % at M=8192 N=8192 K=3584 W=8; "
          "reduce GB/s")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_llama70b.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_digest() -> str:
    """Hash of the GEMM kernel's sources: a stored traffic figure is valid
    only for the code it was measured on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tensor_gemm_reduce_lds_amd", "csrc")
    for f in ("gemm_bf16.hip", "gemm_rs_internal.h"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic():
    """HBM bytes per GEMM launch from the committed rocprofv3 counter
    summary, or None if absent or taken on other kernel code."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_source_digest") != kernel_source_digest():
            return None
        return float(kv["fetch_bytes_per_launch"]) + float(kv["write_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def algorithmic_bytes(w, elem):
    """GEMM kernel: A + B read once, fp32 staging written once, C read once
    (one row when broadcast).  Reduce: staging read once, out written once."""
    gemm = w.W * w.M * w.K * elem + w.W * w.K * w.N * elem + w.W * w.M * w.N * 4
    if w.has_c:
        gemm += (w.N if w.ldc == 0 else w.M * w.N) * elem
    red = w.W * w.M * w.N * 4 + w.M * w.N * elem
    return gemm, red


def gemm_roofline(flops, gemm_bytes, gemm_ms, peak_tflops, traffic):
    """The GEMM kernel's roofline object: MFMA-bound above the ridge point
    (peak flop/s over peak bytes/s), HBM-bound below it (the m <= 64 decode
    shard), with the achieved rate from algorithmic flops or bytes."""
    if flops / gemm_bytes >= peak_tflops * 1e12 / (PEAK_HBM_GBPS * 1e9):
        tflops = flops / (gemm_ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak_tflops,
                "unit": "TFLOP/s", "frac": round(tflops / peak_tflops, 4),
                "traffic": traffic}
    gbps = gemm_bytes / (gemm_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS,
            "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": traffic}


def cpu_baseline(w, x, budget_s: float):
    """Time the oracle (fp64 reference rows, every rank, OpenMP over rows)
    on the first rows of the workload for about budget_s seconds."""
    import oracle as O
    kw = dict(dtype=O.BF16 if w.dtype == "bf16" else O.F32, alpha=w.alpha,
              beta=w.beta, ldc=w.ldc,
              order=O.TWO_LEVEL if w.order == "two_level" else O.FLAT,
              groups=w.groups)
    threads = O.num_threads()
    rows, t = threads, 0.0
    t0 = time.perf_counter()
    O.reference_rows(x["A"], x["B"], x["C"], row_lo=0, row_hi=rows, **kw)
    t = time.perf_counter() - t0
    if t < budget_s / 3:
        more = max(threads, int(rows * (budget_s - t) / max(t, 1e-3)) // threads * threads)
        more = min(more, w.M - rows)
        t1 = time.perf_counter()
        O.reference_rows(x["A"], x["B"], x["C"], row_lo=rows, row_hi=rows + more, **kw)
        t += time.perf_counter() - t1
        rows += more
    flops = rows * w.W * 2 * w.N * w.K
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    # single-thread oracle times on the two small configurations: the whole
    # fp32 tiny case, and the first rows of the m <= 64 decode shard
    from tensor_gemm_reduce_lds_amd import inputs as I
    single = {}
    O.set_threads(1)
    try:
        for name, n_rows in (("tiny_f32", None), ("decode", 8)):
            ws = I.WORKLOADS[name]
            xs = I.make_inputs(ws)
            kws = dict(dtype=O.BF16 if ws.dtype == "bf16" else O.F32, alpha=ws.alpha,
                       beta=ws.beta, ldc=ws.ldc)
            hi = ws.M if n_rows is None else n_rows
            t1 = time.perf_counter()
            O.reference_rows(xs["A"], xs["B"], xs["C"], row_lo=0, row_hi=hi, **kws)
            ts = time.perf_counter() - t1
            fl = hi * ws.W * 2 * ws.N * ws.K
            single[name] = {"rows": hi, "of_rows": ws.M, "seconds": round(ts, 4),
                            "gflops": round(fl / ts / 1e9, 3)}
    finally:
        O.set_threads(threads)
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": threads,
            "single_thread": single,
            "kind": "oracle", "cpu_model": cpu_model, "os_cpu_count": os.cpu_count(),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "sample": "fp64 reference of output rows [0, %d) of %d (all %d ranks, "
                      "K=%d, N=%d): %.3g GFLOP in %.1f s" % (
                          rows, w.M, w.W, w.K, w.N, flops / 1e9, t)}


def ablation_measure(plan, A, B, C, out, w, stream, steps):
    """The pages' ablation modes and reference points, reported beside the
    headline (none is a target).  kernel-sync: every step followed by a
    stream synchronisation.  clear-kernel: the staging buffer cleared before
    every step, the memset a design that accumulates in place would need
    (this one stores per-source slots and never clears).  clear-only: the
    memset and a synchronisation alone.  clear-kernel-sync: memset, sync,
    step, sync.  Cold reduce: the
    GEMM alone, then a 512 MiB write that flushes the memory-side cache,
    then the reduce alone.  Context: torch.bmm (hipBLASLt) on the same W
    GEMMs with a bfloat16 output and no scatter; the library never calls it."""
    import ctypes
    import statistics
    import torch
    from tensor_gemm_reduce_lds_amd import gemm_rs as G
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemsetAsync.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t,
                                   ctypes.c_void_p]
    hip.hipMemsetAsync.restype = ctypes.c_int
    n = max(5, steps // 2)
    info = plan.info

    def run(flags=G.RUN_ALL):
        plan.run(A, B, C, w.alpha, w.beta, out, stream, flags)

    def check(what):
        rc, detail = plan.status(stream)
        if rc != G.OK:
            raise RuntimeError("%s failed: %s %s" % (what, G.gemm_rs_strerror(rc), detail))

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        run()
        stream.synchronize()
    sync_ms = (time.perf_counter() - t0) * 1e3 / n
    check("kernel-sync")

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        if hip.hipMemsetAsync(info.staging, 0, info.staging_bytes, stream.cuda_stream) != 0:
            raise RuntimeError("hipMemsetAsync failed")
        run()
    torch.cuda.synchronize()
    clear_ms = (time.perf_counter() - t0) * 1e3 / n
    check("clear-kernel")

    # clear-only (the memset and the synchronisation, no kernel) and
    # clear-kernel-sync (memset, sync, step, sync); the pages' host barrier
    # between ranks has no counterpart with one process
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        if hip.hipMemsetAsync(info.staging, 0, info.staging_bytes, stream.cuda_stream) != 0:
            raise RuntimeError("hipMemsetAsync failed")
        stream.synchronize()
    clear_only_ms = (time.perf_counter() - t0) * 1e3 / n
    t0 = time.perf_counter()
    for _ in range(n):
        if hip.hipMemsetAsync(info.staging, 0, info.staging_bytes, stream.cuda_stream) != 0:
            raise RuntimeError("hipMemsetAsync failed")
        stream.synchronize()
        run()
        stream.synchronize()
    clear_sync_ms = (time.perf_counter() - t0) * 1e3 / n
    check("clear-kernel-sync")

    flush = torch.empty((512 << 20) // 4, dtype=torch.float32, device=out.device)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cold = []
    for _ in range(n):
        run(G.RUN_GEMM)
        flush.fill_(1.0)
        e0.record(stream)
        run(G.RUN_REDUCE)
        e1.record(stream)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    check("cold reduce")
    del flush
    cold_ms = statistics.median(cold)
    _, red_bytes = algorithmic_bytes(w, w.elem_bytes)
    result = {
        "kernel_sync_ms_per_step": round(sync_ms, 4),
        "clear_kernel_ms_per_step": round(clear_ms, 4),
        "clear_only_ms": round(clear_only_ms, 4),
        "clear_kernel_sync_ms_per_step": round(clear_sync_ms, 4),
        "clear_bytes": int(info.staging_bytes),
        "cold_reduce_ms": round(cold_ms, 4),
        "cold_reduce_gbps": round(red_bytes / (cold_ms * 1e-3) / 1e9, 1),
    }
    if w.dtype == "bf16":
        Ab = A.view(torch.bfloat16)
        Bb = B.view(torch.bfloat16).contiguous()
        Cb = torch.empty((w.W, w.M, w.N), dtype=torch.bfloat16, device=out.device)
        for _ in range(2):
            torch.bmm(Ab, Bb, out=Cb)
        e0.record(stream)
        for _ in range(n):
            torch.bmm(Ab, Bb, out=Cb)
        e1.record(stream)
        torch.cuda.synchronize()
        bmm_ms = e0.elapsed_time(e1) / n
        result["torch_bmm_ms"] = round(bmm_ms, 4)
        result["torch_bmm_tflops"] = round(w.flops / (bmm_ms * 1e-3) / 1e12, 2)
        del Cb
    result["note"] = ("ablations and context, not targets: kernel-sync and clear-kernel are "
                      "whole steps; torch_bmm is hipBLASLt on the same GEMMs without the "
                      "scatter epilogue or the reduce")
    return result


def ag_measure(steps, stream):
    """All-gather + GEMM on the Llama-3-70B-like up-projection shard: copy
    alone, GEMM alone (gathered input resident), both in order on one
    stream, and fused (copies on a second stream, tiles gated on signals).
    Overlap efficiency: (T_copy + T_gemm - T_fused) / T_copy."""
    import numpy as np
    import torch
    from tensor_gemm_reduce_lds_amd import gemm_rs as G
    from tensor_gemm_reduce_lds_amd import inputs as I
    p = I.AG_WORKLOADS["llama70b_up"]
    M, N, K, W = p["M"], p["N"], p["K"], p["W"]
    x = I.make_ag_inputs(M, N, K, W, index=p["index"])
    X = torch.from_numpy(x["X"].view(np.int16)).to("cuda:0")
    B = torch.from_numpy(x["B"].view(np.int16)).to("cuda:0")
    del x
    out = torch.empty((W, M, N), dtype=torch.int16, device="cuda:0")
    n = max(5, steps // 2)
    with G.AgPlan(M=M, N=N, K=K, W=W) as ag:
        def timed(flags):
            for _ in range(2):
                ag.run(X, B, out, stream, flags)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(n):
                ag.run(X, B, out, stream, flags)
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t0) * 1e3 / n
            rc, detail = ag.status(stream)
            if rc != G.OK:
                raise RuntimeError("all-gather run failed: %s %s" % (G.gemm_rs_strerror(rc), detail))
            return ms
        copy_ms = timed(G.AG_RUN_COPY)
        gemm_ms = timed(G.AG_RUN_GEMM)
        serial_ms = timed(G.AG_RUN_ALL)
        fused_ms = timed(G.AG_RUN_ALL | G.AG_FUSED)
    flops = W * 2 * M * N * K
    copy_bytes = 2 * W * M * K * 2        # every rank's gathered X read and written
    return {
        "workload": "llama70b up-projection shard (all-gather + GEMM)",
        "W": W, "M": M, "N": N, "K": K,
        "ms_fused": round(fused_ms, 4),
        "value_fused": round(flops / (fused_ms * 1e-3) / 1e12, 2),
        "ms_serial": round(serial_ms, 4),
        "ms_gemm_only": round(gemm_ms, 4),
        "gemm_tflops": round(flops / (gemm_ms * 1e-3) / 1e12, 2),
        "ms_copy_only": round(copy_ms, 4),
        "copy_gbps": round(copy_bytes / (copy_ms * 1e-3) / 1e9, 1),
        "overlap_efficiency": round((copy_ms + gemm_ms - fused_ms) / copy_ms, 3),
        "unit": "TFLOP/s",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama70b")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of CPU oracle work for cpu_baseline (0: skip)")
    ap.add_argument("--no-overlap", action="store_true",
                    help="skip the overlapped-reduce timing (profiling runs: every "
                         "GEMM and reduce launch is then a full launch)")
    ap.add_argument("--fused-only", action="store_true",
                    help="time only the owner-fused steps (the reduce fused into the last "
                         "tile-order step) and print their object (profiling runs of that mode)")
    ap.add_argument("--ag-only", action="store_true",
                    help="time only the all-gather + GEMM half and print its object "
                         "(profiling runs of that path)")
    ap.add_argument("--soak", type=float, default=0.0,
                    help="seconds: only run --soak-kernel back to back for this long after "
                         "a warm-up (board power and clocks can then be sampled from "
                         "outside) and print its launch rate")
    ap.add_argument("--soak-kernel", default="gemm", choices=["gemm", "step", "bmm"],
                    help="what --soak runs: the GEMM launch, the serial step (GEMM and "
                         "reduce), or torch.bmm on the same GEMMs (hipBLASLt, context)")
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="MiB: run one plain device copy of this size first "
                         "(reference point for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only (W virtual ranks on one "
              "device); --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from tensor_gemm_reduce_lds_amd import gemm_rs as G
    from tensor_gemm_reduce_lds_amd import inputs as I

    if args.ag_only:
        print(json.dumps({"ag_gemm": ag_measure(args.steps, torch.cuda.current_stream())}),
              flush=True)
        return

    w = I.WORKLOADS[args.workload]
    log("bench: workload", w)
    t0 = time.perf_counter()
    x = I.make_inputs(w, seed=args.seed)
    log("bench: inputs generated in %.1f s" % (time.perf_counter() - t0))
    dev = torch.device("cuda", 0)

    def up(a):
        if a is None:
            return None
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    A, B, C = up(x["A"]), up(x["B"]), up(x["C"])
    out = torch.empty((w.M, w.N), dtype=torch.int16 if w.dtype == "bf16" else torch.float32,
                      device=dev)
    plan_fields = dict(M=w.M, N=w.N, K=w.K, W=w.W,
                       dtype=G.BF16 if w.dtype == "bf16" else G.F32,
                       tile_m=w.tile_m, tile_n=w.tile_n,
                       order=G.ORDER_TWO_LEVEL if w.order == "two_level" else G.ORDER_FLAT,
                       groups=w.groups, has_c=int(w.has_c), ldc=w.ldc)
    plan = G.Plan(**plan_fields)
    stream = torch.cuda.current_stream()

    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("bench: calibration copy of %d MiB done" % args.copy_calibration)
        del src, dst

    if args.soak > 0:
        if args.soak_kernel == "bmm":
            if w.dtype != "bf16":
                raise SystemExit("--soak-kernel bmm needs a bf16 workload")
            Ab = A.view(torch.bfloat16)
            Bb = B.view(torch.bfloat16).contiguous()
            Cb = torch.empty((w.W, w.M, w.N), dtype=torch.bfloat16, device=dev)
            one = lambda: torch.bmm(Ab, Bb, out=Cb)
        else:
            # the GEMM alone sets every flag again each launch; one reduce
            # after the loop puts them back
            flags = G.RUN_GEMM if args.soak_kernel == "gemm" else G.RUN_ALL
            one = lambda: plan.run(A, B, C, w.alpha, w.beta, out, stream, flags)
        for _ in range(max(args.warmup, 1)):
            one()
        torch.cuda.synchronize()
        log("soak: running %s for %.0f s" % (args.soak_kernel, args.soak))
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < args.soak:
            for _ in range(20):
                one()
            torch.cuda.synchronize()
            n += 20
        dt = time.perf_counter() - t0
        if args.soak_kernel == "gemm":
            plan.run(A, B, C, w.alpha, w.beta, out, stream, G.RUN_REDUCE)
        if args.soak_kernel != "bmm":
            rc, detail = plan.status(stream)
            if rc != G.OK:
                raise RuntimeError("soak run failed: %s %s" % (G.gemm_rs_strerror(rc), detail))
        log("soak: done")
        print(json.dumps({"soak": {"workload": w.name, "kernel": args.soak_kernel,
                                   "seconds": round(dt, 2), "iterations": n,
                                   "ms_per_iteration": round(dt * 1e3 / n, 4)}}), flush=True)
        plan.close()
        return

    if args.fused_only:
        # warm-up, then the timed owner-fused steps with HIP events around
        # each (one run call: both GEMM launches)
        for _ in range(args.warmup):
            plan.run(A, B, C, w.alpha, w.beta, out, stream, G.RUN_ALL | G.OVERLAP_REDUCE)
        fev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            fev[k][0].record(stream)
            plan.run(A, B, C, w.alpha, w.beta, out, stream, G.RUN_ALL | G.OVERLAP_REDUCE)
            fev[k][1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        rc, detail = plan.status(stream)
        if rc != G.OK:
            raise RuntimeError("fused run failed: %s %s" % (G.gemm_rs_strerror(rc), detail))
        ms = sum(e[0].elapsed_time(e[1]) for e in fev) / args.steps
        print(json.dumps({"fused": {"workload": w.name, "steps": args.steps,
                                    "ms_per_step": round(wall * 1e3 / args.steps, 4),
                                    "ms_per_step_events": round(ms, 4),
                                    "value": round(w.flops / (ms * 1e-3) / 1e12, 2)}}),
              flush=True)
        plan.close()
        return

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        plan.run(A, B, C, w.alpha, w.beta, out, stream, G.RUN_GEMM)
        if ev is not None:
            ev[1].record(stream)
        plan.run(A, B, C, w.alpha, w.beta, out, stream, G.RUN_REDUCE)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    rc, detail = plan.status(stream)
    if rc != G.OK:
        raise RuntimeError("warmup failed: %s %s" % (G.gemm_rs_strerror(rc), detail))

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    rc, detail = plan.status(stream)
    if rc != G.OK:
        raise RuntimeError("timed run failed: %s %s" % (G.gemm_rs_strerror(rc), detail))

    # the same steps with the reduce taken off the serial path; whole-step
    # wall time only.  Remote-first order: the owner-fused reduce (every
    # rank's own-chunk step sums its tiles' partials in its epilogue, no
    # separate reduce); identity order (a second plan): chunk c's reduce
    # overlaps the GEMM of chunk c+1 on the plan's second stream.
    def overlapped_ms(p, flags=G.RUN_ALL | G.OVERLAP_REDUCE):
        for _ in range(2):
            p.run(A, B, C, w.alpha, w.beta, out, stream, flags)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(args.steps):
            p.run(A, B, C, w.alpha, w.beta, out, stream, flags)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t1) * 1e3 / args.steps
        rc, detail = p.status(stream)
        if rc != G.OK:
            raise RuntimeError("overlapped run failed: %s %s" % (G.gemm_rs_strerror(rc), detail))
        return ms

    ov_ms = ov_id_ms = la_ms = None
    if not args.no_overlap:
        ov_ms = overlapped_ms(plan)
        la_ms = overlapped_ms(plan, G.RUN_ALL | G.LAST_ARRIVER)
        with G.Plan(**dict(plan_fields, swizzle=G.SWIZZLE_IDENTITY)) as plan_id:
            ov_id_ms = overlapped_ms(plan_id)

    # the optional bfloat16-staging mode (each partial rounded to bfloat16
    # when staged; its own accuracy bar), same serial step, separate plan
    bf16_staging = None
    if not args.no_overlap and w.dtype == "bf16":
        with G.Plan(**dict(plan_fields, staging_dtype=G.STAGING_BF16)) as pb:
            def step_b(ev=None):
                if ev is not None:
                    ev[0].record(stream)
                pb.run(A, B, C, w.alpha, w.beta, out, stream, G.RUN_GEMM)
                if ev is not None:
                    ev[1].record(stream)
                pb.run(A, B, C, w.alpha, w.beta, out, stream, G.RUN_REDUCE)
                if ev is not None:
                    ev[2].record(stream)
            for _ in range(2):
                step_b()
            evb = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
                   for _ in range(args.steps)]
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            for k in range(args.steps):
                step_b(evb[k])
            torch.cuda.synchronize()
            b_step = (time.perf_counter() - t1) * 1e3 / args.steps
            rc, detail = pb.status(stream)
            if rc != G.OK:
                raise RuntimeError("bf16-staging run failed: %s %s" % (G.gemm_rs_strerror(rc), detail))
            b_gemm = sum(e[0].elapsed_time(e[1]) for e in evb) / args.steps
            b_red = sum(e[1].elapsed_time(e[2]) for e in evb) / args.steps
            b_red_bytes = w.W * w.M * w.N * 2 + w.M * w.N * 2
            bf16_staging = {
                "ms_per_step": round(b_step, 4),
                "value": round(w.flops / (b_step * 1e-3) / 1e12, 2),
                "gemm_kernel_ms": round(b_gemm, 4),
                "gemm_tflops": round(w.flops / (b_gemm * 1e-3) / 1e12, 2),
                "reduce_kernel_ms": round(b_red, 4),
                "reduce_gbps": round(b_red_bytes / (b_red * 1e-3) / 1e9, 1),
                "reduce_algorithmic_bytes": b_red_bytes,
                "note": "optional mode: partials staged in bfloat16 (second rounding; "
                        "its own accuracy bar), not the headline configuration",
            }

    ablation = None
    if not args.no_overlap:
        ablation = ablation_measure(plan, A, B, C, out, w, stream, args.steps)

    # all-gather fused into the GEMM prologue, on the up-projection shard of
    # the same layer (a second workload, reported beside the headline)
    ag_gemm = None
    if not args.no_overlap and w.name == "llama70b":
        ag_gemm = ag_measure(args.steps, stream)

    gemm_list = sorted(e[0].elapsed_time(e[1]) for e in evs)
    red_list = sorted(e[1].elapsed_time(e[2]) for e in evs)
    gemm_ms = sum(gemm_list) / args.steps
    red_ms = sum(red_list) / args.steps
    step_ms = wall * 1e3 / args.steps
    flops = w.flops
    elem = w.elem_bytes
    gemm_bytes, red_bytes = algorithmic_bytes(w, elem)
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    red_gbps = red_bytes / (red_ms * 1e-3) / 1e9
    traffic = stored_traffic() if w.name == "llama70b" else None
    info = plan.info
    roofline = gemm_roofline(flops, gemm_bytes, gemm_ms, peak, traffic)

    result = {
        "metric": METRIC,
        "value": round(flops / (step_ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded PCG64: A~N(0,1), B~N(0,1/K), bias~N(0,0.02^2))",
        "config": {"workload": "%s FFN down-projection shard" % w.name, "W": w.W,
                   "M": w.M, "N": w.N, "K": w.K, "alpha": w.alpha, "beta": w.beta,
                   "bias": ("row-broadcast" if w.ldc == 0 else "full") if w.has_c else None,
                   "tile": "%dx%d" % (info.tile_m, info.tile_n), "order": w.order,
                   "staging": "fp32", "parallelism": "1 GPU, %d virtual ranks" % w.W},
        "roofline": roofline,
        "gemm_kernel_ms": round(gemm_ms, 4),
        "gemm_kernel_ms_median": round(gemm_list[len(gemm_list) // 2], 4),
        "gemm_kernel_ms_min": round(gemm_list[0], 4),
        "gemm_tflops": round(gemm_tflops, 2),
        "mfma_util_pct": round(100 * gemm_tflops / peak, 2),
        "gemm_algorithmic_bytes": gemm_bytes,
        "reduce_kernel_ms": round(red_ms, 4),
        "reduce_kernel_ms_median": round(red_list[len(red_list) // 2], 4),
        "reduce_kernel_ms_min": round(red_list[0], 4),
        "reduce_gbps": round(red_gbps, 1),
        "reduce_hbm_frac": round(red_gbps / PEAK_HBM_GBPS, 4),
        "reduce_algorithmic_bytes": red_bytes,
        "overlap_mode": "owner-fused reduce in the last tile-order step (remote-first order)",
        "ms_per_step_overlap": None if ov_ms is None else round(ov_ms, 4),
        "value_overlap": None if ov_ms is None else round(flops / (ov_ms * 1e-3) / 1e12, 2),
        # overlap efficiency as the pages define it: hidden communication
        # (here: reduce) time over hideable time, (T_gemm + T_reduce - T_e2e) / T_reduce
        "overlap_efficiency": (None if ov_ms is None
                               else round((gemm_ms + red_ms - ov_ms) / red_ms, 3)),
        "ms_per_step_overlap_identity": None if ov_id_ms is None else round(ov_id_ms, 4),
        "overlap_efficiency_identity": (None if ov_id_ms is None
                                        else round((gemm_ms + red_ms - ov_id_ms) / red_ms, 3)),
        "value_overlap_identity": (None if ov_id_ms is None
                                   else round(flops / (ov_id_ms * 1e-3) / 1e12, 2)),
        # one launch, each tile summed by its last producer (agent-scope
        # release per producer, acquire per summing workgroup)
        "ms_per_step_last_arriver": None if la_ms is None else round(la_ms, 4),
        "value_last_arriver": None if la_ms is None else round(flops / (la_ms * 1e-3) / 1e12, 2),
        "bf16_staging": bf16_staging,
        "ablation": ablation,
        "ag_gemm": ag_gemm,
    }
    plan.close()
    del A, B, C, out
    if args.cpu_budget > 0:
        log("bench: timing the CPU oracle (~%.0f s)" % args.cpu_budget)
        result["cpu_baseline"] = cpu_baseline(w, x, args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
