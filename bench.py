#!/usr/bin/env python3
"""Benchmark of the swizzled-operand GEMM on one MI355X.

One step = one library call (one kernel launch; two for the split weight-
streaming path) computing the whole product for the workload on inputs
already resident in HBM.  Default workload: the square dense 8192^3 bf16
GEMM with both operands K-major (N(0,1) inputs, seed 0), the metric's "bf16
8192^3".  The other workloads (the single 128x256x64 tile, 4096^3 bf16,
8192^3 fp16 MN-major A with beta=1, the skinny 64x16384x8192 weight-streaming
shape, 8192^3 MX-fp8 -- the metric's second configuration --, 8192^3 MX-fp4,
MX-fp6 in both 6-bit formats, E4M3 A against E2M3, padded E2M1 or dense E2M1
B, and bf16 8192^3 with B MN-major or both operands MN-major) are timed in the same run
and reported under "also", each with its own roofline and sampled oracle
baseline.

Prints ONE JSON line (rank 0).  ``roofline`` reports the dominant kernel
against the MI355X dense MFMA peak (or HBM peak for the skinny shape), using
the average kernel duration from HIP events recorded on the launch stream
over the timed region.  ``cpu_baseline`` times the fp64 oracle, as it stands,
on a bounded sample of the same workload on this host's cores.

Warm-up: after the requested warm-up launches, launches continue until at
least ``--settle-ms`` (default 250 ms) of back-to-back work has passed since
the first one.  The chip's power management needs about 40-60 ms of
sustained MFMA load after an idle start to settle; launches before that run
up to 20 % slower, which would put a short timed region on the transient
rather than on the steady state of a loaded GPU.  The extra warm-up launches
are reported (``warmup_settle``); the timed region is exactly ``--steps``
launches.

``value`` and ``roofline`` come from back-to-back launches, where operands of
256 MiB or less can stay partly resident in the 256 MiB MALL between calls.
``caches_flushed`` therefore reports each workload once more: single calls,
each preceded by an untimed read of another 512 MiB buffer that evicts the
operands from the L2s and the MALL, with the median and minimum per-call time and, for
comparison, the median of the same per-call timing without the flush.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s on 1 MI355X (bf16 8192³, MX-fp8 8192³) and % of MFMA peak"
# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s).
MFMA_PEAK = {"bf16": 2516.6, "f16": 2516.6, "e4m3": 5033.2, "e2m1": 10066.4, "e2m3": 10066.4, "e3m2": 10066.4, "e2m1p": 10066.4}
HBM_PEAK = 8000.0


def mfma_peak(w) -> float:
    """Dense MFMA peak of the workload's operand kinds (the slower one when A
    and B differ: a mixed MFMA runs at the wider format's rate)."""
    return min(MFMA_PEAK[w.kind], MFMA_PEAK[w.kind_b])


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "mma_swizzled_operand_amd", "csrc", "*"))):
        h.update(os.path.basename(p).encode())
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def traffic_for(workload: str, n_launch_units: int = 1):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary of this
    workload, if it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"gemm_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except Exception:
        return None
    if d.get("kernel_hash") != kernel_source_hash():
        return None
    return float(d["hbm_bytes_per_launch"]) * n_launch_units


def setup(w, seed=0):
    import numpy as np
    import torch

    import mma_swizzled_operand_amd as mswz
    import workloads as wl

    x = wl.generate(w, seed=seed)

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).cuda()

    plan = mswz.gemm_plan_create(w.M, w.N, w.K, w.kind, w.kind_b, "f32", w.a_major, w.b_major, w.V)
    A, B = dev(x["A"]), dev(x["B"])
    D = dev(x["D0"]) if w.beta else torch.zeros((w.M, w.N), dtype=torch.float32, device="cuda")
    if w.V:
        if w.sf_major == "mn":   # the same scales stored [K/32][M] and [K/32][N]
            mswz.gemm_plan_set_scale_major(plan, "mn")
            SFA, SFB = dev(x["SFA"].T), dev(x["SFB"].T)
        else:
            SFA, SFB = dev(x["SFA"]), dev(x["SFB"])

        def step():
            mswz.gemm_run_blockscaled(plan, A, B, SFA, SFB, D, w.beta)
    elif plan.workspace_bytes() > 0:
        # weight streaming with K split over workgroups: the library's
        # workspace path (the caller's workspace holds the fp32 partials)
        ws = torch.empty(plan.workspace_bytes(), dtype=torch.uint8, device="cuda")

        def step():
            mswz.gemm_run_ws(plan, A, B, D, ws, w.beta)
    else:
        def step():
            mswz.gemm_run(plan, A, B, D, w.beta)
    return x, plan, step


def warm_up(step, warmup, settle_ms):
    """`warmup` launches, then more until at least settle_ms of back-to-back
    launches have passed since the first (batches sized from the measured
    rate, about 20 ms each).  Returns (extra launches, total ms)."""
    import torch
    t0 = time.perf_counter()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    done, extra = warmup, 0
    while (time.perf_counter() - t0) * 1e3 < settle_ms:
        per = max((time.perf_counter() - t0) * 1e3 / max(done, 1), 1e-3)
        n = max(1, min(int(20.0 / per), 100000))
        for _ in range(n):
            step()
        torch.cuda.synchronize()
        done += n
        extra += n
    return extra, (time.perf_counter() - t0) * 1e3


def time_steps(step, steps, warmup, settle_ms=0.0):
    """Wall time of `steps` launches, and their mean duration from two HIP
    events on the launch stream bracketing the timed region (events between
    launches would each add a few microseconds of idle GPU time); also the
    warm-up's extra launches and length."""
    import torch
    settle = warm_up(step, warmup, settle_ms)
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, ev0.elapsed_time(ev1) / steps, settle


# Bytes of the buffer copied between calls to empty the caches: twice the
# 256 MiB MALL (Infinity Cache) and far beyond the 8 x 4 MiB of L2.
FLUSH_BYTES = 512 << 20


def make_flush():
    """A callable that reads FLUSH_BYTES of another buffer (a sum into one
    scalar), which evicts every line of the operands from the L2s and the MALL
    and leaves them holding clean lines.  A flush that writes (a copy, a fill)
    leaves dirty lines whose write-back then lands inside the next timed call:
    measured on the skinny shape, a copy flush makes the call 1.36x and a fill
    1.7x slower than this read-only flush does."""
    import torch
    buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    acc = torch.zeros((), dtype=torch.float32, device="cuda")
    return lambda: torch.sum(buf, dim=0, out=acc)


def per_call_ms(step, calls, flush=None):
    """Duration of each of `calls` library calls, from one HIP event pair per
    call on the launch stream; with `flush`, the (untimed) cache flush runs
    before every call.  Sorted ascending."""
    import torch
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(calls)]
    for e0, e1 in evs:
        if flush is not None:
            flush()
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    return sorted(e0.elapsed_time(e1) for e0, e1 in evs)


def cold_entry(w, warm_ms, cold_ms):
    """Median and minimum per-call time with and without the flush, and the
    rates at the flushed median."""
    med = cold_ms[len(cold_ms) // 2]
    out = {"calls": len(cold_ms), "flushed_us_median": round(med * 1e3, 2),
           "flushed_us_min": round(cold_ms[0] * 1e3, 2),
           "unflushed_us_median": round(warm_ms[len(warm_ms) // 2] * 1e3, 2),
           "TFLOP/s": round(w.flops / (med * 1e-3) / 1e12, 1),
           "frac_mfma_peak": round(w.flops / (med * 1e-3) / 1e12 / mfma_peak(w), 4),
           "GB/s_algorithmic": round(w.algorithmic_bytes() / (med * 1e-3) / 1e9, 1)}
    if w.name == "c4":
        out["frac_hbm_peak"] = round(out["GB/s_algorithmic"] / HBM_PEAK, 4)
    return out


def measure(name, steps, warmup, cold=0, flush=None, settle_ms=0.0):
    import workloads as wl
    w = wl.WORKLOADS[name]
    log(f"{name}: generating inputs ({w.title})")
    x, plan, step = setup(w)
    log(f"{name}: plan {plan.describe()}; timing {steps} steps after {warmup} warm-up "
        f"(and at least {settle_ms:.0f} ms of warm-up launches)")
    wall, avg_ms, (extra, settle_total) = time_steps(step, steps, warmup, settle_ms)
    r = {
        "warmup_settle": {"extra_launches": extra, "warmup_ms": round(settle_total, 1)},
        "workload": w,
        "inputs": x,
        "plan": plan.describe(),
        "wall_s": wall,
        "ms_per_step": wall / steps * 1e3,
        "kernel_avg_ms": avg_ms,
        "tflops": w.flops / (wall / steps) / 1e12,
        "kernel_tflops": w.flops / (avg_ms * 1e-3) / 1e12,
        "kernel_gbs": w.algorithmic_bytes() / (avg_ms * 1e-3) / 1e9,
    }
    log(f"{name}: {r['kernel_avg_ms'] * 1e3:.1f} us/launch, {r['kernel_tflops']:.1f} TFLOP/s, "
        f"{r['kernel_gbs']:.0f} GB/s algorithmic")
    if cold:
        # after the timed region, so that its dispatches stay contiguous
        r["cold"] = cold_entry(w, per_call_ms(step, cold), per_call_ms(step, cold, flush))
        log(f"{name}: caches flushed before each call: {r['cold']['flushed_us_median']:.1f} us "
            f"median ({r['cold']['unflushed_us_median']:.1f} us unflushed, one event pair per call)")
    return r


def cpu_baseline(w, x, target_s):
    """The oracle, unmodified, on the first R rows of the workload's output
    (R a multiple of the thread count, grown until ~target_s of CPU work)."""
    import oracle
    threads = oracle.get_threads()

    def run(r):
        t0 = time.perf_counter()
        oracle.gemm(w.M, w.N, w.K, w.kind, w.a_major, x["A"], w.kind_b, w.b_major, x["B"],
                    V=w.V, SFA=x.get("SFA"), SFB=x.get("SFB"), beta=w.beta, D0=x.get("D0"),
                    rows=list(range(r)))
        return time.perf_counter() - t0

    # each call also decodes all of B once, so the first small sample
    # overstates the time per row: grow in up to three rounds
    r = min(threads, w.M)
    t = run(r)
    for _ in range(3):
        if t >= 0.6 * target_s or r >= w.M:
            break
        r = min(w.M, max(r + threads, int(r * target_s / max(t, 1e-3)) // threads * threads))
        t = run(r)
    flops = 2.0 * r * w.N * w.K
    return {"value": round(flops / t / 1e12, 5), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"first {r} of {w.M} output rows (all {w.N} columns, K={w.K}) of the "
                      f"same workload in fp64: {flops / 1e9:.2f} GFLOP in {t:.2f} s"}


# One compute unit's share of the bf16 / fp16 dense peak (256 CUs): the bound
# of a one-workgroup launch such as the single 128x256 tile.
ONE_CU_PEAK = MFMA_PEAK["bf16"] / 256


def roofline_of(r):
    """The roofline object of one measured workload: HBM-bound for the skinny
    weight-streaming shape, MFMA-bound (the operand kinds' dense peak)
    otherwise, from the launch-averaged kernel duration."""
    w = r["workload"]
    if w.name == "c4":
        achieved, peak, unit, bound = r["kernel_gbs"], HBM_PEAK, "GB/s", "hbm"
    else:
        achieved, peak, unit, bound = r["kernel_tflops"], mfma_peak(w), "TFLOP/s", "mfma"
    return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic_for(w.name)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--settle-ms", type=float, default=250.0,
                    help="keep warming up until this many ms of back-to-back launches have passed")
    ap.add_argument("--workload", default="c3b")
    ap.add_argument("--also", default="c5,c1,c2,c3,c4,c6,c7,c8,c9,c10,c11,c12,c13,c14",
                    help="comma-separated extra workloads timed in the same run ('' for none)")
    ap.add_argument("--cold-calls", type=int, default=50,
                    help="after the timed steps, time this many single calls of each workload "
                         "with the L2s and the MALL flushed before every call (0: skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="oracle sample length for the headline workload")
    ap.add_argument("--cpu-seconds-also", type=float, default=2.0,
                    help="oracle sample length for each 'also' workload")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of the GEMM, time a plain device-to-device copy of this many "
                         "bytes (used to calibrate the HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the GEMM path is built and timed on a single "
              "MI355X; multi-GPU sharding is a design note, not a measured path.", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as wl
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    import mma_swizzled_operand_amd as mswz
    mswz.load()

    if args.copy_bytes:
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device="cuda").random_(0, 255)
        dst = torch.empty_like(src)
        wall, avg_ms, _ = time_steps(lambda: dst.copy_(src), args.steps, args.warmup, args.settle_ms)
        print(json.dumps({"copy_bytes": args.copy_bytes, "steps": args.steps,
                          "avg_ms": round(avg_ms, 5),
                          "GB/s": round(2 * args.copy_bytes / (avg_ms * 1e-3) / 1e9, 1)}), flush=True)
        return

    names = [args.workload] + [s for s in args.also.split(",") if s and s != args.workload]
    for n in names:
        if n not in wl.WORKLOADS:
            raise SystemExit(f"unknown workload {n}")
    flush = make_flush() if args.cold_calls else None
    head = measure(args.workload, args.steps, args.warmup, args.cold_calls, flush, args.settle_ms)
    w = head["workload"]
    roofline = roofline_of(head)

    also = {}
    for name in names[1:]:
        r = measure(name, args.steps, args.warmup, args.cold_calls, flush, args.settle_ms)
        ow = r["workload"]
        entry = {"title": ow.title, "us_per_call": round(r["kernel_avg_ms"] * 1e3, 2),
                 "TFLOP/s": round(r["kernel_tflops"], 1),
                 "frac_mfma_peak": round(r["kernel_tflops"] / mfma_peak(ow), 4),
                 "GB/s_algorithmic": round(r["kernel_gbs"], 1),
                 "tile": [r["plan"]["tile_m"], r["plan"]["tile_n"], r["plan"]["tile_k"]],
                 "roofline": roofline_of(r),
                 "warmup_settle": r["warmup_settle"]}
        if ow.name == "c4":
            entry["frac_hbm_peak"] = round(r["kernel_gbs"] / HBM_PEAK, 4)
        if ow.name == "c1":
            # one workgroup: the bound is one compute unit's share of the peak
            entry["frac_one_cu_peak"] = round(r["kernel_tflops"] / ONE_CU_PEAK, 4)
        if "cold" in r:
            entry["caches_flushed"] = r["cold"]
        if not args.no_cpu_baseline:
            log(f"cpu baseline: oracle on a sample of {name} (~{args.cpu_seconds_also:.0f} s)")
            entry["cpu_baseline"] = cpu_baseline(ow, r["inputs"], args.cpu_seconds_also)
        also[name] = entry
        del r

    cpu = None
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on a sample of {w.name} (~{args.cpu_seconds:.0f} s)")
        cpu = cpu_baseline(w, head["inputs"], args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(head["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.kind,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.title}", "M": w.M, "N": w.N, "K": w.K,
                   "a_major": w.a_major, "b_major": w.b_major, "beta": w.beta,
                   "scale_vec_len": w.V, "tile": head["plan"], "frac_mfma_peak":
                   round(head["kernel_tflops"] / mfma_peak(w), 4)},
        "roofline": roofline,
        "kernel_avg_us": round(head["kernel_avg_ms"] * 1e3, 2),
        "warmup_settle": head["warmup_settle"],
        "caches_flushed": head.get("cold"),
        "cpu_baseline": cpu,
        "also": also,
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
