#!/usr/bin/env python3
"""Benchmark of the swizzled-operand GEMM on one MI355X.

One step = one library call (one kernel launch) computing the whole product
for the workload on inputs already resident in HBM.  Default workload: the
square dense 4096^3 bf16 GEMM with both operands K-major (N(0,1) inputs,
seed 0).  The other full-size workloads (8192^3 fp16 MN-major A with beta=1,
8192^3 bf16, the skinny 64x16384x8192 weight-streaming shape, 8192^3 MX-fp8,
8192^3 MX-fp4, 8192^3 MX-fp6 in both 6-bit formats, and 8192^3 with E4M3 A
against E2M3 or padded E2M1 B) are timed in the same run and reported under
"also".

Prints ONE JSON line (rank 0).  ``roofline`` reports the dominant kernel
against the MI355X dense MFMA peak (or HBM peak for the skinny shape), using
the average kernel duration from HIP events recorded on the launch stream
over the timed region.  ``cpu_baseline`` times the fp64 oracle, as it stands,
on a bounded sample of the same workload on this host's cores.

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
        SFA, SFB = dev(x["SFA"]), dev(x["SFB"])

        def step():
            mswz.gemm_run_blockscaled(plan, A, B, SFA, SFB, D, w.beta)
    elif plan.workspace_bytes() > 0:
        # weight streaming with K split over workgroups: the library's
        # workspace path (zero-filled once; every call leaves it so)
        ws = torch.zeros(plan.workspace_bytes(), dtype=torch.uint8, device="cuda")

        def step():
            mswz.gemm_run_ws(plan, A, B, D, ws, w.beta)
    else:
        def step():
            mswz.gemm_run(plan, A, B, D, w.beta)
    return x, plan, step


def time_steps(step, steps, warmup):
    """Wall time of `steps` launches, and their mean duration from two HIP
    events on the launch stream bracketing the timed region (events between
    launches would each add a few microseconds of idle GPU time)."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, ev0.elapsed_time(ev1) / steps


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


def measure(name, steps, warmup, cold=0, flush=None):
    import workloads as wl
    w = wl.WORKLOADS[name]
    log(f"{name}: generating inputs ({w.title})")
    x, plan, step = setup(w)
    log(f"{name}: plan {plan.describe()}; timing {steps} steps after {warmup} warm-up")
    wall, avg_ms = time_steps(step, steps, warmup)
    r = {
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

    r = min(threads, w.M)
    t = run(r)
    grow = max(1, min(int(target_s / max(t, 1e-3)), w.M // r))
    if grow > 1:
        r *= grow
        t = run(r)
    flops = 2.0 * r * w.N * w.K
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"first {r} of {w.M} output rows (all {w.N} columns, K={w.K}) of the "
                      f"same workload in fp64: {flops / 1e9:.1f} GFLOP in {t:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # The default warm-up (400 launches, 45 ms to 0.4 s of back-to-back work
    # depending on the workload) outlasts the chip's power-management settling
    # after an idle start, about the first 40 ms of sustained MFMA load,
    # during which launches run up to 20 % slower; the timed steps then see
    # the steady clock that a continuously loaded GPU runs at.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--workload", default="c2")
    ap.add_argument("--also", default="c3,c3b,c4,c5,c6,c7,c8,c9,c10",
                    help="comma-separated extra workloads timed in the same run ('' for none)")
    ap.add_argument("--cold-calls", type=int, default=50,
                    help="after the timed steps, time this many single calls of each workload "
                         "with the L2s and the MALL flushed before every call (0: skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
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
        wall, avg_ms = time_steps(lambda: dst.copy_(src), args.steps, args.warmup)
        print(json.dumps({"copy_bytes": args.copy_bytes, "steps": args.steps,
                          "avg_ms": round(avg_ms, 5),
                          "GB/s": round(2 * args.copy_bytes / (avg_ms * 1e-3) / 1e9, 1)}), flush=True)
        return

    if args.workload not in wl.WORKLOADS:
        raise SystemExit(f"unknown workload {args.workload}")
    flush = make_flush() if args.cold_calls else None
    head = measure(args.workload, args.steps, args.warmup, args.cold_calls, flush)
    w = head["workload"]

    hbm = w.name == "c4"
    if hbm:
        achieved, peak, unit = head["kernel_gbs"], HBM_PEAK, "GB/s"
    else:
        achieved, peak, unit = head["kernel_tflops"], mfma_peak(w), "TFLOP/s"
    roofline = {"bound": "hbm" if hbm else "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": unit, "frac": round(achieved / peak, 4),
                "traffic": traffic_for(w.name)}

    also = {}
    for name in [s for s in args.also.split(",") if s and s != args.workload]:
        r = measure(name, args.steps, args.warmup, args.cold_calls, flush)
        ow = r["workload"]
        entry = {"title": ow.title, "us_per_call": round(r["kernel_avg_ms"] * 1e3, 2),
                 "TFLOP/s": round(r["kernel_tflops"], 1),
                 "frac_mfma_peak": round(r["kernel_tflops"] / mfma_peak(ow), 4),
                 "GB/s_algorithmic": round(r["kernel_gbs"], 1),
                 "tile": [r["plan"]["tile_m"], r["plan"]["tile_n"], r["plan"]["tile_k"]]}
        if ow.name == "c4":
            entry["frac_hbm_peak"] = round(r["kernel_gbs"] / HBM_PEAK, 4)
        if "cold" in r:
            entry["caches_flushed"] = r["cold"]
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
        "caches_flushed": head.get("cold"),
        "cpu_baseline": cpu,
        "also": also,
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
