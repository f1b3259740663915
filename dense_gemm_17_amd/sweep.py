#!/usr/bin/env python3
"""Time every kernel of libmi355gemm on every workload it takes.

The workloads are the plain products of the benchmark set and the
transposed-factor and batched ones (GPT backward pass, attention).

For each (workload, kernel) pair the kernel is forced through the library's
test hook and timed with HIP events around back-to-back calls on one stream
(median of several windows).  Bandwidth-bound shapes rotate through copies of
their operands whose total exceeds the 256 MB last-level cache, so HBM, not
the cache, is measured.  An "identity null" (a 1 x 1 x 1 product: one launch
doing nothing measurable) is timed the same way, as the devpost write-up does
("How we know the numbers are real"), to show the launch floor.

Each line also records the GPU core clock and board power sampled while that
pair was timed, and the first line the toolchain.  With --processes N the
sweep runs N times in fresh child processes and reports, per pair, the
median and the range of the N per-process times (the timing protocol of the
devpost write-up, "How we know the numbers are real": separate processes,
median and spread, beside the identity null).

Output: one JSON line per pair, with the dispatch table's own choice marked.
Usage:  python dense_gemm_17_amd/sweep.py [--workloads a,b] [--windows 5] [--processes 3]
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

import dense_gemm_17_amd as g  # noqa: E402
import workloads  # noqa: E402
from dense_gemm_17_amd.measure import ClockSampler, toolchain  # noqa: E402

PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6, "f16": 2516.6, "fp8": 5033.2}
LLC_BYTES = 256 * 1024 * 1024
CODE = {"f32": g.F32, "bf16": g.BF16, "f16": g.F16, "fp8": g.FP8}
ALL_WORKLOADS = {**workloads.WORKLOADS, **workloads.GENERAL_WORKLOADS, **workloads.FP8_WORKLOADS}


def operands(w, dev):
    """(a, b, c) on the device for workload w: plain products as (M, K),
    (K, N); transposed or batched ones as the views a caller passes."""
    if w.name in workloads.FP8_WORKLOADS:
        A, Bt = workloads.make_fp8_inputs(w)
        return A.to(dev), Bt.to(dev).t(), torch.empty((w.M, w.N), dtype=torch.float32, device=dev)
    if w.name in workloads.GENERAL_WORKLOADS:
        As, Bs = workloads.make_general_inputs(w)
        a, b = workloads.general_views(w, As.to(dev), Bs.to(dev))
        shape = (w.batch, w.M, w.N) if w.batch > 1 else (w.M, w.N)
    else:
        A, B = workloads.make_inputs(w)
        a, b, shape = A.to(dev), B.to(dev), (w.M, w.N)
    return a, b, torch.empty(shape, dtype=torch.float32, device=dev)


def plan(w, a, b, c):
    """The kernel id the library picks (or the forced one accepts) for
    gemm(a, b, out=c), as a pure host call."""
    code = CODE[w.dtype]
    if w.name in workloads.FP8_WORKLOADS:
        return g.gemm_plan_batched(code, 0, 1, w.M, w.N, w.K, 1, A=a.data_ptr(),
                                   lda=a.stride(-2), stride_a=0, B=b.data_ptr(),
                                   ldb=b.stride(-1), stride_b=0, C=c.data_ptr(),
                                   ldc=c.stride(-2), stride_c=0)
    if w.name not in workloads.GENERAL_WORKLOADS:
        return g.gemm_plan(code, w.M, w.N, w.K, a.data_ptr(), a.stride(0), b.data_ptr(),
                           b.stride(0), c.data_ptr(), c.stride(0))
    ta, lda = g._layout(a, "a")
    tb, ldb = g._layout(b, "b")
    return g.gemm_plan_batched(code, ta, tb, w.M, w.N, w.K, w.batch, A=a.data_ptr(), lda=lda,
                               stride_a=g._batch_stride(a), B=b.data_ptr(), ldb=ldb,
                               stride_b=g._batch_stride(b), C=c.data_ptr(), ldc=c.stride(-2),
                               stride_c=g._batch_stride(c))


def time_calls(fn, windows: int, target_ms: float = 60.0, max_reps: int = 2000) -> float:
    """Median per-call milliseconds over `windows` event-timed windows."""
    s = torch.cuda.current_stream()
    fn(); fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s); fn(); e1.record(s); torch.cuda.synchronize()
    one = max(e0.elapsed_time(e1), 1e-3)
    reps = max(1, min(max_reps, int(target_ms / one), 2000))
    out = []
    for _ in range(windows):
        e0.record(s)
        for _ in range(reps):
            fn()
        e1.record(s)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / reps)
    out.sort()
    return out[len(out) // 2]


def repeat_in_processes(args):
    """Run the sweep args.processes times, each in a fresh process (this
    process never touches the GPU), and print median and range per pair."""
    cmd = [sys.executable, os.path.abspath(__file__), "--workloads", args.workloads,
           "--windows", str(args.windows), "--max-reps", str(args.max_reps)]
    if args.table_only:
        cmd.append("--table-only")
    runs = []
    for i in range(args.processes):
        lines = []
        with subprocess.Popen(cmd, stdout=subprocess.PIPE, text=True) as proc:
            for raw in proc.stdout:              # pass each line on as progress
                if raw.startswith("{"):
                    d = json.loads(raw)
                    lines.append(d)
                    print(json.dumps({"process": i, **d}), flush=True)
        if proc.returncode != 0:
            sys.exit(proc.returncode)
        runs.append(lines)
    head = runs[0][0]
    nulls = [r[0]["ms"] for r in runs]
    print(json.dumps({"workload": "identity_null_1x1x1", "processes": args.processes,
                      "ms_median": round(statistics.median(nulls), 5),
                      "ms_min": min(nulls), "ms_max": max(nulls),
                      "toolchain": head.get("toolchain")}), flush=True)
    keyed = {}
    for r in runs:
        for d in r[1:]:
            keyed.setdefault((d["workload"], d["kernel"]), []).append(d)
    for (wl, k), ds in keyed.items():
        ms = [d["ms"] for d in ds]
        med = statistics.median(ms)
        w = ALL_WORKLOADS[wl]
        tflops = w.flops / (med * 1e-3) / 1e12
        sclk = [d["sclk_mhz"]["median"] for d in ds if d.get("sclk_mhz")]
        print(json.dumps({
            "workload": wl, "M": w.M, "N": w.N, "K": w.K, "dtype": w.dtype, "kernel": k,
            "table_choice": ds[0]["table_choice"], "processes": len(ds),
            "ms_median": round(med, 5), "ms_min": min(ms), "ms_max": max(ms),
            "tflops": round(tflops, 2), "frac_peak": round(tflops / PEAK_TFLOPS[w.dtype], 4),
            "gbs": round(w.algorithmic_bytes / (med * 1e-3) / 1e9, 1),
            "sclk_mhz_median": statistics.median(sclk) if sclk else None,
            "operand_copies": ds[0]["operand_copies"]}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--workloads", default=",".join(ALL_WORKLOADS))
    ap.add_argument("--windows", type=int, default=5)
    ap.add_argument("--processes", type=int, default=1)
    ap.add_argument("--table-only", action="store_true",
                    help="time only the dispatch table's choice for each workload")
    ap.add_argument("--max-reps", type=int, default=2000,
                    help="calls per timing window at most (keep small under a counter profiler)")
    ap.add_argument("--kernel", default=None,
                    help="time only this kernel (forced) on each workload that it takes")
    ap.add_argument("--no-null", action="store_true",
                    help="skip the identity null (counter runs: every library dispatch is then "
                         "the workload's)")
    args = ap.parse_args()
    if args.processes > 1:
        repeat_in_processes(args)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if not args.no_null:
        a1 = torch.ones((1, 1), device=dev)
        null_ms = time_calls(lambda: g.gemm(a1, a1), args.windows, max_reps=args.max_reps)
        print(json.dumps({"workload": "identity_null_1x1x1", "ms": round(null_ms, 5),
                          "toolchain": toolchain(g.gemm_build_info())}), flush=True)

    for name in args.workloads.split(","):
        w = ALL_WORKLOADS[name]
        per_copy = w.algorithmic_bytes
        copies = 1 if per_copy * 2 > LLC_BYTES else max(2, -(-2 * LLC_BYTES // per_copy))
        ops = [operands(w, dev) for _ in range(copies)]
        code = CODE[w.dtype]
        table = plan(w, *ops[0])
        for kid in range(g.gemm_kernel_count()):
            if g.gemm_kernel_dtype(kid) != code:
                continue
            if g.gemm_kernel_name(kid).startswith("naive") and w.flops > 4e11:
                continue
            if args.table_only and kid != table:
                continue
            if args.kernel and g.gemm_kernel_name(kid) != args.kernel:
                continue
            g.gemm_force_kernel(kid)
            try:
                if plan(w, *ops[0]) != kid:
                    continue
                state = {"i": 0}

                def call():
                    a, b, c = ops[state["i"] % copies]
                    state["i"] += 1
                    g.gemm(a, b, out=c)

                with ClockSampler() as clocks:
                    ms = time_calls(call, args.windows, max_reps=args.max_reps)
            finally:
                g.gemm_force_kernel(-1)
            tflops = w.flops / (ms * 1e-3) / 1e12
            print(json.dumps({
                "workload": name, "M": w.M, "N": w.N, "K": w.K, "dtype": w.dtype,
                "kernel": g.gemm_kernel_name(kid), "table_choice": kid == table,
                "ms": round(ms, 5), "tflops": round(tflops, 2),
                "frac_peak": round(tflops / PEAK_TFLOPS[w.dtype], 4),
                "gbs": round(w.algorithmic_bytes / (ms * 1e-3) / 1e9, 1),
                "operand_copies": copies, **clocks.summary()}), flush=True)
        del ops
        torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
