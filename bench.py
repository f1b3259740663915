#!/usr/bin/env python3
"""Throughput of libmi355gemm on one MI355X: GFLOP/s (2MNK/t) at 8192^3.

One step = one fp32 GEMM and one bf16-in / fp32-accumulate GEMM, both
8192 x 8192 x 8192 row-major, through the C-ABI on torch's current stream,
with operands resident in HBM before timing starts.  `value` is the step's
total flops over its time.  Each GEMM is also bracketed by HIP events, which
give the per-kernel average durations used for the roofline fractions.

Prints exactly one JSON line.  Extra legs:
  --cpu-baseline (default on): the CPU oracle on a bounded sample of the same
      workload (a few rows of each product) on this host's cores.
  --copy-calibration: also runs a plain device copy of known size, so that
      hardware byte counters (FETCH_SIZE / WRITE_SIZE) read under a profiler
      can be scaled against it.
  --ingest-counters FETCH_DIR WRITE_DIR: turn two rocprofv3 --pmc runs of
      this script (FETCH_SIZE, then WRITE_SIZE, with --copy-calibration) into
      profiles/hbm_traffic_8192.txt: HBM bytes per launch of each kernel,
      scaled by what the counters read for the copy, tagged with a digest of
      the kernel's sources.  The benchmark line reports that traffic for the
      dominant kernel only while the digest still matches (else null).
  other configurations (default on, --no-configs skips it): the table's
      kernel on every other workload of the set (the small, GPT-shaped,
      skinny and ragged products), time per call of back-to-back calls (and
      of a replayed HIP graph for calls under 20 us), the roofline it sits under (HBM below the ridge point, the
      matrix cores above) and a sampled check against the oracle.  Context
      beside the step, not part of `value`.
  Every line also records the GPU clock and board power sampled over the
  timed steps and the toolchain.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import workloads  # noqa: E402

PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6, "f16": 2516.6,     # MI355X dense, per dtype
               "fp8": 5033.2}
HBM_PEAK_GBS = 8000.0
METRIC = "GFLOP/s (2MNK/t) fp32 & bf16 GEMM at 8192³; % of MI355X dtype peak"
STEP_WORKLOADS = ("f32_8192", "bf16_8192")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_8192.txt")
CSRC = os.path.join(ROOT, "dense_gemm_17_amd", "csrc")
# library kernel name -> (symbol substring in profiler output, source files)
KERNEL_SOURCES = {
    "mfma_f32": ("mfma_f32_kernel<256, 256, true>", ["mfma_f32.hip"]),
    "mfma_f32_128": ("mfma_f32_kernel<128, 128, true>", ["mfma_f32.hip"]),
    "mfma_f32_direct": ("mfma_f32_direct_kernel<256, 256, 16, false, false, false, false, false>",
                        ["mfma_f32.hip"]),
    "mfma_bf16_direct": ("mfma_bf16_d16_kernel<true, false, false, false, false>",
                         ["mfma_bf16.hip"]),
    "mfma_bf16": ("mfma_bf16_kernel<true>", ["mfma_bf16.hip"]),
}
# The traffic a kernel causes is set by its own source and the tile order;
# gemm_internal.h only declares the launchers and the host-side argument
# struct, so it is not part of the digest.
COMMON_SOURCES = ["tile_map.h"]
COPY_BYTES = 256 * 1024 * 1024


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workloads", default=",".join(STEP_WORKLOADS),
                   help="comma-separated workload names making up one step")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target length of the CPU-baseline sample")
    p.add_argument("--copy-calibration", action="store_true")
    p.add_argument("--check-rows", type=int, default=8,
                   help="rows per product checked against the oracle after timing")
    p.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    p.add_argument("--runs", type=int, default=3,
                   help="processes the step is timed in (this one and runs-1 children, each "
                        "started before this process touches the GPU) for the spread")
    p.add_argument("--child", action="store_true", help=argparse.SUPPRESS)
    p.add_argument("--no-configs", action="store_true",
                   help="skip the other configurations' section (profiler runs of the step)")
    return p.parse_args()


def code_text(path: str) -> str:
    """Source text without comments and with whitespace runs collapsed: what
    the compiler sees of it (a comment edit does not change the kernel)."""
    return code_text_from(open(path, encoding="utf-8").read())


def code_text_from(text: str) -> str:
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest(kernel: str):
    if kernel not in KERNEL_SOURCES:
        return None
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel][1] + COMMON_SOURCES:
        h.update(code_text(os.path.join(CSRC, f)).encode())
    return h.hexdigest()[:16]


def read_counter(run_dir: str, counter: str):
    """{kernel symbol: [KiB per dispatch, ...]} from a rocprofv3 --pmc run."""
    out = {}
    for path in glob.glob(os.path.join(run_dir, "*counter_collection.csv")):
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                out.setdefault(r["Kernel_Name"], []).append(
                    (int(r["Grid_Size"]), float(r["Counter_Value"])))
    return out


def ingest_counters(fetch_dir: str, write_dir: str):
    fetch = read_counter(fetch_dir, "FETCH_SIZE")
    write = read_counter(write_dir, "WRITE_SIZE")

    def copy_kib(table):
        vals = [v for name, rows in table.items() if "copyBuffer" in name
                for (grid, v) in rows]
        return max(vals)   # the 256 MiB device copy is the largest copy dispatch

    fetch_scale = COPY_BYTES / (copy_kib(fetch) * 1024)
    write_scale = COPY_BYTES / (copy_kib(write) * 1024)
    rec = {"copy_bytes": COPY_BYTES, "fetch_scale": round(fetch_scale, 4),
           "write_scale": round(write_scale, 4), "kernels": {}}
    for kernel, (sym, _) in KERNEL_SOURCES.items():
        f = [v for name, rows in fetch.items() if sym in name for (_, v) in rows]
        w = [v for name, rows in write.items() if sym in name for (_, v) in rows]
        if not f or not w:
            continue
        fb = sum(f) / len(f) * 1024 * fetch_scale
        wb = sum(w) / len(w) * 1024 * write_scale
        rec["kernels"][kernel] = {"fetch_bytes": round(fb), "write_bytes": round(wb),
                                  "bytes_per_launch": round(fb + wb), "dispatches": len(f),
                                  "source_digest": source_digest(kernel)}
    with open(TRAFFIC_FILE, "w") as fh:
        run = ("python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-configs "
               "--copy-calibration --runs 1")
        fh.write("# Bytes between L2 and the memory fabric per launch at 8192^3 (L2 misses:\n"
                 "# MALL hits included), one rocprofv3 run per counter:\n")
        for ctr, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
            fh.write(f"#   timeout -s KILL 120 rocprofv3 --pmc {ctr} -d {d} -o pmc "
                     f"--output-format csv -- {run}\n")
        fh.write("# then: python bench.py --ingest-counters <fetch dir> <write dir>.\n")
        fh.write("# Each counter is scaled by its reading of a 256 MiB device copy.\n")
        fh.write(json.dumps(rec, indent=1) + "\n")
    print(json.dumps(rec))


def traffic_for(kernel: str):
    """HBM bytes per launch for `kernel`, or None if not measured for the
    current sources."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    rec = json.loads(text[text.index("{"):])
    k = rec.get("kernels", {}).get(kernel)
    if not k or k.get("source_digest") != source_digest(kernel):
        return None
    return k["bytes_per_launch"]


def cpu_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit():
        n = min(n, int(cap))
    return max(1, n)


def main():
    args = parse()
    if args.ingest_counters:
        ingest_counters(*args.ingest_counters)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    # The spread over separate processes: the children run first, before
    # this process initialises the GPU, each timing the same step on its own.
    children = []
    if not args.child:
        for _ in range(max(0, args.runs - 1)):
            children.append(child_run(args))
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import dense_gemm_17_amd as g   # fails loudly if the HIP library is missing
    from dense_gemm_17_amd.measure import ClockSampler, toolchain

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    names = [n for n in args.workloads.split(",") if n]
    ws = [workloads.WORKLOADS[n] for n in names]

    host = {}
    ops = []
    for w in ws:
        A, B = workloads.make_inputs(w)
        host[w.name] = (A, B)
        Ad, Bd = A.to(dev), B.to(dev)
        Cd = torch.empty((w.M, w.N), dtype=torch.float32, device=dev)
        ops.append((w, Ad, Bd, Cd))
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)

    def step(evs=None):
        for i, (w, Ad, Bd, Cd) in enumerate(ops):
            if evs is not None:
                evs[i][0].record(stream)
            g.gemm(Ad, Bd, out=Cd)
            if evs is not None:
                evs[i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    kernel_of = {w.name: g.gemm_kernel_name(g.gemm_plan(
        CODE[w.dtype], w.M, w.N, w.K,
        Ad.data_ptr(), Ad.stride(0), Bd.data_ptr(), Bd.stride(0), Cd.data_ptr(), Cd.stride(0)))
        for (w, Ad, Bd, Cd) in ops}

    ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
           for _ in ops] for _ in range(args.steps)]
    torch.cuda.synchronize()
    with ClockSampler() as clocks:
        t0 = time.perf_counter()
        for s in range(args.steps):
            step(ev[s])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0

    per = {}
    for i, (w, *_rest) in enumerate(ops):
        ms = [ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps)]
        avg = float(np.mean(ms))
        tflops = w.flops / (avg * 1e-3) / 1e12
        per[w.name] = {
            "kernel": kernel_of[w.name], "M": w.M, "N": w.N, "K": w.K, "dtype": w.dtype,
            "avg_ms": round(avg, 4), "min_ms": round(float(np.min(ms)), 4),
            "max_ms": round(float(np.max(ms)), 4),
            "tflops": round(tflops, 2), "frac_peak": round(tflops / PEAK_TFLOPS[w.dtype], 4),
        }

    total_flops = sum(w.flops for w in ws)
    ms_per_step = wall * 1e3 / args.steps
    value = total_flops / (wall / args.steps) / 1e9
    if args.child:
        print(json.dumps({"ms_per_step": ms_per_step,
                          "avg_ms": {n: r["avg_ms"] for n, r in per.items()}}), flush=True)
        return
    null_us = identity_null(dev, args.steps * len(ops))

    # correctness of what was timed: a few rows against the oracle
    check = {}
    cpu = None
    import oracle
    rng = np.random.default_rng(0)
    for (w, Ad, Bd, Cd) in ops:
        A, B = host[w.name]
        rows = sorted(set([0, w.M - 1] + rng.choice(w.M, size=min(w.M, args.check_rows),
                                                     replace=False).tolist()))
        fn = getattr(oracle, "gemm_" + w.dtype)
        Cref, D = fn(workloads.as_numpy_operand(A), workloads.as_numpy_operand(B), rows=rows,
                     threads=cpu_threads())
        e, _, _ = oracle.normalized_error(Cd[rows].cpu().numpy(), Cref, D)
        check[w.name] = float(f"{e:.3e}")

    if not args.no_cpu_baseline:
        cpu = cpu_baseline(ws, host, args.cpu_seconds)

    copy = None
    if args.copy_calibration:
        copy = copy_calibration(dev)

    others = general = sequence = fp8 = attention = mx = None
    if not args.no_configs:
        others = other_configs(dev, set(names), args.check_rows)
        general = general_configs(dev, args.check_rows)
        sequence = sequence_config(dev)
        fp8 = fp8_configs(dev, args.check_rows)
        attention = attention_configs(dev)
        mx = mx_configs(dev)

    dom = max(per.values(), key=lambda r: r["avg_ms"])
    dom_w = next(w for w in ws if per[w.name] is dom)
    roofline = {
        "bound": "mfma", "kernel": dom["kernel"], "workload": dom_w.name,
        "achieved": dom["tflops"], "peak": PEAK_TFLOPS[dom_w.dtype], "unit": "TFLOP/s",
        "frac": dom["frac_peak"], "traffic": traffic_for(dom["kernel"]),
    }
    runs = [{"ms_per_step": ms_per_step, "avg_ms": {n: r["avg_ms"] for n, r in per.items()}}]
    runs += [c for c in children if c is not None]
    spread = {"processes": len(runs), "ms_per_step": spread_of([r["ms_per_step"] for r in runs])}
    for n in per:
        spread[n + "_avg_ms"] = spread_of([r["avg_ms"][n] for r in runs if n in r["avg_ms"]])
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "+".join(sorted({w.dtype for w in ws})),
        "data": "synthetic (seed 1234; fp32 uniform[-1,1], bf16 from N(0,1))",
        "config": {"workload": "+".join(names),
                   "shapes": {w.name: [w.M, w.N, w.K] for w in ws}},
        # each product's own rate: value above is the step's flops over the
        # step's time, which blends the two dtypes
        "headline": {n: {"gflops": round(r["tflops"] * 1e3, 1), "frac_peak": r["frac_peak"],
                         "kernel": r["kernel"], "avg_ms": r["avg_ms"]} for n, r in per.items()},
        # the step timed in separate processes (median, min, max)
        "spread": spread,
        # a do-nothing kernel timed the same way as each product (one launch
        # between two events on the same stream)
        "identity_null_us": null_us,
        "per_kernel": per, "max_norm_err_sampled": check,
        "roofline": roofline,
        "roofline_by_kernel": {n: {"bound": "mfma", "achieved": r["tflops"],
                                   "peak": PEAK_TFLOPS[r["dtype"]], "unit": "TFLOP/s",
                                   "frac": r["frac_peak"]} for n, r in per.items()},
        "cpu_baseline": cpu,
        # every other configuration of the set, the table's kernel, time per
        # call (short calls also from a replayed HIP graph), its roofline and
        # a sampled check against the oracle; context, not `value`
        "other_configs": others,
        # the same for products with a transposed factor or a batch (the GPT
        # backward pass and attention shapes)
        "general_configs": general,
        # a launch-bound sequence (one GPT forward pass over 256 tokens, with
        # the attention unfused and fused): back-to-back calls against the
        # same calls replayed from a HIP graph, every output checked
        "sequence": sequence,
        "fp8": fp8,
        # the fused attention forward on the GPT's shapes, read in place from
        # the QKV projection's output; beside it the same attention unfused
        # (the per-head score and probability x value products above)
        "attention": attention,
        # 8-bit products with MX block scales (one E8M0 scale per 32 elements
        # of K of each row of A and of Bt)
        "mx_fp8": mx,
        # GPU core clock and board power sampled over the timed steps, and
        # the toolchain that built the kernels
        "env": dict(clocks.summary(), toolchain=toolchain(g.gemm_build_info())),
    }
    if copy is not None:
        line["copy_calibration"] = copy
    print(json.dumps(line), flush=True)


LLC_BYTES = 256 * 1024 * 1024   # MI355X last-level (Infinity) cache
CODE = {"f32": 0, "bf16": 1, "f16": 2}   # element type codes of the library


def other_configs(dev, skip, check_rows):
    """The table's kernel on every configuration not in the step, timed as
    back-to-back calls through the binding (median of 5 windows).  Operands
    too small to outgrow the last-level cache rotate through enough copies
    that each call reads from HBM.  Calls under 20 us, whose pace the host
    sets, are also replayed from a HIP graph for the GPU's own time."""
    import dense_gemm_17_amd as g
    import oracle
    out = {}
    rng = np.random.default_rng(1)
    for name, w in workloads.WORKLOADS.items():
        if name in skip:
            continue
        A, B = workloads.make_inputs(w)
        per_copy = w.algorithmic_bytes
        copies = 1 if per_copy * 2 > LLC_BYTES else max(2, -(-2 * LLC_BYTES // per_copy))
        ops = [(A.to(dev), B.to(dev), torch.empty((w.M, w.N), dtype=torch.float32, device=dev))
               for _ in range(copies)]
        code = CODE[w.dtype]
        a0, b0, c0 = ops[0]
        kernel = g.gemm_kernel_name(g.gemm_plan(code, w.M, w.N, w.K, a0.data_ptr(), a0.stride(0),
                                                b0.data_ptr(), b0.stride(0), c0.data_ptr(),
                                                c0.stride(0)))
        state = {"i": 0}

        def call():
            a, b, c = ops[state["i"] % copies]
            state["i"] += 1
            g.gemm(a, b, out=c)

        ms, graph_ms, clocks = time_calls(dev, call, copies)
        rows = sorted(set([0, w.M - 1] + rng.choice(w.M, size=min(w.M, check_rows),
                                                     replace=False).tolist()))
        fn = getattr(oracle, "gemm_" + w.dtype)
        Cref, D = fn(workloads.as_numpy_operand(A), workloads.as_numpy_operand(B), rows=rows,
                     threads=cpu_threads())
        err, _, _ = oracle.normalized_error(c0[rows].cpu().numpy(), Cref, D)
        tflops = w.flops / (ms * 1e-3) / 1e12
        gbs = per_copy / (ms * 1e-3) / 1e9
        ridge = PEAK_TFLOPS[w.dtype] * 1e3 / HBM_PEAK_GBS     # flop per byte
        hbm = w.flops / per_copy < ridge
        out[name] = {
            "M": w.M, "N": w.N, "K": w.K, "dtype": w.dtype, "kernel": kernel,
            "us_per_call": round(ms * 1e3, 2), "tflops": round(tflops, 2), "gbs": round(gbs, 1),
            "bound": "hbm" if hbm else "mfma",
            "frac": round(gbs / HBM_PEAK_GBS if hbm else tflops / PEAK_TFLOPS[w.dtype], 4),
            "us_per_call_graph": round(graph_ms * 1e3, 2) if graph_ms is not None else None,
            "operand_copies": copies, "max_norm_err_sampled": float(f"{err:.3e}"),
            "sclk_mhz": (clocks.summary()["sclk_mhz"] or {}).get("median"),
        }
        del ops
        torch.cuda.empty_cache()
    return out


def time_calls(dev, call, copies):
    """Median time per call (ms) of back-to-back calls on a side stream over 5
    windows of at least ~20 ms; for calls under 20 us also the time of the
    same calls replayed from a HIP graph; and the clock sampler."""
    from dense_gemm_17_amd.measure import ClockSampler
    st = torch.cuda.Stream(dev)
    st.wait_stream(torch.cuda.current_stream(dev))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def windows(run, reps):
        times = []
        for _ in range(5):
            e0.record(st)
            run()
            e1.record(st)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / reps)
        return float(np.median(times))

    graph_ms = None
    with torch.cuda.stream(st):
        for _ in range(copies):
            call()
        e0.record(st)
        call()
        e1.record(st)
        torch.cuda.synchronize()
        one = max(e0.elapsed_time(e1), 1e-3)
        reps = copies * max(1, min(2000 // copies, int(20.0 / one / copies) + 1))
        # back-to-back calls from Python, as an application makes them
        with ClockSampler() as clocks:
            ms = windows(lambda: [call() for _ in range(reps)], reps)
        if ms < 0.02:
            # short calls: the host call sets their pace, so the same
            # calls replayed from a HIP graph give the GPU's own time
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=st):
                for _ in range(reps):
                    call()
            graph.replay()
            torch.cuda.synchronize()
            graph_ms = windows(graph.replay, reps)
            del graph
    return ms, graph_ms, clocks


def sequence_config(dev, windows: int = 5, reps: int = 20):
    """One GPT forward pass over a single sequence of 256 tokens (fp32), the
    launch-bound regime: as 37 library calls with the attention unfused
    (per-head score and probability x value products) and as 31 with the
    fused attention reading the QKV projection's output in place.  Each is
    timed as back-to-back calls through the binding and as the same calls
    captured once into a HIP graph and replayed; after a replay every
    product (and attention) output is checked against the oracle on the
    inputs it read."""
    import dense_gemm_17_amd as g
    import oracle
    from oracle import attention as att
    gen = workloads.generator()
    heads, dh, T = 6, 64, 256

    def operand(shape, sigma):
        return workloads.draw(shape, ("normal", sigma), gen).to(dev)

    def build(fused):
        ops = []     # ("gemm", a, b, c) or ("attn", qkv, o)
        for (name, nb, M, N, K, ta, tb) in workloads.gpt_forward_sequence():
            kind = name.split("_", 1)[1]
            if fused and kind == "pv":
                continue
            if fused and kind == "scores":
                qkv = ops[-1][3]                            # this layer's QKV output
                o = torch.empty((T, heads * dh), dtype=torch.float32, device=dev)
                ops.append(("attn", qkv, o))
                continue
            lead = (nb,) if nb > 1 else ()
            w = 0.02 if kind in ("qkv", "proj", "mlp_up", "mlp_down", "head") else 1.0
            A = operand(lead + ((K, M) if ta else (M, K)), 1.0)
            B = operand(lead + ((N, K) if tb else (K, N)), w)
            C = torch.empty(lead + (M, N), dtype=torch.float32, device=dev)
            ops.append(("gemm", A.transpose(-1, -2) if ta else A,
                        B.transpose(-1, -2) if tb else B, C))
        return ops

    def qkv_views(qkv):
        t = qkv.view(1, T, 3, heads, dh)
        return tuple(t[:, :, i].permute(0, 2, 1, 3) for i in range(3))

    def run(ops):
        for op in ops:
            if op[0] == "gemm":
                g.gemm(op[1], op[2], out=op[3])
            else:
                q, k, v = qkv_views(op[1])
                g.attention(q, k, v, causal=True, scale=dh ** -0.5,
                            out=op[2].view(1, T, heads, dh).permute(0, 2, 1, 3))

    def flops(ops):
        f = 0
        for op in ops:
            if op[0] == "gemm":
                a, b = op[1], op[2]
                nb = a.shape[0] if a.dim() == 3 else 1
                f += 2 * nb * a.shape[-2] * a.shape[-1] * b.shape[-1]
            else:
                f += 4 * heads * (T * (T + 1) // 2) * dh
        return f

    def check(ops):
        worst = 0.0
        for op in ops:
            if op[0] == "gemm":
                a, b, c = op[1].cpu(), op[2].cpu(), op[3].cpu()
                if a.dim() == 2:
                    a, b, c = a[None], b[None], c[None]
                for i in range(a.shape[0]):
                    Cref, D = oracle.gemm_f32(np.ascontiguousarray(a[i].numpy()),
                                              np.ascontiguousarray(b[i].numpy()))
                    worst = max(worst, oracle.normalized_error(c[i].numpy(), Cref, D)[0])
            else:
                q, k, v = (x.cpu().numpy() for x in qkv_views(op[1]))
                Oref, DN, _, _ = att.attention_fwd(q, k, v, True, dh ** -0.5)
                o = op[2].cpu().view(1, T, heads, dh).permute(0, 2, 1, 3).numpy()
                worst = max(worst, att.normalized_error(o, Oref, DN)[0])
        return worst

    st = torch.cuda.Stream(dev)
    st.wait_stream(torch.cuda.current_stream(dev))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        ts = []
        for _ in range(windows):
            e0.record(st)
            for _ in range(reps):
                fn()
            e1.record(st)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / reps)
        return float(np.median(ts))

    out = {}
    for label, fused in (("unfused_attention", False), ("fused_attention", True)):
        ops = build(fused)
        with torch.cuda.stream(st):
            for _ in range(3):
                run(ops)
            torch.cuda.synchronize()
            eager_ms = timed(lambda: run(ops))
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=st):
                run(ops)
            for op in ops:
                op[-1].fill_(float("nan"))
            graph.replay()
            torch.cuda.synchronize()
            err = check(ops)
            graph_ms = timed(graph.replay)
            del graph
        f = flops(ops)
        out[label] = {"calls": len(ops), "gflop": round(f / 1e9, 3),
                      "eager_us": round(eager_ms * 1e3, 1), "graph_us": round(graph_ms * 1e3, 1),
                      "eager_us_per_call": round(eager_ms * 1e3 / len(ops), 2),
                      "graph_us_per_call": round(graph_ms * 1e3 / len(ops), 2),
                      "graph_tflops": round(f / (graph_ms * 1e-3) / 1e12, 2),
                      "max_norm_err_every_output": float(f"{err:.3e}")}
    return out


def general_configs(dev, check_rows):
    """Transposed-factor and batched products (the GPT backward pass and
    attention shapes): the table's kernel timed like the configurations
    above, with sampled rows of the first and last product checked against
    the oracle."""
    import dense_gemm_17_amd as g
    import oracle
    out = {}
    rng = np.random.default_rng(2)
    for name, w in workloads.GENERAL_WORKLOADS.items():
        As, Bs = workloads.make_general_inputs(w)
        per_copy = w.algorithmic_bytes
        copies = 1 if per_copy * 2 > LLC_BYTES else max(2, -(-2 * LLC_BYTES // per_copy))
        shape = (w.batch, w.M, w.N) if w.batch > 1 else (w.M, w.N)
        ops = []
        for _ in range(copies):
            a, b = workloads.general_views(w, As.to(dev), Bs.to(dev))
            ops.append((a, b, torch.empty(shape, dtype=torch.float32, device=dev)))
        state = {"i": 0}

        def call():
            a, b, c = ops[state["i"] % copies]
            state["i"] += 1
            g.gemm(a, b, out=c)

        ms, graph_ms, clocks = time_calls(dev, call, copies)
        kernel = g.gemm_kernel_name(g.gemm_last_kernel())
        c0 = ops[0][2].reshape(w.batch, w.M, w.N)
        err = 0.0
        for bi in sorted({0, w.batch - 1}):
            rows = sorted(set([0, w.M - 1] + rng.choice(w.M, size=min(w.M, check_rows),
                                                         replace=False).tolist()))
            A_b = As[bi] if As.dim() == 3 else As
            B_b = Bs[bi] if Bs.dim() == 3 else Bs
            A_rows = (A_b.t()[rows] if w.ta else A_b[rows]).contiguous()
            Cref, D = oracle.gemm_batched(workloads.as_numpy_operand(A_rows),
                                          workloads.as_numpy_operand(B_b), False, w.tb,
                                          threads=cpu_threads())
            e, _, _ = oracle.normalized_error(c0[bi][rows].cpu().numpy(), Cref, D)
            err = max(err, e)
        tflops = w.flops / (ms * 1e-3) / 1e12
        gbs = per_copy / (ms * 1e-3) / 1e9
        ridge = PEAK_TFLOPS[w.dtype] * 1e3 / HBM_PEAK_GBS
        hbm = w.flops / per_copy < ridge
        ws_rec = None
        ws_bytes = g.gemm_workspace_size(CODE[w.dtype], w.ta, w.tb, w.M, w.N, w.K, w.batch)
        if ws_bytes:
            # the same call with a workspace: K split over work-groups
            wsbuf = torch.empty((ws_bytes // 4,), dtype=torch.float32, device=dev)
            state["i"] = 0

            def call_ws():
                a, b, c = ops[state["i"] % copies]
                state["i"] += 1
                g.gemm(a, b, out=c, workspace=wsbuf)

            ms_ws, _, _ = time_calls(dev, call_ws, copies)
            c0w = ops[0][2].reshape(w.batch, w.M, w.N)
            e_ws = 0.0
            for bi in sorted({0, w.batch - 1}):
                rows = sorted(set([0, w.M - 1] + rng.choice(w.M, size=min(w.M, check_rows),
                                                             replace=False).tolist()))
                A_b = As[bi] if As.dim() == 3 else As
                B_b = Bs[bi] if Bs.dim() == 3 else Bs
                A_rows = (A_b.t()[rows] if w.ta else A_b[rows]).contiguous()
                Cref, D = oracle.gemm_batched(workloads.as_numpy_operand(A_rows),
                                              workloads.as_numpy_operand(B_b), False, w.tb,
                                              threads=cpu_threads())
                e, _, _ = oracle.normalized_error(c0w[bi][rows].cpu().numpy(), Cref, D)
                e_ws = max(e_ws, e)
            tf_ws = w.flops / (ms_ws * 1e-3) / 1e12
            ws_rec = {"workspace_bytes": ws_bytes, "us_per_call": round(ms_ws * 1e3, 2),
                      "tflops": round(tf_ws, 2), "frac": round(tf_ws / PEAK_TFLOPS[w.dtype], 4),
                      "partials_kernel": g.gemm_kernel_name(g.gemm_last_kernel()),
                      "max_norm_err_sampled": float(f"{e_ws:.3e}")}
            del wsbuf
        out[name] = {
            "batch": w.batch, "M": w.M, "N": w.N, "K": w.K, "transa": w.ta, "transb": w.tb,
            "dtype": w.dtype, "kernel": kernel,
            "us_per_call": round(ms * 1e3, 2), "tflops": round(tflops, 2), "gbs": round(gbs, 1),
            "bound": "hbm" if hbm else "mfma",
            "frac": round(gbs / HBM_PEAK_GBS if hbm else tflops / PEAK_TFLOPS[w.dtype], 4),
            "us_per_call_graph": round(graph_ms * 1e3, 2) if graph_ms is not None else None,
            "operand_copies": copies, "max_norm_err_sampled": float(f"{err:.3e}"),
            "sclk_mhz": (clocks.summary()["sclk_mhz"] or {}).get("median"),
            "with_workspace": ws_rec,
        }
        del ops
        torch.cuda.empty_cache()
    return out


def fp8_configs(dev, check_rows):
    """8-bit float products (e4m3 / e5m2, B given transposed): the table's
    kernel timed like the configurations above, sampled rows checked against
    the oracle."""
    import dense_gemm_17_amd as g
    import oracle
    out = {}
    rng = np.random.default_rng(4)
    for name, w in workloads.FP8_WORKLOADS.items():
        A, Bt = workloads.make_fp8_inputs(w)
        per_copy = w.algorithmic_bytes
        copies = 1 if per_copy * 2 > LLC_BYTES else max(2, -(-2 * LLC_BYTES // per_copy))
        ops = [(A.to(dev), Bt.to(dev).t(), torch.empty((w.M, w.N), dtype=torch.float32,
                                                       device=dev)) for _ in range(copies)]
        state = {"i": 0}

        def call():
            a, b, c = ops[state["i"] % copies]
            state["i"] += 1
            g.gemm(a, b, out=c)

        ms, graph_ms, clocks = time_calls(dev, call, copies)
        kernel = g.gemm_kernel_name(g.gemm_last_kernel())
        rows = sorted(set([0, w.M - 1] + rng.choice(w.M, size=min(w.M, check_rows),
                                                     replace=False).tolist()))
        Cref, D = oracle.gemm_fp8_batched(workloads.fp8_bits(A[rows]), workloads.fp8_bits(Bt),
                                          w.fa, w.fb, False, True, threads=cpu_threads())
        err, _, _ = oracle.normalized_error(ops[0][2][rows].cpu().numpy(), Cref, D)
        tflops = w.flops / (ms * 1e-3) / 1e12
        gbs = per_copy / (ms * 1e-3) / 1e9
        hbm = w.flops / per_copy < PEAK_TFLOPS["fp8"] * 1e3 / HBM_PEAK_GBS
        out[name] = {
            "M": w.M, "N": w.N, "K": w.K, "formats": ["e4m3", "e5m2"][w.fa] + "x" +
            ["e4m3", "e5m2"][w.fb], "kernel": kernel,
            "us_per_call": round(ms * 1e3, 2), "tflops": round(tflops, 2), "gbs": round(gbs, 1),
            "bound": "hbm" if hbm else "mfma",
            "frac": round(gbs / HBM_PEAK_GBS if hbm else tflops / PEAK_TFLOPS["fp8"], 4),
            "us_per_call_graph": round(graph_ms * 1e3, 2) if graph_ms is not None else None,
            "operand_copies": copies, "max_norm_err_sampled": float(f"{err:.3e}"),
            "sclk_mhz": (clocks.summary()["sclk_mhz"] or {}).get("median"),
        }
        del ops
        torch.cuda.empty_cache()
    return out


def spread_of(xs):
    xs = sorted(float(x) for x in xs)
    if not xs:
        return None
    return {"median": round(float(np.median(xs)), 4), "min": round(xs[0], 4),
            "max": round(xs[-1], 4), "n": len(xs)}


def child_run(args):
    """Time the step in a process of its own (started as a child, never by
    replacing this one); returns its per-step and per-product times, or None
    if it failed."""
    import subprocess
    cmd = [sys.executable, os.path.abspath(__file__), "--child", "--steps", str(args.steps),
           "--warmup", str(args.warmup), "--workloads", args.workloads, "--no-cpu-baseline",
           "--no-configs", "--check-rows", "1"]
    try:
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    except subprocess.TimeoutExpired:
        return None
    if r.returncode != 0:
        print(f"bench child run failed ({r.returncode}): {r.stderr[-400:]}", file=sys.stderr)
        return None
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    return json.loads(lines[-1]) if lines else None


def identity_null(dev, reps):
    """Microseconds per launch of a kernel that does nothing, timed like
    the products: one launch between two events on the current stream,
    averaged over `reps` launches."""
    import dense_gemm_17_amd as g
    stream = torch.cuda.current_stream(dev)
    for _ in range(10):
        g.gemm_null_launch(stream.cuda_stream)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for e0, e1 in evs:
        e0.record(stream)
        rc = g.gemm_null_launch(stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"gemm_null_launch failed: {rc}")
        e1.record(stream)
    torch.cuda.synchronize()
    return round(float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3, 2)


def cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


MX_WORKLOADS = {"mx_e4m3_8192": (8192, 8192, 8192), "mx_gpt_qkv": (16384, 1152, 384),
                "mx_skinny_4x8192x8192": (4, 8192, 8192)}


def mx_configs(dev, check_rows=4):
    """8-bit e4m3 products with MX block scales drawn in [2^-7, 2^7]: the
    table's kernel timed like the configurations above, sampled rows checked
    against the oracle."""
    import dense_gemm_17_amd as g
    import oracle
    out = {}
    rng = np.random.default_rng(5)
    for name, (M, N, K) in MX_WORKLOADS.items():
        gen = workloads.generator()
        A = workloads.draw((M, K), ("normal", 1.0), gen).to(torch.float8_e4m3fn)
        Bt = workloads.draw((N, K), ("normal", 1.0), gen).to(torch.float8_e4m3fn)
        SA = torch.randint(120, 135, (K // 32, -(-M // 4) * 4), generator=gen).to(torch.uint8)
        SB = torch.randint(120, 135, (K // 32, -(-N // 4) * 4), generator=gen).to(torch.uint8)
        per_copy = M * K + N * K + 4 * M * N + (K // 32) * (M + N)
        copies = 1 if per_copy * 2 > LLC_BYTES else max(2, -(-2 * LLC_BYTES // per_copy))
        ops = [(A.to(dev), SA.to(dev), Bt.to(dev).t(), SB.to(dev),
                torch.empty((M, N), dtype=torch.float32, device=dev)) for _ in range(copies)]
        state = {"i": 0}

        def call():
            a, sa, b, sb, c = ops[state["i"] % copies]
            state["i"] += 1
            g.gemm_mx(a, sa, b, sb, out=c)

        ms, graph_ms, clocks = time_calls(dev, call, copies)
        kernel = g.gemm_kernel_name(g.gemm_last_kernel())
        rows = sorted(set([0, M - 1] + rng.choice(M, size=min(M, check_rows), replace=False).tolist()))
        Cref, D = oracle.gemm_mxfp8(workloads.fp8_bits(A[rows]), SA[:, rows].numpy(),
                                    workloads.fp8_bits(Bt), SB.numpy(), 0, 0, threads=cpu_threads())
        err, _, _ = oracle.normalized_error(ops[0][4][rows].cpu().numpy(), Cref, D)
        flops = 2 * M * N * K
        tflops = flops / (ms * 1e-3) / 1e12
        gbs = per_copy / (ms * 1e-3) / 1e9
        hbm = flops / per_copy < PEAK_TFLOPS["fp8"] * 1e3 / HBM_PEAK_GBS
        out[name] = {
            "M": M, "N": N, "K": K, "formats": "e4m3xe4m3, E8M0 scales per 32", "kernel": kernel,
            "us_per_call": round(ms * 1e3, 2), "tflops": round(tflops, 2), "gbs": round(gbs, 1),
            "bound": "hbm" if hbm else "mfma",
            "frac": round(gbs / HBM_PEAK_GBS if hbm else tflops / PEAK_TFLOPS["fp8"], 4),
            "us_per_call_graph": round(graph_ms * 1e3, 2) if graph_ms is not None else None,
            "operand_copies": copies, "max_norm_err_sampled": float(f"{err:.3e}"),
            "sclk_mhz": (clocks.summary()["sclk_mhz"] or {}).get("median"),
        }
        del ops
        torch.cuda.empty_cache()
    return out


def attention_configs(dev):
    """The fused attention forward on each attention workload: Q, K, V read
    in place from a QKV projection buffer, O written token-major, timed like
    the configurations above; the first sequence's heads checked against
    the oracle."""
    import dense_gemm_17_amd as g
    from oracle import attention as att
    out = {}
    for name, w in workloads.ATTENTION_WORKLOADS.items():
        qkv = workloads.make_attention_qkv(w)
        per_copy = w.algorithmic_bytes
        copies = 1 if per_copy * 2 > LLC_BYTES else max(2, -(-2 * LLC_BYTES // per_copy))
        ops = []
        for _ in range(copies):
            qd = qkv.to(dev)
            o = torch.empty((w.B * w.S, w.H * w.D), dtype=torch.float32, device=dev)
            lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
            ops.append((workloads.attention_views(w, qd),
                        o.view(w.B, w.S, w.H, w.D).permute(0, 2, 1, 3), lse))
        state = {"i": 0}

        def call():
            (q, k, v), o, lse = ops[state["i"] % copies]
            state["i"] += 1
            g.attention(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)

        ms, graph_ms, clocks = time_calls(dev, call, copies)
        Q, K, V = workloads.attention_views(w, qkv)
        Oref, DN, _, _ = att.attention_fwd(Q[:1].numpy(), K[:1].numpy(), V[:1].numpy(),
                                           w.causal, w.scale)
        err, _ = att.normalized_error(ops[0][1][:1].cpu().numpy(), Oref, DN)
        tflops = w.flops / (ms * 1e-3) / 1e12
        out[name] = {
            "B": w.B, "H": w.H, "S": w.S, "D": w.D, "causal": w.causal,
            "kernel": f"attention_fwd_kernel<{w.D}>", "us_per_call": round(ms * 1e3, 2),
            "tflops": round(tflops, 2), "bound": "mfma",
            "frac": round(tflops / PEAK_TFLOPS["f32"], 4),
            "gbs": round(per_copy / (ms * 1e-3) / 1e9, 1),
            "us_per_call_graph": round(graph_ms * 1e3, 2) if graph_ms is not None else None,
            "operand_copies": copies, "max_norm_err_first_sequence": float(f"{err:.3e}"),
            "sclk_mhz": (clocks.summary()["sclk_mhz"] or {}).get("median"),
        }
        del ops
        torch.cuda.empty_cache()
    return out


def cpu_baseline(ws, host, seconds):
    """The oracle, as it stands, on a bounded sample: the first R rows of each
    product of the step, R sized from a short calibration run."""
    import oracle
    th = cpu_threads()
    probe_rows = max(1, th)
    t0 = time.perf_counter()
    for w in ws:
        A, B = host[w.name]
        fn = getattr(oracle, "gemm_" + w.dtype)
        fn(workloads.as_numpy_operand(A), workloads.as_numpy_operand(B),
           rows=list(range(min(probe_rows, w.M))), threads=th)
    t_probe = time.perf_counter() - t0
    rows = max(probe_rows, int(probe_rows * seconds / max(t_probe, 1e-3)) // th * th)
    flops = 0
    t0 = time.perf_counter()
    for w in ws:
        A, B = host[w.name]
        r = min(rows, w.M)
        fn = getattr(oracle, "gemm_" + w.dtype)
        fn(workloads.as_numpy_operand(A), workloads.as_numpy_operand(B),
           rows=list(range(r)), threads=th)
        flops += 2 * r * w.N * w.K
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e9, 3), "unit": "GFLOP/s", "cores": th,
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"first {rows} rows of each product of the step "
                      f"({flops / 1e9:.1f} GFLOP in {dt:.1f} s, fp64 accumulation)"}


def copy_calibration(dev):
    """A plain device-to-device copy of 256 MiB, timed, for counter scaling."""
    n = 64 * 1024 * 1024
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"bytes_read": 4 * n, "bytes_written": 4 * n, "launches": 3}


if __name__ == "__main__":
    main()
