#!/usr/bin/env python3
"""Summarize rocprofv3 counter runs of the sweep into one table per kernel.

Each directory given is one `rocprofv3 --pmc ... -d DIR -o pmc
--output-format csv -- python3 dense_gemm_17_amd/sweep.py --workloads W
--table-only --no-null ...` run, named `<workload>__<pass>`.  For the library's
dispatches in it (the table's kernel on workload W) the counters are
averaged per dispatch and turned into:

  * MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES summed over the 1024 SIMDs, over
    GRBM_GUI_ACTIVE summed over the 8 XCDs (both per dispatch), i.e. the
    fraction of the dispatch's cycles each SIMD's matrix core was busy;
  * VALU issue rate: SQ_INSTS_VALU per SIMD over the dispatch's cycles per
    XCD.  A loop of nothing but scalar fp32 FMAs reaches 90% of the 157.3
    TFLOP/s vector peak on gfx950 (profiles/mfma_ceiling.md), i.e. a wave64
    FMA issues in about two cycles, so such a loop sits near 0.45-0.5;
  * LDS bank-conflict cycles per LDS instruction;
  * HBM bytes fetched per dispatch: FETCH_SIZE (KiB) x 1024 x the copy
    calibration factor of profiles/hbm_traffic_8192.txt (a plain 256 MiB
    device copy reads back as half its bytes on this counter);
  * register use and occupancy from the compiler's remarks
    (dense_gemm_17_amd/_build/resources.txt).

Usage: python dense_gemm_17_amd/counters.py DIR [DIR ...]  (markdown to stdout)
"""
from __future__ import annotations

import collections
import csv
import json
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SIMDS, XCDS = 1024, 8


def fetch_scale() -> float:
    path = os.path.join(ROOT, "profiles", "hbm_traffic_8192.txt")
    try:
        text = "".join(l for l in open(path) if not l.startswith("#"))
        return float(json.loads(text)["fetch_scale"])
    except (OSError, ValueError, KeyError):
        return 2.0


def resources():
    """{demangled kernel (short form): compiler remarks} from the build."""
    raw, cur = {}, None
    path = os.path.join(HERE, "_build", "resources.txt")
    if not os.path.exists(path):
        return {}
    for line in open(path):
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            raw[cur] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z \[\]/]+?):\s+(\S+)\s+\[-Rpass", line)
        if m and cur:
            raw[cur][m.group(1).strip()] = m.group(2)
    names = list(raw)
    try:
        out = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True,
                             text=True, timeout=60).stdout.splitlines()
    except (OSError, subprocess.SubprocessError):
        return {}
    return {short(d): raw[m] for m, d in zip(names, out)}


def short(name: str) -> str:
    """mi355gemm::(anonymous namespace)::foo_kernel<...>(args) -> foo_kernel<...>"""
    name = name.split("(anonymous namespace)::")[-1]
    depth, end = 0, len(name)
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            end = i
            break
    return name[:end].replace("void ", "")


def read_dir(d: str):
    """{kernel: {counter: mean per dispatch}} for the library's dispatches."""
    path = os.path.join(d, "pmc_counter_collection.csv")
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    for r in csv.DictReader(open(path)):
        if "mi355gemm" not in r["Kernel_Name"]:
            continue
        per[(short(r["Kernel_Name"]), r["Dispatch_Id"])][r["Counter_Name"]] += float(r["Counter_Value"])
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for (k, _), cs in per.items():
        for c, v in cs.items():
            agg[k][c].append(v)
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} | {"_dispatches": len(next(iter(cs.values())))}
            for k, cs in agg.items()}


def main(dirs):
    scale = fetch_scale()
    res = resources()
    rows = collections.defaultdict(dict)
    for d in dirs:
        base = os.path.basename(os.path.normpath(d))
        workload = base.split("__")[0]
        for k, cs in read_dir(d).items():
            rows[(workload, k)].update({c: v for c, v in cs.items() if c != "_dispatches"})
            rows[(workload, k)]["_dispatches"] = max(cs["_dispatches"],
                                                     rows[(workload, k)].get("_dispatches", 0))
    print("| Workload | Kernel | Dispatches | MFMA busy | VALU instr / SIMD / cycle | LDS conflict cycles / LDS instr "
          "| HBM fetch per dispatch (MB) | VGPR | AGPR | waves/SIMD |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    for (w, k), cs in sorted(rows.items()):
        grbm = cs.get("GRBM_GUI_ACTIVE")
        mfma = cs.get("SQ_VALU_MFMA_BUSY_CYCLES")
        busy = f"{100 * (mfma / SIMDS) / (grbm / XCDS):.1f}%" if mfma is not None and grbm else ""
        valu = cs.get("SQ_INSTS_VALU")
        vbusy = f"{(valu / SIMDS) / (grbm / XCDS):.3f}" if valu is not None and grbm else ""
        lds = cs.get("SQ_INSTS_LDS")
        conf = cs.get("SQ_LDS_BANK_CONFLICT")
        ldsr = f"{conf / lds:.3f}" if lds and conf is not None else ""
        fetch = cs.get("FETCH_SIZE")
        fmb = f"{fetch * 1024 * scale / 1e6:.1f}" if fetch is not None else ""
        r = res.get(k, {})
        print(f"| {w} | `{k}` | {cs['_dispatches']} | {busy} | {vbusy} | {ldsr} | {fmb} | "
              f"{r.get('VGPRs', '')} | {r.get('AGPRs', '')} | {r.get('Occupancy [waves/SIMD]', '')} |")


if __name__ == "__main__":
    if len(sys.argv) < 2:
        sys.exit(__doc__)
    main(sys.argv[1:])
