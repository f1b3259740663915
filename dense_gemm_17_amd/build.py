"""Build libmi355gemm.so in-tree with hipcc for gfx950.

Every HIP source under csrc/ is compiled to an object (in parallel), then the
objects are linked into ``dense_gemm_17_amd/libmi355gemm.so``.  The compiler's
per-kernel resource remarks (VGPR/AGPR/SGPR counts, scratch, LDS, occupancy)
are kept in ``_build/resources.txt`` for the resource-budget test.

Usage:  python dense_gemm_17_amd/build.py   (run by path: importing the package
        needs the library this script builds)
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmi355gemm.so")
ROOT = os.path.dirname(HERE)

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 VALU ops are switched off for every HIP file: only scalar fp32
# FMAs and the matrix cores do fp32 arithmetic here.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wextra", "-Wno-unused-parameter",
    "-I", os.path.join(ROOT, "include"),
]
REMARKS = ["-Rpass-analysis=kernel-resource-usage"]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def _compile(src: str) -> tuple:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *HIP_FLAGS, *REMARKS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj, r.stderr


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link the shared library; returns its
    path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", "8"))))
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, srcs))
    with open(os.path.join(BUILD, "resources.txt"), "w") as f:
        for _, remarks in results:
            f.write(remarks)
    _link([o for o, _ in results], LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


# Host-side sanitizers for the C-ABI layer (argument validation, extents,
# overlap and dispatch arithmetic): only api.hip's host code is
# instrumented; device code is built as usual.
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-shared-libsan",
             "-Xarch_host", "-fno-omit-frame-pointer"]


def build_sanitized_host(out: str) -> str:
    """Link a copy of the library whose api.hip host code is built with
    AddressSanitizer and UndefinedBehaviorSanitizer, from the objects of the
    last build() for the other sources.  Load it with the ASan runtime
    preloaded (``asan_runtime()``) and MI355GEMM_LIBRARY pointing at it."""
    san_dir = os.path.join(BUILD, "san")
    os.makedirs(san_dir, exist_ok=True)
    api = os.path.join(CSRC, "api.hip")
    obj = os.path.join(san_dir, "api.o")
    r = subprocess.run([HIPCC, *HIP_FLAGS, *SAN_FLAGS, "-c", api, "-o", obj],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {api}:\n{r.stderr}")
    others = [os.path.join(BUILD, os.path.basename(src)[:-4] + ".o") for src in sources()
              if os.path.basename(src) != "api.hip"]
    missing = [o for o in others if not os.path.exists(o)]
    if missing:
        raise FileNotFoundError(f"build() first: missing {missing}")
    tmp = out + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *SAN_FLAGS, obj,
                        *others, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


def asan_runtime() -> str:
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True, check=True)
    return r.stdout.strip()


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
