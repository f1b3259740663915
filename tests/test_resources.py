"""Resource budget of every kernel, read from the compiler's own remarks.

"Bare Metal Bard" (page 1, fourth paragraph) describes a compiler upgrade
that spent extra registers to remove a small spill, crossed an occupancy
cliff and cost a fifth of the throughput while every correctness test kept
passing.  These checks make such a change fail loudly: no kernel may use
scratch memory or spill vector registers, and each family keeps the
occupancy (waves per SIMD) its design assumes.  The numbers come from
`-Rpass-analysis=kernel-resource-usage`, recorded by the build in
dense_gemm_17_amd/_build/resources.txt (built here if missing).
"""
import importlib.util
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RESOURCES = os.path.join(ROOT, "dense_gemm_17_amd", "_build", "resources.txt")

# family (substring of the mangled name) -> minimum waves per SIMD
OCCUPANCY_BUDGET = {
    "mfma_f32_kernelILi256ELi256E": 1,
    "mfma_f32_kernelILi128ELi128E": 2,
    "mfma_bf16_kernel": 1,
    "mfma_bf16_d16_kernel": 1,
    "mfma_bf16_direct_kernelILi128ELi128E": 2,
    "mfma_fp8_direct_kernelILi128ELi128E": 2,
    "mfma_fp8_direct_kernelILi256ELi128E": 1,
    "mfma_f32_direct_kernelILi256ELi256E": 1,
    "mfma_f32_direct_kernelILi128ELi128E": 2,
    "mfma_f32_direct_kernelILi128ELi64E": 3,
    "mfma_f32_direct_kernelILi64ELi64E": 5,
    "mfma_f32_splitk_kernel": 2,
    "3f3214batched_kernelILi256ELi256E": 1,
    "3f3214batched_kernelILi128ELi128E": 2,
    "2bf14batched_kernelILi256ELi256E": 1,
    "2bf14batched_kernelILi128ELi128E": 2,
    "2sk10f32_kernel": 2,
    "valu_f32_kernel": 3,
    "skinny_kernel": 1,
    "skinny_ksplit_kernel": 2,
    "skinny_fp8_kernel": 2,
    "naive_kernel": 8,
}


def parse():
    if not os.path.exists(RESOURCES):
        spec = importlib.util.spec_from_file_location(
            "_b", os.path.join(ROOT, "dense_gemm_17_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    kernels, cur = {}, None
    for line in open(RESOURCES):
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z \[\]/]+?):\s+(\S+)\s+\[-Rpass", line)
        if m and cur:
            kernels[cur][m.group(1).strip()] = m.group(2)
    return kernels


@pytest.fixture(scope="module")
def kernels():
    k = parse()
    assert k, "no kernel resource remarks found"
    return k


def test_no_scratch_and_no_vgpr_spills(kernels):
    for name, r in kernels.items():
        assert r.get("ScratchSize [bytes/lane]") == "0", (name, r)
        assert r.get("VGPRs Spill") == "0", (name, r)


def test_occupancy_budget(kernels):
    seen = set()
    for name, r in kernels.items():
        for fam, waves in OCCUPANCY_BUDGET.items():
            if fam in name:
                seen.add(fam)
                assert int(r["Occupancy [waves/SIMD]"]) >= waves, (name, r)
    assert seen == set(OCCUPANCY_BUDGET), f"families missing from the build: {set(OCCUPANCY_BUDGET) - seen}"


def test_matrix_core_accumulators_live_in_agprs(kernels):
    # the 256 x 256 tiles keep all 256 accumulators per lane in AGPRs
    big = ("mfma_f32_kernelILi256ELi256E", "mfma_f32_direct_kernelILi256ELi256E",
           "mfma_bf16_kernel", "mfma_bf16_d16_kernel",
           "3f3214batched_kernelILi256ELi256E", "2bf14batched_kernelILi256ELi256E")
    seen = 0
    for name, r in kernels.items():
        if any(f in name for f in big):
            seen += 1
            assert int(r["AGPRs"]) == 256, (name, r)
    assert seen >= 4


def test_lds_within_gfx950_limit(kernels):
    for name, r in kernels.items():
        assert int(r["LDS Size [bytes/block]"]) <= 160 * 1024, (name, r)
