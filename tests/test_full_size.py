"""Whole-output parity at the headline size, 8192 x 8192 x 8192.

The other parity tests compare sampled rows at this size; here every one of
the 67M outputs is compared with the full CPU oracle, in the launch
configuration the benchmark times (the table's kernel through the plain
entry points, 1024 tiles of 256 x 256 over all eight XCDs, so the XCD remap
and the grouped tile order are checked on every tile).

Small-integer operands make the check exact: fp32 entries in [-4, 4] and
16- and 8-bit entries in [-8, 8] keep every partial sum an integer below
2^24 (at most 64 * 8192 = 2^19 in magnitude), so any summation order gives
the exact integer, and the kernel's output must equal the oracle's bit for
bit.  The two products the benchmark times are also checked on their own
random operands against the 5e-4 gate on every element.

Each full oracle pass is ~1.1e12 fp64 flops: about half a minute on 16 cores.
"""
import sys

import numpy as np
import pytest
import torch

import dense_gemm_17_amd as g
import oracle
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
S = 8192


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _compare_exact(name, C, Cref):
    Ch = C.cpu().numpy().astype(np.float64)
    bad = np.argwhere(Ch != Cref)
    say(f"[full] {name} kernel={g.gemm_kernel_name(g.gemm_last_kernel())} "
        f"mismatches={len(bad)}")
    assert len(bad) == 0, f"{len(bad)} outputs differ, first at {tuple(bad[0])}: " \
                          f"{Ch[tuple(bad[0])]} vs {Cref[tuple(bad[0])]}"


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_8192_small_integers_whole_output(dtype):
    gen = workloads.generator(8192)
    lim = 4 if dtype == "f32" else 8
    tdt = workloads.TORCH_DTYPE[dtype]
    A = workloads.small_int((S, S), -lim, lim, gen, tdt)
    B = workloads.small_int((S, S), -lim, lim, gen, tdt)
    say(f"[full] {dtype} 8192^3 small integers: oracle")
    fn = {"f32": oracle.gemm_f32, "bf16": oracle.gemm_bf16, "f16": oracle.gemm_f16}[dtype]
    Cref, _ = fn(workloads.as_numpy_operand(A), workloads.as_numpy_operand(B))
    say(f"[full] {dtype} 8192^3 small integers: GPU")
    C = g.gemm(A.to(DEV), B.to(DEV))
    torch.cuda.synchronize()
    _compare_exact(f"{dtype}_8192_int", C, Cref)


def test_8192_fp8_small_integers_whole_output():
    # e4m3 activations times an e5m2 weight stored N x K (the layout the
    # 8-bit entry points take); integers up to 8 are exact in both formats
    gen = workloads.generator(8193)
    A = workloads.small_int((S, S), -8, 8, gen).to(torch.float8_e4m3fn)
    Wt = workloads.small_int((S, S), -8, 8, gen).to(torch.float8_e5m2)
    say("[full] fp8 8192^3 small integers: oracle")
    Cref, _ = oracle.gemm_fp8_batched(workloads.fp8_bits(A), workloads.fp8_bits(Wt), 0, 1,
                                      False, True)
    say("[full] fp8 8192^3 small integers: GPU")
    C = g.gemm(A.to(DEV), Wt.to(DEV).t())
    torch.cuda.synchronize()
    _compare_exact("fp8_8192_int", C, Cref)


@pytest.mark.parametrize("name", ["f32_8192", "bf16_8192"])
def test_8192_benchmark_operands_whole_output(name):
    w = workloads.WORKLOADS[name]
    A, B = workloads.make_inputs(w)
    say(f"[full] {name}: oracle")
    fn = {"f32": oracle.gemm_f32, "bf16": oracle.gemm_bf16}[w.dtype]
    Cref, D = fn(workloads.as_numpy_operand(A), workloads.as_numpy_operand(B))
    say(f"[full] {name}: GPU")
    C = g.gemm(A.to(DEV), B.to(DEV))
    torch.cuda.synchronize()
    e, at, n = oracle.normalized_error(C.cpu().numpy(), Cref, D)
    say(f"[full] {name} kernel={g.gemm_kernel_name(g.gemm_last_kernel())} e={e:.3e} at={at} "
        f"n>1e-5={n}")
    assert e <= oracle.GATE, f"normalized error {e} at {at}"
