"""The dispatch table's choices against measurement (GPU).

The table picks a kernel from a cost model whose efficiencies were measured
on one board (the devpost write-up, "What we built": classify the shape,
then route it through a fixed table).  Its golden tests pin the choices;
this test re-checks the reason for them: on the benchmark's shapes and a
few around the tile boundaries, every kernel that takes the shape is timed
and the table's kernel must be within TOL of the fastest.  A kernel change
that makes the table pick a clearly slower tile fails here.  Operands stay
resident (the same pair every call); each time is the median of five
windows of back-to-back calls.
"""
import sys

import pytest
import torch

import dense_gemm_17_amd as g
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 1.3
TDT = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": workloads.FP8_TORCH[0]}

# (dtype, M, N, K, A stored transposed)
SHAPES = [
    ("f32", 256, 256, 256, False), ("f32", 4096, 4096, 4096, False),
    ("f32", 16384, 1152, 384, False), ("f32", 16384, 1536, 384, False),
    ("f32", 16384, 384, 1536, False), ("f32", 1000, 3000, 777, False),
    ("f32", 4097, 4095, 1023, False), ("f32", 640, 640, 2048, False),
    ("f32", 1024, 1024, 4096, False), ("f32", 384, 1152, 16384, True),
    ("f32", 512, 512, 8192, False), ("f32", 768, 768, 4096, False), ("f32", 384, 1152, 1024, True),
    ("f32", 1024, 1024, 1024, False),
    ("bf16", 16384, 1152, 384, False), ("bf16", 16384, 384, 1536, False),
    ("bf16", 2048, 2048, 8192, False), ("bf16", 384, 1152, 16384, True),
    # 8-bit floats: B is always the transposed view of a row-major (N, K) tensor
    ("fp8", 8192, 8192, 8192, False), ("fp8", 4096, 4096, 4096, False),
    ("fp8", 2048, 2048, 8192, False), ("fp8", 2048, 2048, 2048, False),
    ("fp8", 16384, 1152, 384, False), ("fp8", 16384, 384, 1536, False),
    # few rows: the bandwidth kernels
    ("f32", 7, 4096, 4096, False), ("f32", 4, 4096, 4096, False),
    ("fp8", 16, 8192, 8192, False), ("fp8", 4, 8192, 8192, False), ("fp8", 12, 4096, 2048, False),
]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def timed_us(a, b, c, reps):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(5):
        e0.record()
        for _ in range(reps):
            g.gemm(a, b, out=c)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / reps * 1e3)
    ts.sort()
    return ts[2]


@pytest.mark.parametrize("dtype,M,N,K,ta", SHAPES)
def test_table_choice_is_near_the_fastest(dtype, M, N, K, ta):
    gen = workloads.generator(71)
    A = torch.randn((K, M) if ta else (M, K), generator=gen).to(TDT[dtype]).to(DEV)
    if dtype == "fp8":
        B = torch.randn((N, K), generator=gen).to(TDT[dtype]).to(DEV).t()
    else:
        B = torch.randn((K, N), generator=gen).to(TDT[dtype]).to(DEV)
    a = A.t() if ta else A
    C = torch.empty((M, N), device=DEV)
    g.gemm(a, B, out=C)
    torch.cuda.synchronize()
    table = g.gemm_kernel_name(g.gemm_last_kernel())
    reps = max(3, min(50, int(2e10 / (2 * M * N * K))))
    code = {"f32": g.F32, "bf16": g.BF16, "fp8": g.FP8}[dtype]
    times = {}
    for name in g.kernel_names():
        if g.gemm_kernel_dtype(g.kernel_id(name)) != code or name.startswith("naive"):
            continue
        assert g.gemm_force_kernel(g.kernel_id(name)) == 0
        try:
            try:
                g.gemm(a, B, out=C)
                torch.cuda.synchronize()
            except g.GemmError:
                continue
            if g.gemm_last_kernel() != g.kernel_id(name):
                continue
            times[name] = timed_us(a, B, C, reps)
        finally:
            g.gemm_force_kernel(-1)
    best = min(times, key=times.get)
    say(f"[table] {dtype} {M}x{N}x{K}{' A^T' if ta else ''}: table {table} {times[table]:.1f} us, "
        f"fastest {best} {times[best]:.1f} us over {len(times)} kernels")
    assert times[table] <= TOL * times[best], (table, times[table], best, times[best])
