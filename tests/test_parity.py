"""GPU parity: every kernel of the library against the CPU oracle.

The gate is the normalized error max_ij |c - C| / sum_k |a_ik b_kj| <= 5e-4
for both element types.  Because that gate is loose (at K = 8192 it sits
just above the worst-case bound of any fp32 summation order), the kernels are
also held to exact results where exactness is available: small-integer
operands (every partial sum is an integer below 2^24, so any order is exact),
identity and permutation operands.  Each kernel is forced through the
library's test hook, so every family is checked on every shape it can take,
and the table's own choice is checked in the launch configuration the
benchmark times.  Calls go through the C-ABI (the Python binding only passes
pointers).
"""
import os
import sys

import numpy as np
import pytest
import torch

import dense_gemm_17_amd as g
import oracle
import workloads
from workloads import WORKLOADS, Workload

pytestmark = pytest.mark.gpu
GATE = oracle.GATE
DEV = "cuda:0"

# Full oracle below this many multiply-adds; sampled rows above it.
FULL_ORACLE_LIMIT = 2.0e10
SAMPLE_ROWS = 48


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


CODE = {"f32": g.F32, "bf16": g.BF16, "f16": g.F16}
TDT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
CODE_OF_TORCH = {torch.float32: g.F32, torch.bfloat16: g.BF16, torch.float16: g.F16}
ORACLE_FN = {"f32": oracle.gemm_f32, "bf16": oracle.gemm_bf16, "f16": oracle.gemm_f16}
DTYPES = ["f32", "bf16", "f16"]


def kernels_for(dtype):
    code = CODE[dtype]
    return [n for n in g.kernel_names() if g.gemm_kernel_dtype(g.kernel_id(n)) == code]


FAKE_C = 3 << 40   # stand-in output address for plan queries (256-byte aligned)


def _ld(t):
    return t.stride(0) if t.shape[0] > 1 and t.shape[1] > 0 else max(t.shape[1], 1)


def takes(name, A, B):
    """Does the library accept kernel `name` for these operands (device or
    host tensors of the call's shape, strides and alignment)?"""
    M, K = A.shape
    N = B.shape[1]
    dt = CODE_OF_TORCH[A.dtype]
    kid = g.kernel_id(name)
    with Forced(name):
        got = g.gemm_plan(dt, M, N, K, A.data_ptr() or (1 << 40), _ld(A),
                          B.data_ptr() or (2 << 40), _ld(B), FAKE_C, N)
    return got == kid


class Forced:
    def __init__(self, name):
        self.kid = g.kernel_id(name) if name else -1

    def __enter__(self):
        assert g.gemm_force_kernel(self.kid) == 0

    def __exit__(self, *exc):
        g.gemm_force_kernel(-1)


def run(A, B, kernel=None, out=None):
    with Forced(kernel):
        C = g.gemm(A, B, out=out)
    torch.cuda.synchronize()
    if kernel:
        assert g.gemm_last_kernel() == g.kernel_id(kernel)
    return C


# ---------------------------------------------------------------- oracle cache
_cache = {}


def sample_rows(M, seed=0):
    r = np.random.default_rng(seed)
    fixed = [0, 1, M - 1, M // 2]
    for t in (31, 32, 63, 64, 127, 128, 255, 256):
        fixed += [t, M - 1 - t]
    rnd = r.choice(M, size=min(M, SAMPLE_ROWS), replace=False).tolist()
    return sorted({x for x in fixed + rnd if 0 <= x < M})


def reference(w: Workload):
    """(A, B) on the CPU, rows checked and (C_ref, D) for those rows."""
    if w.name not in _cache:
        A, B = workloads.make_inputs(w)
        An, Bn = workloads.as_numpy_operand(A), workloads.as_numpy_operand(B)
        fn = ORACLE_FN[w.dtype]
        if w.M * w.N * w.K <= FULL_ORACLE_LIMIT:
            rows = None
            C, D = fn(An, Bn)
        else:
            rows = sample_rows(w.M)
            C, D = fn(An, Bn, rows=rows)
        _cache[w.name] = (A, B, rows, C, D)
    return _cache[w.name]


def check(w: Workload, kernel):
    A, B, rows, Cref, D = reference(w)
    Ad, Bd = A.to(DEV), B.to(DEV)
    if kernel and not takes(kernel, Ad, Bd):
        pytest.skip(f"{kernel} does not take {w.name}")
    say(f"[parity] {w.name} kernel={kernel or 'table'} rows={'all' if rows is None else len(rows)}")
    C = run(Ad, Bd, kernel)
    C2 = run(Ad, Bd, kernel)
    assert torch.equal(C, C2), "kernel is not deterministic"
    Ch = C.cpu().numpy()
    if rows is not None:
        Ch = Ch[rows]
    e, at, n = oracle.normalized_error(Ch, Cref, D)
    say(f"[parity] {w.name} kernel={kernel or g.gemm_kernel_name(g.gemm_last_kernel())} "
        f"e={e:.3e} at={at} n>1e-5={n}")
    assert e <= GATE, f"normalized error {e} at {at}"
    return e


# -------------------------------------------------------------------- tests

SMALL_WORKLOADS = ["f32_256", "gpt_qkv", "gpt_mlp_up", "gpt_mlp_down", "skinny_1x8960x1536",
                   "skinny_7x4096x4096", "ragged_1000x3000x777", "ragged_4097x4095x1023",
                   "bf16_gpt_qkv", "bf16_gpt_mlp_down"]
LARGE_WORKLOADS = ["f32_4096", "f32_8192", "bf16_8192", "f16_8192"]


def kernel_workload_cases():
    cases = []
    for wn in SMALL_WORKLOADS + LARGE_WORKLOADS:
        w = WORKLOADS[wn]
        for k in kernels_for(w.dtype):
            if k.startswith("naive") and wn in LARGE_WORKLOADS:
                continue   # the debug kernel is only run on the smaller shapes
            cases.append((wn, k))
    return cases


@pytest.mark.parametrize("wn", SMALL_WORKLOADS + LARGE_WORKLOADS)
def test_table_choice_matches_oracle(wn):
    check(WORKLOADS[wn], None)


@pytest.mark.parametrize("wn,kernel", kernel_workload_cases())
def test_kernel_matches_oracle(wn, kernel):
    check(WORKLOADS[wn], kernel)


EXACT_SHAPES = [(1, 1, 1), (3, 5, 7), (64, 64, 64), (65, 63, 67), (256, 256, 512),
                (257, 383, 129), (300, 520, 200), (1, 8960, 96), (7, 1000, 300),
                (513, 17, 1025), (17, 513, 33), (128, 256, 4100), (1, 8, 32), (255, 264, 96),
                (520, 776, 2048), (16, 4096, 1024)]


@pytest.mark.parametrize("dtype", DTYPES)
def test_small_integer_exact(dtype):
    """Integer operands: every kernel must be exact (bitwise equal to int64)."""
    gen = workloads.generator(77)
    tdt = TDT[dtype]
    lo, hi = (-4, 4) if dtype == "f32" else (-8, 8)
    for (M, N, K) in EXACT_SHAPES:
        A = workloads.small_int((M, K), lo, hi, gen, tdt)
        B = workloads.small_int((K, N), lo, hi, gen, tdt)
        exact = (A.to(torch.int64) @ B.to(torch.int64)).to(torch.float64).numpy()
        Ad, Bd = A.to(DEV), B.to(DEV)
        for k in kernels_for(dtype):
            if not takes(k, Ad, Bd):
                continue
            say(f"[exact] {dtype} {M}x{N}x{K} kernel={k}")
            C = run(Ad, Bd, k).cpu().numpy().astype(np.float64)
            bad = np.argwhere(C != exact)
            assert bad.size == 0, f"{k} {M}x{N}x{K}: {len(bad)} wrong, first {bad[:3].tolist()}"


@pytest.mark.parametrize("dtype", DTYPES)
def test_identity_and_permutation_exact(dtype):
    tdt = TDT[dtype]
    gen = workloads.generator(78)
    for (K, N) in [(300, 260), (320, 264)]:
        B = workloads.draw((K, N), ("uniform", 1.0), gen).to(tdt)
        perm = torch.randperm(K, generator=gen)
        P = torch.zeros((K, K), dtype=tdt)
        P[torch.arange(K), perm] = 1
        Bd, Id, Pd = B.to(DEV), torch.eye(K, dtype=tdt, device=DEV), P.to(DEV)
        for k in kernels_for(dtype):
            if not takes(k, Id, Bd):
                continue
            say(f"[identity] {dtype} K={K} N={N} kernel={k}")
            C = run(Id, Bd, k)
            assert torch.equal(C.cpu(), B.float())
            C = run(Pd, Bd, k)
            assert torch.equal(C.cpu(), B.float()[perm])


# Skinny family: every compiled row count (1, 2, 4, 8, 16 after rounding up),
# every strip width (the table picks 64/128/256-byte strips from N) and
# work-group tier, K not a multiple of the 4-row blocks, for both element
# types, plus one unaligned layout per case (element-load path).
SKINNY_M = [1, 2, 3, 5, 8, 9, 16]
SKINNY_NK = [(1000, 37), (4100, 260), (8192, 44), (8200, 61), (16400, 36)]


@pytest.mark.parametrize("dtype", DTYPES)
def test_skinny_configurations_exact(dtype):
    tdt = TDT[dtype]
    lo, hi = (-4, 4) if dtype == "f32" else (-8, 8)
    gen = workloads.generator(81)
    for (N, K) in SKINNY_NK:
        B = workloads.small_int((K, N + 3), lo, hi, gen, tdt)
        Bd_al = B[:, :N].contiguous().to(DEV)
        Bd_un = B.to(DEV)[:, 1:N + 1]            # row stride N + 3, offset one element
        for M in SKINNY_M:
            A = workloads.small_int((M, K), lo, hi, gen, tdt)
            exact = (A.to(torch.int64) @ B[:, :N].to(torch.int64)).to(torch.float64).numpy()
            exact_un = (A.to(torch.int64) @ B[:, 1:N + 1].to(torch.int64)).to(torch.float64).numpy()
            Ad = A.to(DEV)
            for Bd, ref, tag in ((Bd_al, exact, "aligned"), (Bd_un, exact_un, "unaligned")):
                k = f"skinny_{dtype}"
                assert takes(k, Ad, Bd)
                say(f"[skinny] {dtype} {M}x{N}x{K} {tag}")
                C = run(Ad, Bd, k).cpu().numpy().astype(np.float64)
                bad = np.argwhere(C != ref)
                assert bad.size == 0, f"{M}x{N}x{K} {tag}: {len(bad)} wrong, first {bad[:3].tolist()}"


# Skinny products with 5-16 rows over long K: the row-split pairs and the
# 16-row work-groups, strip widths from 16 to 32 columns, K with a partial
# last block, both the LDS copy of A (aligned rows that fit) and reads of A
# from the caches (A offset by one element).
LONG_K_CASES = [(5, 4096, 4096), (7, 4096, 4096), (8, 1000, 1027), (9, 2050, 2048),
                (12, 4100, 1536), (16, 1024, 1032)]


@pytest.mark.parametrize("dtype", DTYPES)
def test_skinny_long_k_exact(dtype):
    tdt = TDT[dtype]
    lo, hi = (-4, 4) if dtype == "f32" else (-8, 8)
    gen = workloads.generator(84)
    for (M, N, K) in LONG_K_CASES:
        A = workloads.small_int((M, K + 4), lo, hi, gen, tdt)
        B = workloads.small_int((K, N), lo, hi, gen, tdt)
        exact = (A[:, :K].to(torch.int64) @ B.to(torch.int64)).to(torch.float64).numpy()
        exact_un = (A[:, 1:K + 1].to(torch.int64) @ B.to(torch.int64)).to(torch.float64).numpy()
        Ad, Bd = A.to(DEV), B.to(DEV)
        for a, ref, tag in ((Ad[:, :K].contiguous(), exact, "aligned"),
                            (Ad[:, 1:K + 1], exact_un, "A offset one element")):
            say(f"[skinny long K] {dtype} {M}x{N}x{K} {tag}")
            C = run(a, Bd, f"skinny_{dtype}")
            bad = np.argwhere(C.cpu().numpy().astype(np.float64) != ref)
            assert bad.size == 0, f"{M}x{N}x{K} {tag}: {len(bad)} wrong, first {bad[:3].tolist()}"


# The fp32 K split over two work-groups (1-16 rows, 96-255 strips of 128
# bytes or 48-95 from K = 8192, K >= 1024 up to 8 rows, K >= 2048 above): every compiled row count
# (1, 4, 8, 16 after rounding up), K with a partial last step in either
# half, a ragged last strip, row strides of A and B wider than the product,
# and rows of A that are not 16-byte aligned (element loads of A).
KSPLIT_CASES = [(1, 4096, 4096), (2, 4092, 1027), (3, 3200, 1024), (4, 4096, 1030),
                (5, 4000, 2051), (7, 4096, 4096), (8, 3072, 1500), (9, 4096, 2048),
                (12, 4064, 2049), (16, 3100, 2050), (7, 6144, 4096), (3, 5000, 1030),
                (7, 2048, 8192), (12, 3000, 8195)]


def test_skinny_k_split_exact():
    gen = workloads.generator(86)
    for (M, N, K) in KSPLIT_CASES:
        # the wide A rows are a multiple of four elements, so the strided case
        # takes the K split also where K is not
        A = workloads.small_int((M, (K + 3) // 4 * 4 + 4), -4, 4, gen)
        B = workloads.small_int((K, N + 4), -4, 4, gen)
        exact = (A[:, :K].to(torch.int64) @ B[:, :N].to(torch.int64)).to(torch.float64).numpy()
        exact_un = (A[:, 1:K + 1].to(torch.int64) @ B[:, :N].to(torch.int64)).to(torch.float64).numpy()
        Ad, Bd = A.to(DEV), B.to(DEV)
        for a, b, ref, tag in ((Ad[:, :K].contiguous(), Bd[:, :N].contiguous(), exact, "packed"),
                               (Ad[:, :K], Bd[:, :N], exact, "strided"),
                               (Ad[:, 1:K + 1], Bd[:, :N], exact_un, "A offset one element")):
            assert takes("skinny_f32", a, b)
            say(f"[skinny k split] {M}x{N}x{K} {tag}")
            C = run(a, b, "skinny_f32")
            bad = np.argwhere(C.cpu().numpy().astype(np.float64) != ref)
            assert bad.size == 0, f"{M}x{N}x{K} {tag}: {len(bad)} wrong, first {bad[:3].tolist()}"
        # random operands: within the gate, and two calls bitwise equal
        Ar = workloads.draw((M, K), ("normal", 1.0), gen)
        Br = workloads.draw((K, N), ("normal", 1.0), gen)
        ref, den = oracle.gemm_f32(Ar.numpy(), Br.numpy())
        C1 = run(Ar.to(DEV), Br.to(DEV), "skinny_f32")
        C2 = run(Ar.to(DEV), Br.to(DEV), "skinny_f32")
        assert torch.equal(C1, C2)
        err = oracle.normalized_error(C1.cpu().numpy(), ref, den)[0]
        assert err <= GATE, f"{M}x{N}x{K}: {err}"


# The 16-bit K split (bf16 and fp16, 1-8 rows, 96-128 strips of 128 bytes
# from K = 1024, 48-95 strips from K = 8192): both compiled row counts (4,
# 8), K with a partial last step in either half, a ragged last strip, row
# strides wider than the product, rows of A not 8-byte aligned.
KSPLIT16_CASES = [(1, 4096, 8192), (3, 4088, 8195), (2, 3200, 9000), (4, 6400, 1024),
                  (5, 8192, 2051), (8, 6400, 1500), (7, 8192, 4096)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_skinny_k_split_16bit_exact(dtype):
    tdt = TDT[dtype]
    gen = workloads.generator(87)
    for (M, N, K) in KSPLIT16_CASES:
        A = workloads.small_int((M, (K + 3) // 4 * 4 + 4), -8, 8, gen)
        B = workloads.small_int((K, N + 8), -8, 8, gen)
        exact = (A[:, :K].to(torch.int64) @ B[:, :N].to(torch.int64)).to(torch.float64).numpy()
        exact_un = (A[:, 1:K + 1].to(torch.int64) @ B[:, :N].to(torch.int64)).to(torch.float64).numpy()
        Ad, Bd = A.to(tdt).to(DEV), B.to(tdt).to(DEV)
        for a, b, ref, tag in ((Ad[:, :K].contiguous(), Bd[:, :N].contiguous(), exact, "packed"),
                               (Ad[:, :K], Bd[:, :N], exact, "strided"),
                               (Ad[:, 1:K + 1], Bd[:, :N], exact_un, "A offset one element")):
            k = f"skinny_{dtype}"
            assert takes(k, a, b)
            say(f"[skinny k split] {dtype} {M}x{N}x{K} {tag}")
            C = run(a, b, k)
            bad = np.argwhere(C.cpu().numpy().astype(np.float64) != ref)
            assert bad.size == 0, f"{M}x{N}x{K} {tag}: {len(bad)} wrong, first {bad[:3].tolist()}"
        # random operands: within the gate, and two calls bitwise equal
        Ar = workloads.draw((M, K), ("normal", 1.0), gen).to(tdt)
        Br = workloads.draw((K, N), ("normal", 1.0), gen).to(tdt)
        ref, den = ORACLE_FN[dtype](workloads.as_numpy_operand(Ar), workloads.as_numpy_operand(Br))
        C1 = run(Ar.to(DEV), Br.to(DEV), f"skinny_{dtype}")
        C2 = run(Ar.to(DEV), Br.to(DEV), f"skinny_{dtype}")
        assert torch.equal(C1, C2)
        err = oracle.normalized_error(C1.cpu().numpy(), ref, den)[0]
        assert err <= GATE, f"{dtype} {M}x{N}x{K}: {err}"


def test_skinny_streams_and_graphs():
    # Calls on two streams with no synchronization between them, then a
    # captured graph replayed between eager calls: every output exact, and
    # on random operands every replay bit-identical to the eager result.
    gen = workloads.generator(85)
    M, N, K = 7, 4096, 4096
    As = [workloads.small_int((M, K), -4, 4, gen).to(DEV) for _ in range(6)]
    Bs = [workloads.small_int((K, N), -4, 4, gen).to(DEV) for _ in range(2)]
    refs = [(a.cpu().to(torch.int64) @ b.cpu().to(torch.int64)).to(torch.float32)
            for a in As for b in Bs]
    streams = [torch.cuda.Stream(DEV), torch.cuda.Stream(DEV)]
    outs = [torch.empty((M, N), device=DEV) for _ in refs]
    torch.cuda.synchronize()
    for i in range(len(refs)):
        st = streams[i % 2]
        with torch.cuda.stream(st):
            g.gemm(As[i // 2], Bs[i % 2], out=outs[i])
    torch.cuda.synchronize()
    say("[skinny] two streams")
    for i, ref in enumerate(refs):
        assert torch.equal(outs[i].cpu(), ref), f"call {i}"
    Ar = workloads.draw((M, K), ("normal", 1.0), gen).to(DEV)
    Br = workloads.draw((K, N), ("normal", 1.0), gen).to(DEV)
    eager = g.gemm(Ar, Br)
    Cg = torch.empty((M, N), device=DEV)
    st = streams[0]
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=st):
            g.gemm(Ar, Br, out=Cg)
    torch.cuda.synchronize()
    for rep in range(3):
        Cg.fill_(float("nan"))
        graph.replay()
        again = g.gemm(Ar, Br)
        torch.cuda.synchronize()
        say(f"[skinny] graph replay {rep}")
        assert torch.equal(Cg, eager) and torch.equal(again, eager)


@pytest.mark.parametrize("dtype", DTYPES)
def test_ones_exact(dtype):
    """A = B = ones gives K everywhere; A = ones with integer B gives every
    row equal to B's column sums (exact: integer partial sums below 2^24)."""
    tdt = TDT[dtype]
    gen = workloads.generator(82)
    for (M, N, K) in [(300, 260, 200), (33, 17, 4100), (1, 8960, 96), (257, 264, 1024)]:
        ones_a = torch.ones((M, K), dtype=tdt)
        Bint = workloads.small_int((K, N), -4, 4, gen, tdt)
        colsum = Bint.to(torch.int64).sum(0).to(torch.float64).numpy()
        Ad, Od, Bd = ones_a.to(DEV), torch.ones((K, N), dtype=tdt, device=DEV), Bint.to(DEV)
        for k in kernels_for(dtype):
            if not takes(k, Ad, Bd):
                continue
            say(f"[ones] {dtype} {M}x{N}x{K} kernel={k}")
            C = run(Ad, Od, k).cpu().numpy()
            assert np.all(C == K), (k, M, N, K)
            C = run(Ad, Bd, k).cpu().numpy().astype(np.float64)
            assert np.all(C == colsum[None, :]), (k, M, N, K)


@pytest.mark.parametrize("dtype", DTYPES)
def test_brute_force_tiny_shapes(dtype):
    """Every (M, N, K) in {1..8}^3, every kernel that takes it, integer
    operands: bitwise equal to the int64 product."""
    tdt = TDT[dtype]
    lo, hi = (-4, 4) if dtype == "f32" else (-8, 8)
    gen = workloads.generator(83)
    A8 = workloads.small_int((8, 8), lo, hi, gen, tdt)
    B8 = workloads.small_int((8, 8), lo, hi, gen, tdt)
    names = kernels_for(dtype)
    say(f"[tiny] {dtype} 512 shapes x {len(names)} kernels")
    for M in range(1, 9):
        for N in range(1, 9):
            for K in range(1, 9):
                A, B = A8[:M, :K].contiguous(), B8[:K, :N].contiguous()
                exact = (A.to(torch.int64) @ B.to(torch.int64)).to(torch.float64).numpy()
                Ad, Bd = A.to(DEV), B.to(DEV)
                for k in names:
                    if not takes(k, Ad, Bd):
                        continue
                    C = run(Ad, Bd, k).cpu().numpy().astype(np.float64)
                    assert np.array_equal(C, exact), (k, M, N, K)


GUARD_CASES = [  # (M, N, K, extra A columns, extra B columns)
    (130, 200, 150, 13, 9), (5, 300, 64, 13, 9), (300, 257, 1000, 13, 9),
    (300, 264, 512, 16, 8), (257, 520, 96, 8, 24),
]


@pytest.mark.parametrize("dtype", DTYPES)
def test_guard_bands_and_poisoned_padding(dtype):
    """Padding of A/B rows holds NaN and must not leak; C padding and the rows
    past M must keep their sentinel."""
    tdt = TDT[dtype]
    gen = workloads.generator(79)
    for (M, N, K, pa, pb) in GUARD_CASES:
        A = workloads.small_int((M, K), -4, 4, gen, tdt)
        B = workloads.small_int((K, N), -4, 4, gen, tdt)
        exact = (A.to(torch.int64) @ B.to(torch.int64)).float()
        Abuf = torch.full((M, K + pa), float("nan"), dtype=tdt)
        Abuf[:, :K] = A
        Bbuf = torch.full((K, N + pb), float("nan"), dtype=tdt)
        Bbuf[:, :N] = B
        Ad, Bd = Abuf.to(DEV)[:, :K], Bbuf.to(DEV)[:, :N]
        for k in kernels_for(dtype):
            if not takes(k, Ad, Bd):
                continue
            say(f"[guard] {dtype} {M}x{N}x{K} kernel={k}")
            Cbuf = torch.full((M + 3, N + 7), -777.0, device=DEV)
            run(Ad, Bd, k, out=Cbuf[:M, :N])
            Ch = Cbuf.cpu()
            assert torch.equal(Ch[:M, :N], exact)
            assert torch.all(Ch[:M, N:] == -777.0) and torch.all(Ch[M:, :] == -777.0)


@pytest.mark.parametrize("dtype", DTYPES)
def test_degenerate_shapes(dtype):
    tdt = TDT[dtype]
    C = torch.full((5, 7), 3.0, device=DEV)
    g.gemm(torch.empty((5, 0), dtype=tdt, device=DEV), torch.empty((0, 7), dtype=tdt, device=DEV),
           out=C)
    torch.cuda.synchronize()
    assert torch.all(C == 0)
    C = g.gemm(torch.empty((0, 4), dtype=tdt, device=DEV), torch.ones((4, 6), dtype=tdt, device=DEV))
    assert C.shape == (0, 6)
    C = g.gemm(torch.ones((3, 4), dtype=tdt, device=DEV), torch.empty((4, 0), dtype=tdt, device=DEV))
    assert C.shape == (3, 0)


def test_invalid_call_raises():
    a = torch.ones((4, 4), device=DEV)
    with pytest.raises(g.GemmError) as ei:
        g.gemm(a, a, out=a)          # C aliases A
    assert ei.value.code == g.HIP_ERROR_INVALID_VALUE


def test_non_default_stream():
    w = WORKLOADS["ragged_1000x3000x777"]
    A, B, rows, Cref, D = reference(w)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        Ad, Bd = A.to(DEV), B.to(DEV)
        C = g.gemm(Ad, Bd)
    s.synchronize()
    Ch = C.cpu().numpy()
    if rows is not None:
        Ch = Ch[rows]
    assert oracle.normalized_error(Ch, Cref, D)[0] <= GATE



@pytest.mark.parametrize("dtype,M,N,K", [("f32", 32768, 256, 32768), ("bf16", 40960, 512, 32768),
                                         ("f16", 40960, 512, 32768)])
def test_large_operands_64bit_offsets(dtype, M, N, K):
    """A spans more than 2^31 bytes (4 GiB fp32, 2.5 GiB bf16), so row
    offsets need 64-bit arithmetic.  Every kernel that takes the shape, and
    the table's choice, is checked on sampled rows (first, last, tile
    boundaries, random) against the oracle."""
    tdt = TDT[dtype]
    gen = workloads.generator(80)
    A = workloads.draw((M, K), ("uniform", 1.0), gen).to(tdt)
    B = workloads.draw((K, N), ("uniform", 1.0), gen).to(tdt)
    rows = sample_rows(M, seed=3)
    fn = ORACLE_FN[dtype]
    Cref, D = fn(workloads.as_numpy_operand(A[rows]), workloads.as_numpy_operand(B))
    Ad, Bd = A.to(DEV), B.to(DEV)
    del A
    C = torch.empty((M, N), dtype=torch.float32, device=DEV)
    for kernel in [None] + [k for k in kernels_for(dtype) if takes(k, Ad, Bd)]:
        C.fill_(float("nan"))
        say(f"[large] {dtype} {M}x{N}x{K} kernel={kernel or 'table'}")
        run(Ad, Bd, kernel, out=C)
        e, at, _ = oracle.normalized_error(C[rows].cpu().numpy(), Cref, D)
        say(f"[large] e={e:.3e} at={at}")
        assert e <= GATE, (kernel, e, at)
    del Ad, Bd, C
    torch.cuda.empty_cache()


def test_concurrent_host_threads_and_streams():
    """The header promises thread safety: four host threads, each on its own
    stream, each running several kernel families; every result must equal
    the single-threaded result bitwise (the kernels are deterministic)."""
    import threading
    gen = workloads.generator(84)
    cases = []
    for (M, N, K, dt) in [(2048, 2048, 512, torch.float32), (16384, 384, 1536, torch.float32),
                          (7, 4096, 1024, torch.float32), (1024, 1024, 1024, torch.bfloat16),
                          (1000, 3000, 777, torch.float32)]:
        A = workloads.draw((M, K), ("uniform", 1.0), gen).to(dt).to(DEV)
        B = workloads.draw((K, N), ("uniform", 1.0), gen).to(dt).to(DEV)
        cases.append((A, B, run(A, B).clone()))
    errors = []

    def worker(tid):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                outs = []
                for rep in range(4):
                    for (A, B, _) in cases:
                        outs.append(g.gemm(A, B))
            s.synchronize()
            for i, C in enumerate(outs):
                if not torch.equal(C, cases[i % len(cases)][2]):
                    errors.append((tid, i))
        except Exception as e:   # noqa: BLE001 - reported below
            errors.append((tid, repr(e)))

    say("[threads] 4 host threads x 4 reps x 5 cases")
    ts = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not errors, errors[:5]


def test_graph_capture_replays_match_eager():
    """Calls captured into a HIP graph (no memset nodes: K = 0 and the
    two-work-group K split start C with a fill kernel) replay with the eager
    result, replay after replay, with eager work and synchronisation between
    replays; plain, transposed and batched calls in every operand type."""
    gen = workloads.generator(85)
    # (M, N, K, dtype, batch, A stored transposed, B stored transposed)
    specs = [(1024, 1024, 512, torch.float32, 1, False, False),
             (512, 768, 256, torch.bfloat16, 1, False, False),
             (3, 4096, 1024, torch.float32, 1, False, False),
             (300, 260, 0, torch.float32, 1, False, False),
             (1000, 3000, 777, torch.float32, 1, False, False),
             (256, 256, 64, torch.float32, 12, False, True),       # batched, B^T
             (384, 1152, 4096, torch.float32, 1, True, False),     # A^T, K over 2 work-groups
             (384, 1152, 4096, torch.bfloat16, 1, True, False),    # the same in bf16
             (2048, 2048, 1024, workloads.FP8_TORCH[0], 1, False, True),   # 8-bit 256^2 tile
             (512, 264, 96, torch.float16, 3, True, True),
             (300, 270, 100, torch.bfloat16, 2, True, False),      # general family
             (7, 4096, 4096, torch.float32, 1, False, False),      # few rows: K over 2 work-groups
             (4, 8192, 2048, torch.bfloat16, 1, False, False),     # the same, 16-bit
             (12, 4096, 2048, workloads.FP8_TORCH[0], 1, False, True)]   # 8-bit few rows
    ins, eager, outs = [], [], []
    for (M, N, K, dt, nb, ta, tb) in specs:
        lead = (nb,) if nb > 1 else ()
        A = workloads.draw(lead + ((K, M) if ta else (M, K)), ("uniform", 1.0), gen).to(dt).to(DEV)
        B = workloads.draw(lead + ((N, K) if tb else (K, N)), ("uniform", 1.0), gen).to(dt).to(DEV)
        A = A.transpose(-1, -2) if ta else A
        B = B.transpose(-1, -2) if tb else B
        ins.append((A, B))
        eager.append(run(A, B).clone())
        outs.append(torch.full(lead + (M, N), 7.0, device=DEV))
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for (A, B), C in zip(ins, outs):       # warm-up on the capture stream
            g.gemm(A, B, out=C)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        for (A, B), C in zip(ins, outs):
            g.gemm(A, B, out=C)
    say("[graph] 3 replays")
    for rep in range(3):
        for C in outs:
            C.fill_(-3.0)                       # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, C in enumerate(outs):
            assert torch.equal(C, eager[i]), (rep, specs[i])
