"""GPU parity of transposed-factor and strided-batched products.

C_b = op(A_b) op(B_b) through gemm_f32_batched / gemm_bf16_f32acc_batched
(the Python binding passes a transposed view such as ``w.t()`` as a
transposed factor and a 3-D tensor as a strided batch), against the oracle's
batched entry point on the same seeded operands.  Exact on small-integer
operands (every partial sum is an integer below 2^24, so any summation order
gives the same bits), the 5e-4 normalized-error gate on random operands, and
the layout edge cases: ragged tails over several tiles, unaligned and padded
rows, shared and stride-0 operands, products side by side in one output
row, K = 0, empty batches, guard bands that must stay untouched.  The GPT
backward-pass and attention shapes are checked in the launch configuration
the benchmark times, on sampled rows.
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
GATE = oracle.GATE
TRANS = [(False, False), (True, False), (False, True), (True, True)]
# kernels that take every layout, and (fp32) the LDS-direct and narrow-load
# tiles, which take the layouts their loads allow
GENERAL = {"f32": ["mfma_f32_batched", "mfma_f32_batched128", "mfma_f32_batched_splitk"],
           "bf16": ["mfma_bf16_batched", "mfma_bf16_batched128"]}
LDS_F32 = ["mfma_f32_direct", "mfma_f32_direct128", "mfma_f32_direct128x64", "mfma_f32_direct64",
           "mfma_f32_narrow128", "mfma_f32_narrow128x64", "mfma_f32_narrow64", "mfma_f32_direct64x2"]
GENERAL["f16"] = ["mfma_f16_batched", "mfma_f16_batched128"]
ALL = {"f32": GENERAL["f32"] + LDS_F32,
       "bf16": GENERAL["bf16"] + ["mfma_bf16_direct", "mfma_bf16_direct128", "mfma_bf16_direct64",
                                  "mfma_bf16_wsplit64", "mfma_bf16_wsplit64x2"],
       "f16": GENERAL["f16"] + ["mfma_f16_direct", "mfma_f16_direct128"]}
TDT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
DTYPES = ["f32", "bf16", "f16"]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class Forced:
    def __init__(self, name):
        self.kid = g.kernel_id(name) if name else -1

    def __enter__(self):
        assert g.gemm_force_kernel(self.kid) == 0

    def __exit__(self, *exc):
        g.gemm_force_kernel(-1)


def stored(x, trans):
    """Storage of the logical matrices x (..., R, C): x itself, or its
    transpose written out ((..., C, R), contiguous)."""
    return x.transpose(-1, -2).contiguous() if trans else x.contiguous()


def view(xs, trans):
    """The logical matrix as a view of its storage (a transposed view when
    the storage is transposed) - what a caller hands to gemm()."""
    return xs.transpose(-1, -2) if trans else xs


def as_oracle(x):
    return workloads.as_numpy_operand(x)


def takes(kernel, a, b, out=None):
    """Does the library accept `kernel` for gemm(a, b, out) (a host plan)?"""
    M, K, N = a.shape[-2], a.shape[-1], b.shape[-1]
    batch = a.shape[0] if a.dim() == 3 else (b.shape[0] if b.dim() == 3 else 1)
    ta, lda = g._layout(a, "a")
    tb, ldb = g._layout(b, "b")
    ldc, sc, cp = N, M * N, 3 << 40
    if out is not None:
        ldc, sc, cp = out.stride(-2), g._batch_stride(out), out.data_ptr()
    dt = {torch.float32: g.F32, torch.bfloat16: g.BF16, torch.float16: g.F16}[a.dtype]
    with Forced(kernel):
        got = g.gemm_plan_batched(dt, ta, tb, M, N, K, batch, a.data_ptr() or (1 << 40), lda,
                                  g._batch_stride(a), b.data_ptr() or (2 << 40), ldb,
                                  g._batch_stride(b), cp, ldc, sc)
    return got == g.kernel_id(kernel)


def run(a, b, kernel=None, out=None):
    with Forced(kernel):
        c = g.gemm(a, b, out=out)
    torch.cuda.synchronize()
    if kernel:
        assert g.gemm_last_kernel() == g.kernel_id(kernel)
    return c


def small_int(shape, dtype, gen):
    lo, hi = (-4, 4) if dtype == "f32" else (-8, 8)
    return workloads.small_int(shape, lo, hi, gen, TDT[dtype])


def exact_case(dtype, kernel, ta, tb, M, N, K, batch, seed):
    gen = workloads.generator(seed)
    A = small_int((batch, M, K), dtype, gen)
    B = small_int((batch, K, N), dtype, gen)
    As, Bs = stored(A, ta), stored(B, tb)
    a, b = view(As.to(DEV), ta), view(Bs.to(DEV), tb)
    if not takes(kernel, a, b):
        return False
    say(f"[batched] exact {dtype} {kernel} ta={ta} tb={tb} M={M} N={N} K={K} batch={batch}")
    C = run(a, b, kernel)
    Cref, _ = oracle.gemm_batched(as_oracle(As), as_oracle(Bs), ta, tb)
    assert C.shape == (batch, M, N)
    assert np.array_equal(C.cpu().numpy().astype(np.float64), Cref)
    C2 = run(a, b, kernel)
    assert torch.equal(C, C2), "not deterministic"
    return True


@pytest.mark.parametrize("dtype,kernel", [(d, k) for d in DTYPES for k in ALL[d]])
@pytest.mark.parametrize("ta,tb", TRANS)
def test_small_integer_exact(dtype, kernel, ta, tb):
    # several tiles in each direction with ragged tails in M, N and K; the
    # second group has M, N multiples of 4 and K of 16, the layouts the
    # LDS-direct tiles take (their edges still ragged against the tiles)
    ran = [exact_case(dtype, kernel, ta, tb, M, N, K, batch, seed)
           for (M, N, K, batch, seed) in [(300, 270, 100, 3, 41), (513, 129, 200, 2, 42),
                                          (7, 9, 3, 5, 43), (516, 268, 96, 3, 48),
                                          (8, 16, 32, 5, 49), (264, 136, 288, 2, 50)]]
    if not any(ran):
        pytest.skip(f"{kernel} takes none of these layouts")


@pytest.mark.parametrize("dtype,kernel", [("bf16", "mfma_bf16_wsplit64"), ("bf16", "mfma_bf16_wsplit64x2"),
                                          ("f32", "mfma_f32_direct64x2")])
@pytest.mark.parametrize("ta,tb", TRANS)
def test_k_split_kernels_exact(ta, tb, dtype, kernel):
    # single products whose K range is split: the bf16 64 x 64 tile whose
    # waves take every fourth K tile (K tile counts that leave the waves
    # unequal shares or none at all); x2: the K tiles also split over two
    # work-groups adding into C (odd tile counts give the halves unequal
    # shares, two tiles one each); ragged tile edges, the weight-gradient
    # shape
    shapes = [(384, 1152, 4096, 61), (200, 136, 2080, 62), (72, 64, 64, 63), (520, 264, 2048, 65),
              (136, 72, 96, 66), (64, 128, 48, 67)]
    if kernel == "mfma_bf16_wsplit64":
        shapes.append((8, 8, 32, 64))
    ran = [exact_case(dtype, kernel, ta, tb, M, N, K, 1, seed) for (M, N, K, seed) in shapes]
    assert all(ran[:5]), "the kernel refused a layout it takes"


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("ta,tb", TRANS)
def test_brute_force_tiny_shapes(dtype, ta, tb):
    # every (M, N, K) in {1..6}^3, two products each, every general kernel;
    # one batch holds all shapes' operands so each kernel launches per shape
    gen = workloads.generator(44)
    for kernel in ALL[dtype]:
        for M in range(1, 7):
            for N in range(1, 7):
                for K in range(1, 7):
                    A = small_int((2, M, K), dtype, gen)
                    B = small_int((2, K, N), dtype, gen)
                    As, Bs = stored(A, ta), stored(B, tb)
                    a, b = view(As.to(DEV), ta), view(Bs.to(DEV), tb)
                    if not takes(kernel, a, b):
                        continue
                    with Forced(kernel):
                        C = g.gemm(a, b)
                    ref = (A.to(torch.int64) @ B.to(torch.int64)).to(torch.float32)
                    assert torch.equal(C.cpu(), ref), (kernel, M, N, K)
        torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("ta,tb", TRANS)
def test_random_operands_gate(dtype, ta, tb):
    w = workloads.Workload("batched_rand", 332, 288, 512, dtype)
    gen = workloads.generator()
    tdt = TDT[dtype]
    A = workloads.draw((4, w.M, w.K), ("uniform", 1.0), gen).to(tdt)
    B = workloads.draw((4, w.K, w.N), ("uniform", 1.0), gen).to(tdt)
    As, Bs = stored(A, ta), stored(B, tb)
    Cref, D = oracle.gemm_batched(as_oracle(As), as_oracle(Bs), ta, tb)
    a, b = view(As.to(DEV), ta), view(Bs.to(DEV), tb)
    for kernel in ALL[dtype] + [None]:
        if kernel and not takes(kernel, a, b):
            continue
        say(f"[batched] gate {dtype} {kernel or 'table'} ta={ta} tb={tb}")
        C = run(a, b, kernel).cpu().numpy()
        e, at, n = oracle.normalized_error(C.reshape(-1, w.N), Cref.reshape(-1, w.N),
                                           D.reshape(-1, w.N))
        say(f"[batched]   e={e:.3e} at={at} n>1e-5={n}")
        assert e <= GATE, (kernel, e, at)


@pytest.mark.parametrize("dtype", DTYPES)
def test_unaligned_padded_and_offset_layouts(dtype):
    # odd leading dimensions and batch strides, operands starting one element
    # into their buffers: the element-load path of every general kernel
    gen = workloads.generator(45)
    M, N, K, batch = 130, 67, 77, 3
    for ta, tb in TRANS:
        A = small_int((batch, M, K), dtype, gen)
        B = small_int((batch, K, N), dtype, gen)
        ref = (A.to(torch.int64) @ B.to(torch.int64)).to(torch.float32)
        ar, ac = (K, M) if ta else (M, K)
        br, bc = (N, K) if tb else (K, N)
        abuf = torch.zeros(batch * (ar * (ac + 3) + 5) + 1, dtype=A.dtype)
        bbuf = torch.zeros(batch * (br * (bc + 1) + 3) + 1, dtype=A.dtype)
        As = abuf[1:1 + batch * (ar * (ac + 3) + 5)].view(batch, -1)[:, :ar * (ac + 3)]
        As = As.reshape(batch, ar, ac + 3)[:, :, :ac]
        Bs = bbuf[1:1 + batch * (br * (bc + 1) + 3)].view(batch, -1)[:, :br * (bc + 1)]
        Bs = Bs.reshape(batch, br, bc + 1)[:, :, :bc]
        As.copy_(stored(A, ta))
        Bs.copy_(stored(B, tb))
        abuf_d, bbuf_d = abuf.to(DEV), bbuf.to(DEV)
        Ad = abuf_d[1:1 + batch * (ar * (ac + 3) + 5)].view(batch, -1)[:, :ar * (ac + 3)]
        Ad = Ad.reshape(batch, ar, ac + 3)[:, :, :ac]
        Bd = bbuf_d[1:1 + batch * (br * (bc + 1) + 3)].view(batch, -1)[:, :br * (bc + 1)]
        Bd = Bd.reshape(batch, br, bc + 1)[:, :, :bc]
        for kernel in ALL[dtype]:
            if not takes(kernel, view(Ad, ta), view(Bd, tb)):
                continue
            say(f"[batched] unaligned {dtype} {kernel} ta={ta} tb={tb}")
            C = run(view(Ad, ta), view(Bd, tb), kernel)
            assert torch.equal(C.cpu(), ref), (kernel, ta, tb)


@pytest.mark.parametrize("dtype", DTYPES)
def test_shared_and_stride_zero_operands(dtype):
    gen = workloads.generator(46)
    M, N, K, batch = 200, 152, 96, 4
    A = small_int((batch, M, K), dtype, gen)
    W = small_int((N, K), dtype, gen)               # a weight stored N x K, used as W^T
    Ad, Wd = A.to(DEV), W.to(DEV)
    ref = (A.to(torch.int64) @ W.to(torch.int64).t()).to(torch.float32)
    for kernel in ALL[dtype] + [None]:
        if kernel and not takes(kernel, Ad, Wd.t()):
            continue
        C = run(Ad, Wd.t(), kernel)                 # 2-D factor shared by the batch
        assert torch.equal(C.cpu(), ref)
        C = run(Ad, Wd.t().unsqueeze(0).expand(batch, K, N), kernel)   # batch stride 0
        assert torch.equal(C.cpu(), ref)
    X = small_int((M, K), dtype, gen)
    Bs = small_int((batch, K, N), dtype, gen)
    ref2 = (X.to(torch.int64) @ Bs.to(torch.int64)).to(torch.float32)
    C = run(X.to(DEV), Bs.to(DEV))
    assert torch.equal(C.cpu(), ref2)


@pytest.mark.parametrize("dtype", DTYPES)
def test_outputs_side_by_side_and_guard_bands(dtype):
    # C viewed as (M, batch, N) inside rows padded by 5: products sit side by
    # side in each row; padding and everything outside stays NaN
    gen = workloads.generator(47)
    M, N, K, batch = 70, 33, 41, 3
    A = small_int((batch, M, K), dtype, gen)
    B = small_int((batch, K, N), dtype, gen)
    ref = (A.to(torch.int64) @ B.to(torch.int64)).to(torch.float32)
    ldc = batch * N + 5
    for kernel in ALL[dtype]:
        buf = torch.full((M * ldc + 64,), float("nan"), device=DEV)
        out = buf[32:32 + M * ldc].view(M, ldc)[:, :batch * N].view(M, batch, N).transpose(0, 1)
        if not takes(kernel, A.to(DEV), B.to(DEV), out):
            continue
        run(A.to(DEV), B.to(DEV), kernel, out=out)
        got = out.cpu()
        assert torch.equal(got, ref)
        rest = buf.cpu().clone()
        rest[32:32 + M * ldc].view(M, ldc)[:, :batch * N] = 0.0
        assert torch.isnan(rest[:32]).all() and torch.isnan(rest[32 + M * ldc:]).all()
        assert torch.isnan(rest[32:32 + M * ldc].view(M, ldc)[:, batch * N:]).all()


@pytest.mark.parametrize("dtype", DTYPES)
def test_degenerate_batches(dtype):
    tdt = TDT[dtype]
    # K = 0: every product is the empty sum
    for kernel in ALL[dtype] + [None]:
        out = torch.full((3, 40, 30), float("nan"), device=DEV)
        a = torch.zeros((3, 0, 40), dtype=tdt, device=DEV).transpose(1, 2)
        b = torch.zeros((3, 0, 30), dtype=tdt, device=DEV)
        if kernel and not takes(kernel, a, b, out):
            continue
        run(a, b, kernel, out=out)
        assert torch.equal(out.cpu(), torch.zeros(3, 40, 30))
    # empty batch, M = 0, N = 0: nothing is written
    out = torch.full((0, 5, 6), 7.0, device=DEV)
    run(torch.zeros((0, 5, 4), dtype=tdt, device=DEV), torch.zeros((0, 4, 6), dtype=tdt, device=DEV),
        out=out)
    out = torch.full((2, 5, 0), 7.0, device=DEV)
    run(torch.zeros((2, 5, 4), dtype=tdt, device=DEV).transpose(1, 2).transpose(1, 2),
        torch.zeros((4, 0), dtype=tdt, device=DEV), out=out)


def test_invalid_batched_calls_raise():
    a = torch.zeros((2, 8, 4), device=DEV)
    b = torch.zeros((2, 4, 8), device=DEV)
    out = torch.zeros((2, 8, 8), device=DEV)
    with pytest.raises(ValueError):
        g.gemm(a, torch.zeros((3, 4, 8), device=DEV))
    # overlapping products in C (stride_c = 1) are refused by the library
    rc = g.gemm_f32_batched(0, 0, 8, 8, 4, a.data_ptr(), 4, 32, b.data_ptr(), 8, 32,
                            out.data_ptr(), 8, 1, 2, 0)
    assert rc == g.HIP_ERROR_INVALID_VALUE
    rc = g.gemm_f32_batched(2, 0, 8, 8, 4, a.data_ptr(), 4, 32, b.data_ptr(), 8, 32,
                            out.data_ptr(), 8, 64, 2, 0)
    assert rc == g.HIP_ERROR_INVALID_VALUE
    # C overlapping A across the batch
    rc = g.gemm_f32_batched(0, 0, 8, 8, 4, a.data_ptr(), 4, 32, b.data_ptr(), 8, 32,
                            a.data_ptr(), 8, 64, 2, 0)
    assert rc == g.HIP_ERROR_INVALID_VALUE
    torch.cuda.synchronize()


def test_plain_problem_keeps_plain_kernels():
    # transa = transb = 0 and batch = 1 through the batched entry point is the
    # plain product and runs the plain table's kernel
    a = torch.rand((512, 512), device=DEV)
    b = torch.rand((512, 512), device=DEV)
    out = torch.empty((512, 512), device=DEV)
    g.gemm(a, b, out=out)
    torch.cuda.synchronize()
    plain = g.gemm_last_kernel()
    rc = g.gemm_f32_batched(0, 0, 512, 512, 512, a.data_ptr(), 512, 0, b.data_ptr(), 512, 0,
                            out.data_ptr(), 512, 0, 1, 0)
    torch.cuda.synchronize()
    assert rc == 0 and g.gemm_last_kernel() == plain
    assert not g.gemm_kernel_name(plain).endswith(("batched", "batched128"))


@pytest.mark.parametrize("name", sorted(workloads.GENERAL_WORKLOADS))
def test_benchmark_shapes_sampled(name):
    """The backward-pass and attention shapes, table choice, sampled rows of
    products spread over the batch."""
    w = workloads.GENERAL_WORKLOADS[name]
    As, Bs = workloads.make_general_inputs(w)
    a, b = workloads.general_views(w, As.to(DEV), Bs.to(DEV))
    say(f"[batched] {name} {w.batch}x({w.M},{w.N},{w.K}) ta={w.ta} tb={w.tb}")
    C = run(a, b)
    C2 = run(a, b)
    assert torch.equal(C, C2)
    Ch = C.cpu().numpy().reshape(w.batch, w.M, w.N)
    rng = np.random.default_rng(5)
    for bi in sorted({0, w.batch - 1, int(rng.integers(w.batch))}):
        rows = sorted({0, w.M - 1, *rng.choice(w.M, size=min(w.M, 12), replace=False).tolist()})
        A_b = As[bi] if As.dim() == 3 else As
        B_b = Bs[bi] if Bs.dim() == 3 else Bs
        # the rows of op(A) that matter, as a small stored operand of their own
        A_rows = (A_b.t()[rows] if w.ta else A_b[rows]).contiguous()
        Cref, D = oracle.gemm_batched(as_oracle(A_rows), as_oracle(B_b), False, w.tb)
        e, at, n = oracle.normalized_error(Ch[bi][rows], Cref, D)
        say(f"[batched]   product {bi}: e={e:.3e} at={at}")
        assert e <= GATE


# ---- K split over work-groups through a caller's workspace -------------------

WS_SHAPES = [(384, 1152, 4096, True, False), (128, 200, 2048, True, True),
             (256, 384, 1536, False, False), (200, 72, 8192, False, True),
             (128, 198, 2048, True, False)]     # N % 4 != 0: element-wise partial sums


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("M,N,K,ta,tb", WS_SHAPES)
def test_workspace_split_exact(dtype, M, N, K, ta, tb):
    gen = workloads.generator(61)
    A = small_int((M, K), dtype, gen)
    B = small_int((K, N), dtype, gen)
    As, Bs = stored(A, ta), stored(B, tb)
    a, b = view(As.to(DEV), ta), view(Bs.to(DEV), tb)
    need = g.workspace_size(a, b)
    assert need > 0, "these shapes split their K range"
    ws = torch.full((need // 4 + 64,), float("nan"), device=DEV)
    say(f"[ws] {dtype} {M}x{N}x{K} ta={ta} tb={tb} workspace={need}")
    C = g.gemm(a, b, workspace=ws)
    C2 = g.gemm(a, b, workspace=ws)
    torch.cuda.synchronize()
    Cref, _ = oracle.gemm_batched(as_oracle(As), as_oracle(Bs), ta, tb)
    assert np.array_equal(C.cpu().numpy().astype(np.float64), Cref)
    assert torch.equal(C, C2), "not deterministic"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_workspace_gate_random(dtype):
    gen = workloads.generator(62)
    M, N, K = 384, 1152, 8192
    tdt = TDT[dtype]
    X = workloads.draw((K, M), ("normal", 1.0), gen).to(tdt)     # activations, stored K x M
    dY = workloads.draw((K, N), ("normal", 1.0), gen).to(tdt)
    a, b = X.to(DEV).t(), dY.to(DEV)
    ws = torch.empty((g.workspace_size(a, b) // 4,), device=DEV)
    C = g.gemm(a, b, workspace=ws).cpu().numpy()
    plain = g.gemm(a, b).cpu().numpy()
    rows = [0, 1, 63, 64, 127, 128, 200, 383]
    A_rows = X.t()[rows].contiguous()
    Cref, D = oracle.gemm_batched(as_oracle(A_rows), as_oracle(dY), False, False)
    for got in (C, plain):
        e, at, n = oracle.normalized_error(got[rows], Cref, D)
        say(f"[ws] {dtype} random e={e:.3e} at={at}")
        assert e <= GATE


def test_workspace_too_small_or_absent_is_the_plain_call():
    gen = workloads.generator(63)
    A = small_int((4096, 384), "f32", gen)
    B = small_int((4096, 1152), "f32", gen)
    a, b = A.to(DEV).t(), B.to(DEV)
    need = g.workspace_size(a, b)
    small = torch.full((need // 4 - 1,), 5.0, device=DEV)
    C = g.gemm(a, b, workspace=small)
    torch.cuda.synchronize()
    assert torch.equal(small, torch.full_like(small, 5.0)), "a short workspace must not be touched"
    ref = (A.to(torch.int64).t() @ B.to(torch.int64)).to(torch.float32)
    assert torch.equal(C.cpu(), ref)
    # shapes that fill the CUs use no workspace
    assert g.workspace_size(torch.empty((4096, 4096), device=DEV),
                            torch.empty((4096, 4096), device=DEV)) == 0


def test_workspace_refused_when_misaligned_or_overlapping():
    a = torch.zeros((4096, 384), device=DEV).t()
    b = torch.zeros((4096, 1152), device=DEV)
    need = g.workspace_size(a, b)
    buf = torch.zeros((need // 4 + 16,), device=DEV)
    with pytest.raises(g.GemmError):
        g.gemm(a, b, workspace=buf[1:])                     # 4-byte offset
    big = torch.zeros((need // 4 + 384 * 1152,), device=DEV)
    out = big[:384 * 1152].view(384, 1152)
    with pytest.raises(g.GemmError):
        g.gemm(a, b, out=out, workspace=big)                # workspace overlapping C
    # C past the bytes the split uses: allowed
    out2 = big[need // 4:].view(384, 1152)
    g.gemm(a, b, out=out2, workspace=big)
    torch.cuda.synchronize()
