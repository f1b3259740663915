"""GPU parity of the 8-bit float products (gemm_fp8_f32acc_batched).

C_b = A_b B_b with A_b stored M x K and B_b given transposed (N x K), OCP
e4m3 / e5m2 operands in all four pairings, against the oracle's 8-bit entry
point on the same seeded bytes.  Every product of two 8-bit floats is exact
in fp32, so small-integer operands give the same bits in any summation
order and are compared exactly; random operands are held to the 5e-4
normalized-error gate.  Each 8-bit kernel is forced on the shapes it takes:
ragged M and N over several tiles, K a multiple of the 64-byte tile or only
of 16 bytes, batches with a shared or per-product factor, padded rows,
K = 0, guard bands; the headline size on sampled rows.
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
FMTS = [(0, 0), (0, 1), (1, 0), (1, 1)]
KERNELS = ["mfma_fp8_direct128", "mfma_fp8_direct256x128", "mfma_fp8_direct256", "mfma_fp8_batched",
           "mfma_fp8_batched128"]
# K from one partial 128-byte block to 64 whole ones: every path of the
# bandwidth kernel's loop (steps of four blocks per wave, the single blocks
# after them, a last block that K does not fill), N not a multiple of 16.
SKINNY_SHAPES = [(1, 300, 1024), (2, 77, 16), (3, 130, 4096), (7, 520, 256), (16, 64, 2048),
                 (9, 1000, 208), (4, 48, 6272), (5, 200, 8192), (16, 33, 6160)]
TORCH = workloads.FP8_TORCH


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


def takes(kernel, M, N, K, batch=1, lda=None, ldb=None):
    kid = g.kernel_id(kernel)
    lda = K if lda is None else lda
    ldb = K if ldb is None else ldb
    with Forced(kernel):
        return g.gemm_plan_batched(g.FP8, 0, 1, M, N, K, batch, lda=lda, ldb=ldb,
                                   stride_a=M * lda, stride_b=N * ldb) == kid


def run(A, Bt, out=None):
    """gemm with A (.., M, K) and B = Bt^T given as the view Bt.transpose."""
    C = g.gemm(A.to(DEV), Bt.to(DEV).transpose(-1, -2), out=out)
    torch.cuda.synchronize()
    return C


def ref(A, Bt, fa, fb):
    return oracle.gemm_fp8_batched(workloads.fp8_bits(A), workloads.fp8_bits(Bt), fa, fb,
                                   False, True)


def randn(shape, fmt, gen, scale=1.0):
    return (torch.randn(shape, generator=gen) * scale).to(TORCH[fmt])


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("fa,fb", FMTS)
def test_small_int_exact(kernel, fa, fb):
    M, N, K = 300, 260, 192
    assert takes(kernel, M, N, K)
    gen = workloads.generator(31)
    A = workloads.small_int((M, K), -8, 8, gen).to(TORCH[fa])
    Bt = workloads.small_int((N, K), -8, 8, gen).to(TORCH[fb])
    say(f"fp8 exact {kernel} formats {fa},{fb} {M}x{N}x{K}")
    with Forced(kernel):
        C = run(A, Bt)
    assert g.gemm_kernel_name(g.gemm_last_kernel()) == kernel
    Cref, _ = ref(A, Bt, fa, fb)
    assert np.array_equal(C.cpu().numpy().astype(np.float64), Cref)


SHAPES = [(300, 260, 192), (257, 129, 320), (64, 64, 64), (1, 300, 128), (513, 77, 1024),
          (130, 250, 208), (40, 520, 16)]


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_random_gate(kernel, M, N, K):
    if not takes(kernel, M, N, K):
        pytest.skip(f"{kernel} does not take K = {K}")
    gen = workloads.generator(32)
    for fa, fb in FMTS:
        A, Bt = randn((M, K), fa, gen), randn((N, K), fb, gen)
        say(f"fp8 gate {kernel} formats {fa},{fb} {M}x{N}x{K}")
        with Forced(kernel):
            C = run(A, Bt)
        Cref, D = ref(A, Bt, fa, fb)
        e, at, _ = oracle.normalized_error(C.cpu().numpy(), Cref, D)
        assert e <= GATE, (fa, fb, e, at)


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("shared_b", [False, True])
def test_batch(kernel, shared_b):
    batch, M, N, K = 3, 200, 136, 256
    gen = workloads.generator(33)
    A = randn((batch, M, K), 0, gen)
    Bt = randn((N, K) if shared_b else (batch, N, K), 1, gen)
    say(f"fp8 batch {kernel} shared_b={shared_b}")
    with Forced(kernel):
        C = run(A, Bt)
    assert C.shape == (batch, M, N)
    for b in range(batch):
        Cref, D = ref(A[b], Bt if shared_b else Bt[b], 0, 1)
        e, at, _ = oracle.normalized_error(C[b].cpu().numpy(), Cref, D)
        assert e <= GATE, (b, e, at)


@pytest.mark.parametrize("kernel", KERNELS)
def test_padded_rows_and_guard_band(kernel):
    M, N, K, pad = 190, 150, 320, 48
    gen = workloads.generator(34)
    Aw = randn((M, K + pad), 0, gen)
    Bw = randn((N, K + pad), 0, gen)
    A, Bt = Aw[:, :K], Bw[:, :K]                 # rows K + pad bytes apart
    big = torch.full((M + 2, N + 8), 7.0, dtype=torch.float32, device=DEV)
    out = big[1:M + 1, 4:N + 4]
    say(f"fp8 padded {kernel}")
    with Forced(kernel):
        g.gemm(Aw.to(DEV)[:, :K], Bw.to(DEV)[:, :K].t(), out=out)
        torch.cuda.synchronize()
    Cref, D = oracle.gemm_fp8_batched(workloads.fp8_bits(A.contiguous()),
                                      workloads.fp8_bits(Bt.contiguous()), 0, 0, False, True)
    e, at, _ = oracle.normalized_error(out.cpu().numpy(), Cref, D)
    assert e <= GATE, (e, at)
    ring = big.clone()
    ring[1:M + 1, 4:N + 4] = 7.0
    assert torch.all(ring == 7.0)


def test_skinny_padded_rows_and_guard_band():
    # the few-row bandwidth kernel (the table's choice up to 16 rows) on rows
    # K + pad bytes apart, writing into a window of a sentinel-filled buffer
    M, N, K, pad = 3, 150, 320, 48
    gen = workloads.generator(35)
    Aw = randn((M, K + pad), 0, gen)
    Bw = randn((N, K + pad), 0, gen)
    big = torch.full((M + 2, N + 8), 7.0, dtype=torch.float32, device=DEV)
    out = big[1:M + 1, 4:N + 4]
    a, bt = Aw.to(DEV)[:, :K], Bw.to(DEV)[:, :K]
    assert g.gemm_kernel_name(g.gemm_plan_batched(
        g.FP8, 0, 1, M, N, K, 1, a.data_ptr(), a.stride(0), 0, bt.data_ptr(), bt.stride(0), 0,
        out.data_ptr(), out.stride(0), 0)) == "skinny_fp8"
    say("fp8 padded skinny_fp8")
    g.gemm(a, bt.t(), out=out)
    torch.cuda.synchronize()
    assert g.gemm_kernel_name(g.gemm_last_kernel()) == "skinny_fp8"
    Cref, D = oracle.gemm_fp8_batched(workloads.fp8_bits(Aw[:, :K].contiguous()),
                                      workloads.fp8_bits(Bw[:, :K].contiguous()), 0, 0, False, True)
    e, at, _ = oracle.normalized_error(out.cpu().numpy(), Cref, D)
    assert e <= GATE, (e, at)
    ring = big.clone()
    ring[1:M + 1, 4:N + 4] = 7.0
    assert torch.all(ring == 7.0)


def test_k_zero_and_empty():
    # K = 0 with few rows (the shape the bandwidth kernel takes at K > 0):
    # C is the empty sum
    for M in (1, 4, 33):
        A = torch.zeros((M, 0), dtype=torch.float8_e4m3fn, device=DEV)
        Bt = torch.zeros((17, 0), dtype=torch.float8_e4m3fn, device=DEV)
        out = torch.full((M, 17), 3.0, device=DEV)
        g.gemm(A, Bt.t(), out=out)
        torch.cuda.synchronize()
        assert torch.all(out == 0), M

    empty = g.gemm(torch.zeros((0, 64), dtype=torch.float8_e4m3fn, device=DEV),
                   torch.zeros((5, 64), dtype=torch.float8_e4m3fn, device=DEV).t())
    assert empty.shape == (0, 5)


def test_rejected_layouts():
    A = torch.zeros((64, 64), dtype=torch.float8_e4m3fn, device=DEV)
    with pytest.raises(ValueError):
        g.gemm(A, A)                                  # B not given transposed
    with pytest.raises(ValueError):
        g.gemm(A.t(), A.t())                          # A transposed
    with pytest.raises(TypeError):
        g.gemm(A, A.float().t())                      # mixed 8-bit and fp32
    A24 = torch.zeros((64, 24), dtype=torch.float8_e4m3fn, device=DEV)
    with pytest.raises(g.GemmError):
        g.gemm(A24, A24.t())                          # K not a multiple of 16
    W = torch.zeros((64, 72), dtype=torch.float8_e4m3fn, device=DEV)
    with pytest.raises(g.GemmError):
        g.gemm(W[:, :64], A.t())                      # lda = 72: not a multiple of 16
    C = torch.empty((64, 64), device=DEV)
    s = torch.cuda.current_stream().cuda_stream
    assert g.gemm_fp8_f32acc(2, 0, 64, 64, 64, A.data_ptr(), 64, A.data_ptr(), 64,
                             C.data_ptr(), 64, s) == g.HIP_ERROR_INVALID_VALUE
    assert g.gemm_fp8_f32acc(0, 1, 64, 64, 64, A.data_ptr(), 64, A.data_ptr(), 64,
                             C.data_ptr(), 64, s) == 0
    torch.cuda.synchronize()


def test_plain_entry_point_matches_batched():
    M, N, K = 320, 192, 448
    gen = workloads.generator(35)
    A, Bt = randn((M, K), 1, gen), randn((N, K), 0, gen)
    Ad, Bd = A.to(DEV), Bt.to(DEV)
    C1 = torch.empty((M, N), device=DEV)
    s = torch.cuda.current_stream().cuda_stream
    assert g.gemm_fp8_f32acc(1, 0, M, N, K, Ad.data_ptr(), K, Bd.data_ptr(), K, C1.data_ptr(),
                             N, s) == 0
    C2 = g.gemm(Ad, Bd.t())
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)


@pytest.mark.parametrize("name", list(workloads.FP8_WORKLOADS))
def test_benchmark_shapes_sampled(name):
    """The table's kernel at the benchmark's sizes; sampled rows against the
    oracle (the rows of A it needs, all of B)."""
    w = workloads.FP8_WORKLOADS[name]
    A, Bt = workloads.make_fp8_inputs(w)
    plan = g.gemm_plan_batched(g.FP8, 0, 1, w.M, w.N, w.K, w.batch)
    say(f"fp8 benchmark shape {name} kernel {g.gemm_kernel_name(plan)}")
    C = run(A, Bt)
    assert g.gemm_last_kernel() == plan
    rng = np.random.default_rng(3)
    rows = sorted(set([0, w.M - 1] + rng.choice(w.M, size=min(w.M, 24), replace=False).tolist()))
    Cref, D = oracle.gemm_fp8_batched(workloads.fp8_bits(A[rows]), workloads.fp8_bits(Bt),
                                      w.fa, w.fb, False, True, threads=8)
    e, at, _ = oracle.normalized_error(C[rows].cpu().numpy(), Cref, D)
    assert e <= GATE, (e, at)


@pytest.mark.parametrize("M,N,K", SKINNY_SHAPES)
def test_skinny_gate_and_exact(M, N, K):
    """At most 16 rows: the bandwidth kernel (Bt streamed once; the table's
    choice without block scales), forced; random operands to the gate, small
    integers exactly, all four format pairings."""
    assert takes("skinny_fp8", M, N, K)
    gen = workloads.generator(36)
    for fa, fb in FMTS:
        A, Bt = randn((M, K), fa, gen), randn((N, K), fb, gen)
        say(f"fp8 skinny formats {fa},{fb} {M}x{N}x{K}")
        with Forced("skinny_fp8"):
            C = run(A, Bt)
        assert g.gemm_kernel_name(g.gemm_last_kernel()) == "skinny_fp8"
        Cref, D = ref(A, Bt, fa, fb)
        e, at, _ = oracle.normalized_error(C.cpu().numpy(), Cref, D)
        assert e <= GATE, (fa, fb, e, at)
        Ai = workloads.small_int((M, K), -8, 8, gen).to(TORCH[fa])
        Bi = workloads.small_int((N, K), -8, 8, gen).to(TORCH[fb])
        with Forced("skinny_fp8"):
            C = run(Ai, Bi)
        Cref, _ = ref(Ai, Bi, fa, fb)
        assert np.array_equal(C.cpu().numpy().astype(np.float64), Cref)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("kernel", ["skinny_fp8", "mfma_fp8_direct128"])
def test_every_finite_pattern_decodes(fmt, kernel):
    """C = A times a one-hot Bt: row 0 of A holds every finite pattern of
    the format once, column j of C picks pattern j, so C[0] is the
    decoded value of each pattern (exact)."""
    bits = np.arange(256, dtype=np.uint8)
    vals = torch.from_numpy(bits.copy()).view(TORCH[fmt]).float()
    keep = torch.isfinite(vals).numpy()
    pats = bits[keep]
    K = 256
    N = len(pats)
    A = np.zeros((1, K), dtype=np.uint8)
    A[0, :N] = pats
    one = torch.ones(1).to(TORCH[fmt]).view(torch.uint8).item()
    Bt = np.zeros((N, K), dtype=np.uint8)
    Bt[np.arange(N), np.arange(N)] = one
    At = torch.from_numpy(A).view(TORCH[fmt])
    Btt = torch.from_numpy(Bt).view(TORCH[fmt])
    say(f"fp8 decode {kernel} format {fmt}")
    with Forced(kernel):
        C = run(At, Btt)
    assert g.gemm_kernel_name(g.gemm_last_kernel()) == kernel
    expect = oracle.load().decode_fp8(fmt, pats)
    got = C[0].cpu().numpy().astype(np.float64)
    assert np.array_equal(got, expect)      # -0 comes out as +0: it is added to +0 terms
