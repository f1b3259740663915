"""GPU parity of 8-bit products with MX block scales (gemm_mxfp8_f32acc).

C = sum_k (a_ik 2^(SA[k/32][i] - 127)) (bt_jk 2^(SB[k/32][j] - 127)) with one
E8M0 scale per 32 elements of K of each row of A and of Bt, against the
oracle's MX entry point on the same seeded bytes.  Each kernel that takes
scales is forced: the bandwidth kernel (at most 8 rows), both LDS-direct
tiles (K a multiple of 64) and the 128 x 128 register-staged tile (K a
multiple of 32 only).  Small-integer operands with scales between 2^-1 and
2^4 keep every partial sum a multiple of 1/2 below 2^22, so any order is
exact and the result is compared bit for bit; random operands with scales
from 2^-9 to 2^9 are held to the 5e-4 normalized-error gate (the magnitude
sum includes the scales).  Also: unit scales give the unscaled product,
scaling one block of one row changes exactly that row, a NaN scale poisons
exactly the outputs it touches, padded scale pitches, ragged edges, and the
refused arguments.
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
TORCH = workloads.FP8_TORCH
KERNELS = ["skinny_fp8", "mfma_fp8_direct128", "mfma_fp8_direct256x128", "mfma_fp8_direct256",
           "mfma_fp8_batched128"]


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


def scales(nblk, rows, lo, hi, gen, pad=0):
    """(nblk, W) uint8 E8M0 scales drawn in [lo, hi] for `rows` rows, W the
    row count rounded up to a multiple of 4 plus `pad`; the padding is set
    to the NaN pattern, which must never reach a stored result."""
    width = -(-rows // 4) * 4 + pad
    s = torch.randint(lo, hi + 1, (nblk, width), generator=gen).to(torch.uint8)
    s[:, rows:] = 255
    return s


def plan(A, SA, Bt, SB, C):
    M, K = A.shape
    N = Bt.shape[0]
    return g.gemm_plan_mxfp8(M, N, K, A.data_ptr(), A.stride(0), SA.data_ptr(), SA.stride(0),
                             Bt.data_ptr(), Bt.stride(0), SB.data_ptr(), SB.stride(0),
                             C.data_ptr(), C.stride(0))


def run(A, SA, Bt, SB, kernel=None):
    """The product on the GPU through the C-ABI, with `kernel` forced."""
    Ad, SAd, Btd, SBd = A.to(DEV), SA.to(DEV), Bt.to(DEV), SB.to(DEV)
    C = torch.full((A.shape[0], Bt.shape[0]), float("nan"), device=DEV)
    with Forced(kernel):
        if kernel:
            assert plan(Ad, SAd, Btd, SBd, C) == g.kernel_id(kernel), f"{kernel} refused the shape"
        g.gemm_mx(Ad, SAd, Btd.t(), SBd, out=C)
        torch.cuda.synchronize()
    if kernel:
        assert g.gemm_last_kernel() == g.kernel_id(kernel)
    return C.cpu()


def ref(A, SA, Bt, SB):
    fa = 0 if A.dtype == torch.float8_e4m3fn else 1
    fb = 0 if Bt.dtype == torch.float8_e4m3fn else 1
    return oracle.gemm_mxfp8(workloads.fp8_bits(A), SA.numpy(), workloads.fp8_bits(Bt),
                             SB.numpy(), fa, fb)


def shape_for(kernel):
    if kernel == "skinny_fp8":
        # up to 16 rows; whole 128-byte steps and a last block K half fills
        return [(1, 300, 1024), (3, 130, 4096), (8, 77, 160), (12, 200, 8192), (16, 33, 6176)]
    if kernel == "mfma_fp8_batched128":
        return [(300, 260, 224), (129, 70, 32)]
    return [(300, 260, 256), (520, 136, 1024)]


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("fa,fb", [(0, 0), (1, 0), (0, 1)])
def test_small_int_exact(kernel, fa, fb):
    gen = workloads.generator(51)
    for (M, N, K) in shape_for(kernel):
        A = workloads.small_int((M, K), -4, 4, gen).to(TORCH[fa])
        Bt = workloads.small_int((N, K), -4, 4, gen).to(TORCH[fb])
        SA = scales(K // 32, M, 126, 129, gen, pad=4)
        SB = scales(K // 32, N, 127, 129, gen, pad=8)
        C = run(A, SA, Bt, SB, kernel)
        Cref, _ = ref(A, SA[:, :M], Bt, SB[:, :N])
        bad = np.argwhere(C.numpy().astype(np.float64) != Cref)
        say(f"[mx] {kernel} {M}x{N}x{K} fmt={fa}{fb} mismatches={len(bad)}")
        assert len(bad) == 0, f"first at {tuple(bad[0])}: {C.numpy()[tuple(bad[0])]} vs " \
                              f"{Cref[tuple(bad[0])]}"


@pytest.mark.parametrize("kernel", KERNELS)
def test_random_scales_gate(kernel):
    gen = workloads.generator(52)
    for (M, N, K) in shape_for(kernel):
        A = (torch.randn((M, K), generator=gen)).to(TORCH[0])
        Bt = (torch.randn((N, K), generator=gen)).to(TORCH[1])
        SA = scales(K // 32, M, 118, 136, gen)
        SB = scales(K // 32, N, 118, 136, gen, pad=4)
        C = run(A, SA, Bt, SB, kernel)
        Cref, D = ref(A, SA, Bt, SB[:, :N])
        e, at, n = oracle.normalized_error(C.numpy(), Cref, D)
        say(f"[mx] {kernel} random {M}x{N}x{K} e={e:.3e} at={at}")
        assert e <= GATE, f"normalized error {e} at {at}"


@pytest.mark.parametrize("kernel", KERNELS)
def test_unit_scales_and_one_scaled_block(kernel):
    gen = workloads.generator(53)
    M, N, K = [s for s in shape_for(kernel) if s[0] >= 3][0]
    A = workloads.small_int((M, K), -8, 8, gen).to(TORCH[0])
    Bt = workloads.small_int((N, K), -8, 8, gen).to(TORCH[0])
    SA = torch.full((K // 32, -(-M // 4) * 4), 127, dtype=torch.uint8)
    SB = torch.full((K // 32, -(-N // 4) * 4), 127, dtype=torch.uint8)
    C1 = run(A, SA, Bt, SB, kernel)
    C0 = g.gemm(A.to(DEV), Bt.to(DEV).t()).cpu()          # the unscaled entry point
    assert torch.equal(C1, C0)
    # block 1 of row 2 of A times 8: only row 2 changes, by 7 times that
    # block's partial products
    SA[1, 2] = 130
    C2 = run(A, SA, Bt, SB, kernel)
    blk = slice(32, 64)
    part = (A[2:3, blk].float() @ Bt[:, blk].float().t())[0]
    assert torch.equal(C2[2], C1[2] + 7 * part)
    keep = [i for i in range(M) if i != 2]
    assert torch.equal(C2[keep], C1[keep])


@pytest.mark.parametrize("kernel", KERNELS)
def test_nan_scale_poisons_its_outputs(kernel):
    gen = workloads.generator(54)
    M, N, K = shape_for(kernel)[0]
    A = workloads.small_int((M, K), -4, 4, gen).to(TORCH[0])
    Bt = workloads.small_int((N, K), -4, 4, gen).to(TORCH[0])
    SA = torch.full((K // 32, -(-M // 4) * 4), 127, dtype=torch.uint8)
    SB = torch.full((K // 32, -(-N // 4) * 4), 127, dtype=torch.uint8)
    SA[0, M - 1] = 255                      # row M-1 of A, block 0
    SB[K // 32 - 1, 5] = 255                # row 5 of Bt, last block
    C = run(A, SA, Bt, SB, kernel)
    nan = torch.isnan(C)
    want = torch.zeros_like(nan)
    want[M - 1, :] = True
    want[:, 5] = True
    assert torch.equal(nan, want)


def test_table_choice_and_headline_size_sampled():
    # the table's kernels: <= 16 rows the bandwidth kernel, whole 64-byte K
    # tiles the LDS-direct tiles, else the 128 x 128 register-staged tile;
    # 8192^3 with random scales on sampled rows
    gen = workloads.generator(55)
    for (M, N, K, want) in [(4, 512, 1024, "skinny_fp8"), (256, 256, 512, "mfma_fp8_direct128"),
                            (2048, 2048, 2048, "mfma_fp8_direct128"),
                            (4096, 4096, 4096, "mfma_fp8_direct256"),
                            (512, 512, 480, "mfma_fp8_batched128")]:
        A = torch.zeros((M, K), dtype=torch.uint8, device=DEV).view(torch.float8_e4m3fn)
        Bt = torch.zeros((N, K), dtype=torch.uint8, device=DEV).view(torch.float8_e4m3fn)
        SA = torch.zeros((K // 32, M), dtype=torch.uint8, device=DEV)
        SB = torch.zeros((K // 32, N), dtype=torch.uint8, device=DEV)
        C = torch.empty((M, N), device=DEV)
        assert g.gemm_kernel_name(plan(A, SA, Bt, SB, C)) == want
    S = 8192
    A = torch.randn((S, S), generator=gen).to(TORCH[0])
    Bt = torch.randn((S, S), generator=gen).to(TORCH[0])
    SA = scales(S // 32, S, 120, 134, gen)
    SB = scales(S // 32, S, 120, 134, gen)
    C = run(A, SA, Bt, SB)
    rows = [0, 1, 255, 256, 4095, 8191] + torch.randint(0, S, (10,), generator=gen).tolist()
    Cref, D = oracle.gemm_mxfp8(workloads.fp8_bits(A[rows]), SA[:, rows].numpy(),
                                workloads.fp8_bits(Bt), SB.numpy(), 0, 0)
    e, at, _ = oracle.normalized_error(C[rows].numpy(), Cref, D)
    say(f"[mx] 8192^3 kernel={g.gemm_kernel_name(g.gemm_last_kernel())} e={e:.3e}")
    assert e <= GATE


def test_refused_arguments():
    st = torch.cuda.current_stream().cuda_stream
    M, N, K = 64, 64, 128
    A = torch.zeros((M, K), dtype=torch.uint8, device=DEV)
    Bt = torch.zeros((N, K), dtype=torch.uint8, device=DEV)
    SA = torch.full((K // 32, M + 4), 127, dtype=torch.uint8, device=DEV)
    SB = torch.full((K // 32, N), 127, dtype=torch.uint8, device=DEV)
    C = torch.zeros((M, N), device=DEV)

    def call(K_=K, sa=SA.data_ptr(), lsa=M + 4, sb=SB.data_ptr(), lsb=N, c=C.data_ptr()):
        return g.gemm_mxfp8_f32acc(0, 0, M, N, K_, A.data_ptr(), K, sa, lsa, Bt.data_ptr(), K,
                                   sb, lsb, c, N, st)

    assert call() == 0
    assert call(K_=96) == 0                              # 3 blocks: the staged tile
    assert call(K_=48) != 0                              # not whole 32-element blocks
    assert call(sa=0) != 0 and call(sb=0) != 0           # null scales
    assert call(lsa=M - 4) != 0                          # scale pitch below M
    assert call(lsa=M + 2) != 0                          # pitch not a multiple of 4
    assert call(sa=SA.data_ptr() + 2) != 0               # misaligned scales
    # C on top of the scales
    big = torch.zeros(M * N + 64, device=DEV)
    assert g.gemm_mxfp8_f32acc(0, 0, M, N, K, A.data_ptr(), K, big.data_ptr(), M, Bt.data_ptr(),
                               K, SB.data_ptr(), N, big.data_ptr(), N, st) != 0
    torch.cuda.synchronize()
