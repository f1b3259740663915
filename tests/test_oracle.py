"""Pins of the CPU oracle against facts that do not come from the oracle itself.

The oracle computes the plain definition of the matrix product (the subject of
"Bare Metal Bard", page 1, first paragraph) in fp64 with the magnitude sum D.
Each pin below is chosen so that a plausible mistake (a dropped term, a wrong
index or transposed operand, a signed magnitude sum, a mis-decoded bf16
pattern) fails at least one of them; the planted-mutant test at the end builds
those mistakes into the oracle and checks exactly that.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads

HERE = os.path.dirname(os.path.abspath(__file__))
ULP53 = 2.0 ** -53


def read_golden(name):
    mats, cur, rows = {}, None, []
    with open(os.path.join(HERE, "golden", name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0].isalpha() or parts[0][0].isalpha():
                if cur:
                    mats[cur] = np.array(rows, dtype=np.float64)
                cur, rows = parts[0], []
            else:
                rows.append([float(x) for x in parts])
    mats[cur] = np.array(rows, dtype=np.float64)
    return mats


def rng(seed=99):
    return np.random.default_rng(seed)


def rand_f32(shape, seed):
    return (rng(seed).random(shape, dtype=np.float32) * 2 - 1).astype(np.float32)


# --------------------------------------------------------------------------
# pins, written as functions of an Oracle instance so the mutant test can
# re-run them against planted mistakes.
# --------------------------------------------------------------------------

def pin_golden(o):
    g = read_golden("textbook_2x3x2.txt")
    C, D = o.gemm_f32(g["A"].astype(np.float32), g["B"].astype(np.float32))
    assert np.array_equal(C, g["C"]) and np.array_equal(D, g["C"])
    C2, D2 = o.gemm_f32(g["A2"].astype(np.float32), g["B"].astype(np.float32))
    assert np.array_equal(C2, g["C2"]) and np.array_equal(D2, g["D2"])


def pin_identity(o):
    B = rand_f32((37, 53), 1)
    C, D = o.gemm_f32(np.eye(37, dtype=np.float32), B)
    assert np.array_equal(C, B.astype(np.float64))
    assert np.array_equal(D, np.abs(B).astype(np.float64))
    A = rand_f32((41, 29), 2)
    C, _ = o.gemm_f32(A, np.eye(29, dtype=np.float32))
    assert np.array_equal(C, A.astype(np.float64))


def pin_permutation(o):
    r = rng(3)
    B = rand_f32((31, 45), 4)
    perm = r.permutation(31)
    P = np.zeros((31, 31), dtype=np.float32)
    P[np.arange(31), perm] = 1.0            # (P B)[i] = B[perm[i]]
    C, _ = o.gemm_f32(P, B)
    assert np.array_equal(C, B[perm].astype(np.float64))
    A = rand_f32((23, 45), 5)
    perm2 = r.permutation(45)
    Q = np.zeros((45, 45), dtype=np.float32)
    Q[perm2, np.arange(45)] = 1.0           # (A Q)[:, j] = A[:, perm2[j]]
    C, _ = o.gemm_f32(A, Q)
    assert np.array_equal(C, A[:, perm2].astype(np.float64))


def pin_ones(o):
    M, N, K = 5, 19, 301
    B = rand_f32((K, N), 6)
    C, D = o.gemm_f32(np.ones((M, K), dtype=np.float32), B)
    # every row of C is the column sums of B; math.fsum is correctly rounded
    colsum = np.array([math.fsum(float(x) for x in B[:, j]) for j in range(N)])
    colabs = np.array([math.fsum(abs(float(x)) for x in B[:, j]) for j in range(N)])
    for i in range(M):
        assert np.all(np.abs(C[i] - colsum) <= K * ULP53 * colabs)
        assert np.all(np.abs(D[i] - colabs) <= K * ULP53 * colabs)
    C1, D1 = o.gemm_f32(np.ones((3, 777), np.float32), np.ones((777, 4), np.float32))
    assert np.all(C1 == 777.0) and np.all(D1 == 777.0)


def pin_small_int_f32(o):
    g = workloads.generator(11)
    for (M, N, K) in [(33, 65, 129), (7, 300, 1000), (64, 64, 64)]:
        A = workloads.small_int((M, K), -4, 4, g).numpy()
        B = workloads.small_int((K, N), -4, 4, g).numpy()
        C, D = o.gemm_f32(A, B)
        Ai, Bi = A.astype(np.int64), B.astype(np.int64)
        assert np.array_equal(C, (Ai @ Bi).astype(np.float64))
        assert np.array_equal(D, (np.abs(Ai) @ np.abs(Bi)).astype(np.float64))


def pin_small_int_bf16(o):
    g = workloads.generator(12)
    for (M, N, K) in [(17, 40, 96), (5, 128, 333)]:
        At = workloads.small_int((M, K), -8, 8, g, torch.bfloat16)
        Bt = workloads.small_int((K, N), -8, 8, g, torch.bfloat16)
        C, D = o.gemm_bf16(workloads.bf16_bits(At), workloads.bf16_bits(Bt))
        Ai = At.to(torch.int64).numpy()
        Bi = Bt.to(torch.int64).numpy()
        assert np.array_equal(C, (Ai @ Bi).astype(np.float64))
        assert np.array_equal(D, (np.abs(Ai) @ np.abs(Bi)).astype(np.float64))


def pin_bf16_matches_decoded_f32(o):
    # torch's bf16 -> fp32 conversion is exact, so the bf16 product must equal
    # the fp32 product of the converted operands bit for bit.
    At, Bt = workloads.make_inputs(workloads.Workload("t", 19, 27, 70, "bf16",
                                                      ("normal", 1.0), ("normal", 1.0)))
    C, D = o.gemm_bf16(workloads.bf16_bits(At), workloads.bf16_bits(Bt))
    C2, D2 = o.gemm_f32(At.float().numpy(), Bt.float().numpy())
    assert np.array_equal(C, C2) and np.array_equal(D, D2)


def pin_numpy_blas(o):
    for (M, N, K), seed in [((256, 256, 256), 7), ((13, 71, 250), 8), ((65, 3, 1000), 9)]:
        A, B = rand_f32((M, K), seed), rand_f32((K, N), seed + 100)
        C, D = o.gemm_f32(A, B)
        ref = A.astype(np.float64) @ B.astype(np.float64)
        dref = np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64))
        assert np.all(np.abs(C - ref) <= 1e-12 * dref)
        assert np.all(np.abs(D - dref) <= 1e-12 * dref)


def pin_brute_force(o, shapes):
    for (M, N, K) in shapes:
        seed = 1000 * M + 100 * N + K
        A, B = rand_f32((M, K), seed), rand_f32((K, N), seed + 7)
        C, D = o.gemm_f32(A, B)
        Af = [[Fraction(float(x)) for x in row] for row in A]
        Bf = [[Fraction(float(x)) for x in row] for row in B]
        for i in range(M):
            for j in range(N):
                exact = sum((Af[i][k] * Bf[k][j] for k in range(K)), Fraction(0))
                mag = sum((abs(Af[i][k] * Bf[k][j]) for k in range(K)), Fraction(0))
                bound = K * ULP53 * float(mag)
                assert abs(Fraction(C[i, j]) - exact) <= Fraction(bound) + Fraction(1, 2**1074)
                assert abs(Fraction(D[i, j]) - mag) <= Fraction(bound) + Fraction(1, 2**1074)


TRANS = [(False, False), (True, False), (False, True), (True, True)]


def stored(x, trans):
    """The storage of a logical matrix x: itself, or its transpose written out."""
    return np.ascontiguousarray(x.T) if trans else np.ascontiguousarray(x)


def pin_transposed_small_int(o):
    # Transposed storage of either factor: the product of the logical
    # matrices, exactly (integer entries, every partial sum below 2^24),
    # against numpy's int64 product.
    g = workloads.generator(13)
    for ta, tb in TRANS:
        for (M, N, K) in [(33, 65, 129), (7, 30, 100), (40, 9, 17)]:
            A = workloads.small_int((M, K), -4, 4, g).numpy()
            B = workloads.small_int((K, N), -4, 4, g).numpy()
            C, D = o.gemm_batched(stored(A, ta), stored(B, tb), ta, tb)
            Ai, Bi = A.astype(np.int64), B.astype(np.int64)
            assert np.array_equal(C, (Ai @ Bi).astype(np.float64))
            assert np.array_equal(D, (np.abs(Ai) @ np.abs(Bi)).astype(np.float64))
        At = workloads.small_int((19, 48), -8, 8, g, torch.bfloat16)
        Bt = workloads.small_int((48, 23), -8, 8, g, torch.bfloat16)
        Ab, Bb = workloads.bf16_bits(At), workloads.bf16_bits(Bt)
        C, D = o.gemm_batched(stored(Ab, ta), stored(Bb, tb), ta, tb)
        Ai, Bi = At.to(torch.int64).numpy(), Bt.to(torch.int64).numpy()
        assert np.array_equal(C, (Ai @ Bi).astype(np.float64))
        assert np.array_equal(D, (np.abs(Ai) @ np.abs(Bi)).astype(np.float64))


def pin_transposed_permutation(o):
    # A transposed permutation factor permutes rows (or columns) of the other
    # factor exactly; reading the storage the wrong way round applies the
    # inverse permutation instead.
    r = rng(14)
    perm = r.permutation(29)
    P = np.zeros((29, 29), dtype=np.float32)
    P[np.arange(29), perm] = 1.0            # (P B)[i] = B[perm[i]]
    B = rand_f32((29, 41), 15)
    C, _ = o.gemm_batched(stored(P, True), B, True, False)
    assert np.array_equal(C, B[perm].astype(np.float64))
    A = rand_f32((17, 29), 16)
    Q = np.zeros((29, 29), dtype=np.float32)
    Q[perm, np.arange(29)] = 1.0            # (A Q)[:, j] = A[:, perm[j]]
    C, _ = o.gemm_batched(A, stored(Q, True), False, True)
    assert np.array_equal(C, A[:, perm].astype(np.float64))


def pin_batched(o):
    # Each product of a strided batch is the product of its own pair, exactly;
    # a 2-D or stride-0 operand is reused by every product; the batch stride
    # may skip matrices of a larger array.
    g = workloads.generator(17)
    nb, M, N, K = 4, 11, 13, 37
    A = workloads.small_int((2 * nb, M, K), -4, 4, g).numpy()[::2]   # batch stride 2*M*K
    B = workloads.small_int((nb, K, N), -4, 4, g).numpy()
    for ta, tb in TRANS:
        As = np.stack([stored(a, ta) for a in A])[:, :, :]
        Bs = np.stack([stored(b, tb) for b in B])
        C, D = o.gemm_batched(As, Bs, ta, tb)
        assert C.shape == (nb, M, N)
        for b in range(nb):
            Ai, Bi = A[b].astype(np.int64), B[b].astype(np.int64)
            assert np.array_equal(C[b], (Ai @ Bi).astype(np.float64))
            assert np.array_equal(D[b], (np.abs(Ai) @ np.abs(Bi)).astype(np.float64))
    C, _ = o.gemm_batched(A, B[1])                                   # shared B
    Cz, _ = o.gemm_batched(np.broadcast_to(A[2], (3, M, K)), B[:3])  # batch stride 0
    for b in range(nb):
        assert np.array_equal(C[b], (A[b].astype(np.int64) @ B[1].astype(np.int64)).astype(np.float64))
    for b in range(3):
        assert np.array_equal(Cz[b], (A[2].astype(np.int64) @ B[b].astype(np.int64)).astype(np.float64))


def pin_f16_decoder(o):
    # every binary16 pattern against numpy's own float16 -> float64 conversion
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = o.decode_f16(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan]))
    # patterns worked by hand: 1, -2, 1 + 2^-10, the smallest subnormal, 65504
    assert list(o.decode_f16(np.array([0x3C00, 0xC000, 0x3C01, 0x0001, 0x7BFF], np.uint16))) == \
        [1.0, -2.0, 1.0 + 2.0 ** -10, 2.0 ** -24, 65504.0]


def pin_small_int_f16(o):
    g = workloads.generator(18)
    for (M, N, K) in [(17, 40, 96), (5, 128, 333)]:
        A = workloads.small_int((M, K), -8, 8, g, torch.float16).numpy()
        B = workloads.small_int((K, N), -8, 8, g, torch.float16).numpy()
        C, D = o.gemm_f16(A, B)
        Ai, Bi = A.astype(np.int64), B.astype(np.int64)
        assert np.array_equal(C, (Ai @ Bi).astype(np.float64))
        assert np.array_equal(D, (np.abs(Ai) @ np.abs(Bi)).astype(np.float64))
        Cb, _ = o.gemm_batched(np.ascontiguousarray(A.T), B, True, False)
        assert np.array_equal(Cb, C)


def pin_f16_matches_decoded_f32(o):
    # fp16 -> fp32 conversion is exact, so the fp16 product must equal the
    # fp32 product of the converted operands bit for bit
    r = rng(19)
    A = (r.standard_normal((23, 70)) * 3).astype(np.float16)
    B = (r.standard_normal((70, 31)) * 1e-3).astype(np.float16)   # subnormals included
    C, D = o.gemm_f16(A, B)
    C2, D2 = o.gemm_f32(A.astype(np.float32), B.astype(np.float32))
    assert np.array_equal(C, C2) and np.array_equal(D, D2)


def pin_rows_subsets(o):
    # the row-sampled entries (the checkers of the largest products) must
    # give exactly the selected rows of the full product, for every element
    # type, with rows repeated and out of order; on small-integer operands
    # they must also equal the exact integer product's rows
    rows = [19, 2, 2, 0, 11]
    r = rng(31)
    A = (r.standard_normal((20, 37)) * 2).astype(np.float16)
    B = (r.standard_normal((37, 15)) * 1e-3).astype(np.float16)    # subnormals included
    C, D = o.gemm_f16(A, B)
    Cr, Dr = o.gemm_f16(A, B, rows=rows, threads=2)
    assert np.array_equal(Cr, C[rows]) and np.array_equal(Dr, D[rows])
    g = workloads.generator(32)
    for dt, fn in ((torch.float16, o.gemm_f16), (torch.float32, o.gemm_f32)):
        Ai = workloads.small_int((20, 41), -8, 8, g, dt)
        Bi = workloads.small_int((41, 9), -8, 8, g, dt)
        Cr, Dr = fn(Ai.numpy(), Bi.numpy(), rows=rows)
        Ae, Be = Ai.to(torch.int64).numpy(), Bi.to(torch.int64).numpy()
        assert np.array_equal(Cr, (Ae @ Be)[rows].astype(np.float64))
        assert np.array_equal(Dr, (np.abs(Ae) @ np.abs(Be))[rows].astype(np.float64))
    Ab = workloads.bf16_bits(workloads.small_int((20, 30), -8, 8, g, torch.bfloat16))
    Bb = workloads.bf16_bits(workloads.small_int((30, 10), -8, 8, g, torch.bfloat16))
    Cb, Db = o.gemm_bf16(Ab, Bb)
    Cbr, Dbr = o.gemm_bf16(Ab, Bb, rows=rows)
    assert np.array_equal(Cbr, Cb[rows]) and np.array_equal(Dbr, Db[rows])


FP8_TORCH = {0: torch.float8_e4m3fn, 1: torch.float8_e5m2}


def fp8_bits(t):
    return t.contiguous().view(torch.uint8).numpy()


def pin_fp8_decoders(o):
    # all 256 patterns of each 8-bit format against torch's own conversion
    bits = np.arange(256, dtype=np.uint8)
    for fmt, tdt in FP8_TORCH.items():
        mine = o.decode_fp8(fmt, bits)
        ref = torch.from_numpy(bits.copy()).view(tdt).to(torch.float64).numpy()
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(mine), nan)
        assert np.array_equal(mine[~nan], ref[~nan])
        assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan]))
    # hand-worked: e4m3 1.0 = 0x38, 448 = 0x7E, smallest subnormal 2^-9 = 0x01;
    # e5m2 1.0 = 0x3C, 57344 = 0x7B, infinity = 0x7C
    assert list(o.decode_fp8(0, np.array([0x38, 0x7E, 0x01, 0xB8], np.uint8))) == \
        [1.0, 448.0, 2.0 ** -9, -1.0]
    assert list(o.decode_fp8(1, np.array([0x3C, 0x7B, 0x7C], np.uint8))) == \
        [1.0, 57344.0, math.inf]


def pin_fp8_products(o):
    # small integers are exact in both formats: the product of the logical
    # matrices exactly, for mixed formats and the transposed-B layout
    g = workloads.generator(21)
    for fa, fb in ((0, 0), (1, 1), (0, 1)):
        A = workloads.small_int((19, 64), -8, 8, g).to(FP8_TORCH[fa])
        B = workloads.small_int((64, 23), -8, 8, g).to(FP8_TORCH[fb])
        C, D = o.gemm_fp8_batched(fp8_bits(A), fp8_bits(B.t()), fa, fb, False, True)
        Ai, Bi = A.to(torch.int64).numpy(), B.to(torch.int64).numpy()
        assert np.array_equal(C, (Ai @ Bi).astype(np.float64))
        assert np.array_equal(D, (np.abs(Ai) @ np.abs(Bi)).astype(np.float64))
    # random operands: bit-equal to the fp32 product of the converted operands
    r = torch.Generator().manual_seed(22)
    A = (torch.randn((17, 96), generator=r) * 4).to(torch.float8_e4m3fn)
    B = (torch.randn((96, 13), generator=r) * 1e-2).to(torch.float8_e5m2)
    C, D = o.gemm_fp8_batched(fp8_bits(A), fp8_bits(B), 0, 1)
    C2, D2 = o.gemm_f32(A.float().numpy(), B.float().numpy())
    assert np.array_equal(C, C2) and np.array_equal(D, D2)


def pin_mx_scales(o):
    """8-bit operands with MX block scales (one E8M0 scale per 32 elements of
    K of each row of A and each column of B)."""
    # the scale decoder on all 256 patterns against torch's own E8M0 type
    bits = np.arange(256, dtype=np.uint8)
    mine = o.decode_e8m0(bits)
    ref = torch.from_numpy(bits.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref)) and np.isnan(mine[255])
    assert np.array_equal(mine[:255], ref[:255]) and mine[127] == 1.0 and mine[130] == 8.0
    g = workloads.generator(40)
    # unit scales (127) are exactly the unscaled product
    A = workloads.small_int((9, 96), -8, 8, g).to(torch.float8_e4m3fn)
    Bt = workloads.small_int((7, 96), -8, 8, g).to(torch.float8_e5m2)
    ones_a = np.full((3, 9), 127, np.uint8)
    ones_b = np.full((3, 7), 127, np.uint8)
    C, D = o.gemm_mxfp8(fp8_bits(A), ones_a, fp8_bits(Bt), ones_b, 0, 1)
    C0, D0 = o.gemm_fp8_batched(fp8_bits(A), fp8_bits(Bt), 0, 1, False, True)
    assert np.array_equal(C, C0) and np.array_equal(D, D0)
    # worked by hand: 1 x 1 x 64 of ones, A's blocks scaled 2 and 1/2, B's 1 and 8:
    # 32 * 2 * 1 + 32 * (1/2) * 8 = 192
    one_a = torch.ones((1, 64)).to(torch.float8_e4m3fn)
    one_b = torch.ones((1, 64)).to(torch.float8_e4m3fn)
    C, D = o.gemm_mxfp8(fp8_bits(one_a), np.array([[128], [126]], np.uint8), fp8_bits(one_b),
                        np.array([[127], [130]], np.uint8))
    assert C[0, 0] == 192.0 and D[0, 0] == 192.0
    C, _ = o.gemm_mxfp8(fp8_bits(one_a), np.array([[255], [127]], np.uint8), fp8_bits(one_b),
                        np.array([[127], [127]], np.uint8))
    assert np.isnan(C[0, 0])                       # the NaN scale
    # small integers with random scales, against exact block sums
    for (M, N, K, fa, fb) in [(5, 6, 128, 0, 0), (3, 11, 96, 1, 0)]:
        A = workloads.small_int((M, K), -8, 8, g).to(FP8_TORCH[fa])
        Bt = workloads.small_int((N, K), -8, 8, g).to(FP8_TORCH[fb])
        SA = torch.randint(118, 137, (K // 32, M + 3), generator=g).to(torch.uint8).numpy()
        SB = torch.randint(118, 137, (K // 32, N), generator=g).to(torch.uint8).numpy()
        C, D = o.gemm_mxfp8(fp8_bits(A), SA[:, :M], fp8_bits(Bt), SB, fa, fb)
        Ai, Bi = A.to(torch.int64).numpy(), Bt.to(torch.int64).numpy()
        want = np.zeros((M, N))
        wabs = np.zeros((M, N))
        for kb in range(K // 32):
            blk = slice(32 * kb, 32 * kb + 32)
            sc = np.exp2(SA[kb, :M].astype(np.float64) - 127)[:, None] * \
                np.exp2(SB[kb].astype(np.float64) - 127)[None, :]
            want += sc * (Ai[:, blk] @ Bi[:, blk].T)
            wabs += sc * (np.abs(Ai[:, blk]) @ np.abs(Bi[:, blk]).T)
        assert np.array_equal(C, want) and np.array_equal(D, wabs)


PINS = [pin_golden, pin_identity, pin_permutation, pin_ones, pin_small_int_f32,
        pin_small_int_bf16, pin_bf16_matches_decoded_f32, pin_numpy_blas,
        pin_transposed_small_int, pin_transposed_permutation, pin_batched,
        pin_f16_decoder, pin_small_int_f16, pin_f16_matches_decoded_f32,
        pin_fp8_decoders, pin_fp8_products, pin_rows_subsets, pin_mx_scales,
        lambda o: pin_brute_force(o, [(2, 3, 4), (3, 1, 5), (4, 4, 2)])]


# --------------------------------------------------------------------------
# the tests proper
# --------------------------------------------------------------------------

@pytest.fixture(scope="module")
def orc():
    return oracle.load()


@pytest.mark.parametrize("pin", PINS, ids=lambda p: getattr(p, "__name__", "brute_small"))
def test_pin(orc, pin):
    pin(orc)


def test_brute_force_all_tiny_shapes(orc):
    shapes = [(m, n, k) for m in range(1, 9) for n in range(1, 9) for k in range(1, 9)]
    pin_brute_force(orc, shapes)


def test_brute_force_edge_shapes(orc):
    pin_brute_force(orc, [(13, 17, 31), (33, 5, 65), (1, 65, 33), (17, 13, 1)])


@pytest.mark.parametrize("ta,tb", TRANS)
def test_brute_force_transposed(orc, ta, tb):
    # exact rational arithmetic on the logical matrices, every tiny shape up to 5
    for (M, N, K) in [(m, n, k) for m in range(1, 6) for n in range(1, 6) for k in range(1, 6)]:
        seed = 7000 + 100 * M + 10 * N + K
        A, B = rand_f32((M, K), seed), rand_f32((K, N), seed + 1)
        C, D = orc.gemm_batched(stored(A, ta), stored(B, tb), ta, tb)
        for i in range(M):
            for j in range(N):
                terms = [Fraction(float(A[i, k])) * Fraction(float(B[k, j])) for k in range(K)]
                exact, mag = sum(terms, Fraction(0)), sum((abs(t) for t in terms), Fraction(0))
                bound = Fraction(K * ULP53 * float(mag)) + Fraction(1, 2**1074)
                assert abs(Fraction(C[i, j]) - exact) <= bound
                assert abs(Fraction(D[i, j]) - mag) <= bound


def test_batched_degenerate_and_invalid(orc):
    C, D = orc.gemm_batched(np.zeros((0, 3, 4), np.float32), np.zeros((0, 4, 5), np.float32))
    assert C.shape == (0, 3, 5)
    C, D = orc.gemm_batched(np.zeros((2, 3, 0), np.float32), np.zeros((2, 0, 5), np.float32))
    assert C.shape == (2, 3, 5) and np.all(C == 0) and np.all(D == 0)
    with pytest.raises(ValueError):
        orc.gemm_batched(np.zeros((2, 3, 4), np.float32), np.zeros((3, 4, 5), np.float32))
    with pytest.raises(ValueError):
        orc.gemm_batched(np.zeros((3, 4), np.float32), np.zeros((3, 5), np.float32), True, True)


def test_thread_count_invariance(orc):
    A, B = rand_f32((97, 130), 20), rand_f32((130, 77), 21)
    C1, D1 = orc.gemm_f32(A, B, threads=1)
    for t in (2, 3, 8, 200):
        Ct, Dt = orc.gemm_f32(A, B, threads=t)
        assert np.array_equal(C1, Ct) and np.array_equal(D1, Dt)


def test_rows_subset_matches_full(orc):
    A, B = rand_f32((50, 40), 22), rand_f32((40, 33), 23)
    C, D = orc.gemm_f32(A, B)
    rows = [49, 0, 17, 17, 3]
    Cr, Dr = orc.gemm_f32(A, B, rows=rows, threads=3)
    assert np.array_equal(Cr, C[rows]) and np.array_equal(Dr, D[rows])
    g = workloads.generator(5)
    Ab = workloads.bf16_bits(workloads.small_int((20, 30), -8, 8, g, torch.bfloat16))
    Bb = workloads.bf16_bits(workloads.small_int((30, 10), -8, 8, g, torch.bfloat16))
    Cb, Db = orc.gemm_bf16(Ab, Bb)
    Cbr, Dbr = orc.gemm_bf16(Ab, Bb, rows=[19, 2])
    assert np.array_equal(Cbr, Cb[[19, 2]]) and np.array_equal(Dbr, Db[[19, 2]])
    with pytest.raises(RuntimeError):
        orc.gemm_f32(A, B, rows=[50])


def test_leading_dimensions(orc):
    # operands that are views into wider buffers (lda > K, ldb > N)
    Abuf, Bbuf = rand_f32((30, 64), 24), rand_f32((50, 40), 25)
    A, B = Abuf[:, :50], Bbuf[:, :21]
    C, D = orc.gemm_f32(A, B)
    C2, D2 = orc.gemm_f32(np.ascontiguousarray(A), np.ascontiguousarray(B))
    assert np.array_equal(C, C2) and np.array_equal(D, D2)


def test_degenerate_sizes(orc):
    C, D = orc.gemm_f32(np.zeros((4, 0), np.float32), np.zeros((0, 6), np.float32))
    assert C.shape == (4, 6) and np.all(C == 0) and np.all(D == 0)
    C, D = orc.gemm_f32(np.zeros((0, 5), np.float32), np.zeros((5, 6), np.float32))
    assert C.shape == (0, 6)
    C, D = orc.gemm_f32(np.ones((3, 5), np.float32), np.zeros((5, 0), np.float32))
    assert C.shape == (3, 0)


def test_bf16_decoder_all_patterns(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = orc.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan]))
    # a few patterns worked by hand from the binary32 layout
    assert list(orc.decode_bf16(np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x8000], np.uint16))) == \
        [1.0, -2.0, 1.0078125, 2.0 ** -133, -0.0]


def test_normalized_error_statistic():
    cref = np.array([[1.0, 2.0], [0.0, -3.0]])
    d = np.array([[2.0, 4.0], [0.0, 3.0]])
    c = cref.copy()
    assert oracle.normalized_error(c, cref, d)[0] == 0.0
    c[0, 1] += 1.0                          # error 1 over magnitude 4
    e, at, n = oracle.normalized_error(c, cref, d)
    assert e == 0.25 and at == (0, 1) and n == 1
    c2 = cref.copy(); c2[1, 0] = 1e-30      # D = 0 demands exactly 0
    assert oracle.normalized_error(c2, cref, d)[0] == math.inf
    c3 = cref.copy(); c3[1, 1] = np.nan
    assert oracle.normalized_error(c3, cref, d)[0] == math.inf


def test_workload_generator_is_seeded():
    w = workloads.WORKLOADS["f32_256"]
    A1, B1 = workloads.make_inputs(w)
    A2, B2 = workloads.make_inputs(w)
    assert torch.equal(A1, A2) and torch.equal(B1, B2)
    assert float(A1.min()) >= -1.0 and float(A1.max()) < 1.0
    wb = workloads.Workload("b", 64, 64, 64, "bf16", ("normal", 1.0), ("normal", 1.0))
    Ab, _ = workloads.make_inputs(wb)
    assert Ab.dtype == torch.bfloat16
    # bf16 inputs are the fp32 draw rounded to nearest even
    g = workloads.generator()
    assert torch.equal(Ab, torch.randn((64, 64), generator=g).to(torch.bfloat16))


@pytest.mark.parametrize("mutant", oracle.MUTANTS)
def test_planted_mutant_fails_a_pin(tmp_path, mutant):
    """Each planted mistake in the oracle must be caught by at least one pin."""
    path = oracle.build(str(tmp_path / f"liboracle_{mutant}.so"), mutant=mutant)
    bad = oracle.Oracle(path)
    caught = []
    for pin in PINS:
        try:
            pin(bad)
        except AssertionError:
            caught.append(getattr(pin, "__name__", "brute_small"))
    assert caught, f"mutant {mutant} passed every pin"
