"""CPU oracle for C = A·B — TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (``dense_gemm_17_amd``) never imports
it and shares no code with it; the two meet only through the seeded input
generators in ``workloads.py``, which hold none of the product's arithmetic.

``oracle.c`` is the plain definition of the matrix product ("Bare Metal Bard",
page 1, first paragraph: the ladder of matmul kernels; vidyal.ai Part 5,
"Writing a Fast Matmul in CUDA, Step by Step"), accumulated in fp64 together
with the magnitude sum D = sum_k |a_ik * b_kj| that the correctness gate
divides by.  Every entry point here is pinned by ``tests/test_oracle.py``
(identity, permutation, ones, exact small-integer, brute force against exact
rational arithmetic, numpy fp64 BLAS, thread-count invariance and planted
mutants).  The row-sampled entries (fp32, bf16 and fp16) are pinned to the
selected rows of the full product and, on small-integer operands, to the
exact integer product's rows, with a planted fp16-rows mistake that the pin
rejects; no function is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

# -O2 without fast-math and with contraction off: the sums are evaluated in
# source order, one rounding per addition, no fused multiply-add.
CFLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
          "-pthread", "-shared", "-fPIC", "-Wall", "-Wextra"]

MUTANTS = ("DROP_LAST_K", "TRANSPOSE_B", "SIGNED_D", "BF16_SWAP", "IGNORE_TA", "BATCH_B0",
           "F16_BIAS", "E4M3_NAN", "F16_ROWS_BF16", "MX_BLOCK16", "E8M0_BIAS")


def build(out: str = _LIB_PATH, mutant: Optional[str] = None) -> str:
    """Compile oracle.c with gcc into ``out``.  ``mutant`` names one planted
    mistake (see MUTANTS) for the oracle's own sensitivity tests."""
    cmd = ["gcc", *CFLAGS, _SRC, "-o", out, "-lm"]
    if mutant is not None:
        if mutant not in MUTANTS:
            raise ValueError(f"unknown oracle mutant {mutant!r}")
        cmd.insert(1, f"-DORACLE_MUTANT_{mutant}")
    subprocess.run(cmd, check=True)
    return out


_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    full = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _i64, ctypes.c_int]
    rows = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _i64, ctypes.c_int]
    for name, argt in (("oracle_gemm_f32", full), ("oracle_gemm_bf16", full),
                       ("oracle_gemm_f16", full), ("oracle_gemm_f32_rows", rows),
                       ("oracle_gemm_bf16_rows", rows), ("oracle_gemm_f16_rows", rows)):
        fn = getattr(lib, name)
        fn.argtypes = argt
        fn.restype = ctypes.c_int
    ci = ctypes.c_int
    lib.oracle_gemm_batched.argtypes = [ci, ci, ci, _i64, _i64, _i64, _vp, _i64, _i64,
                                        _vp, _i64, _i64, _i64, _vp, _vp, _i64, ci]
    lib.oracle_gemm_batched.restype = ci
    for name in ("oracle_decode_bf16", "oracle_decode_f16"):
        getattr(lib, name).argtypes = [_vp, _vp, _i64]
        getattr(lib, name).restype = None
    lib.oracle_gemm_fp8_batched.argtypes = [ci, ci, ci, ci, _i64, _i64, _i64, _vp, _i64, _i64,
                                            _vp, _i64, _i64, _i64, _vp, _vp, _i64, ci]
    lib.oracle_gemm_fp8_batched.restype = ci
    lib.oracle_decode_fp8.argtypes = [ci, _vp, _vp, _i64]
    lib.oracle_decode_fp8.restype = None
    lib.oracle_gemm_mxfp8.argtypes = [ci, ci, _i64, _i64, _i64, _vp, _i64, _vp, _i64,
                                      _vp, _i64, _vp, _i64, _vp, _vp, _i64, ci]
    lib.oracle_gemm_mxfp8.restype = ci
    lib.oracle_decode_e8m0.argtypes = [_vp, _vp, _i64]
    lib.oracle_decode_e8m0.restype = None
    return lib


_lib: Optional["Oracle"] = None


class Oracle:
    """Thin ctypes wrapper around one build of oracle.c."""

    def __init__(self, path: str):
        self.path = path
        self.lib = _bind(ctypes.CDLL(path))

    @staticmethod
    def _operand(x: np.ndarray, dtype) -> Tuple[np.ndarray, int]:
        if x.ndim != 2:
            raise ValueError("operands must be 2-D")
        if x.dtype != dtype:
            raise TypeError(f"expected {np.dtype(dtype)}, got {x.dtype}")
        if x.shape[0] and x.shape[1] and x.strides[1] != x.itemsize:
            x = np.ascontiguousarray(x)
        ld = x.strides[0] // x.itemsize if x.shape[0] > 1 else max(1, x.shape[1])
        return x, max(ld, x.shape[1], 1)

    def _call(self, fn_name, dtype, A, B, rows, threads):
        A, lda = self._operand(A, dtype)
        B, ldb = self._operand(B, dtype)
        M, K = A.shape
        K2, N = B.shape
        if K != K2:
            raise ValueError(f"inner dimensions differ: {A.shape} x {B.shape}")
        if rows is None:
            nr = M
        else:
            rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
            nr = rows.shape[0]
        C = np.zeros((nr, N), dtype=np.float64)
        D = np.zeros((nr, N), dtype=np.float64)
        ptr = lambda a: a.ctypes.data if a.size else None  # noqa: E731
        if rows is None:
            rc = getattr(self.lib, fn_name)(M, N, K, ptr(A), lda, ptr(B), ldb,
                                            ptr(C), ptr(D), max(N, 1), threads)
        else:
            rc = getattr(self.lib, fn_name + "_rows")(M, N, K, ptr(A), lda, ptr(B), ldb,
                                                      ptr(rows), nr, ptr(C), ptr(D),
                                                      max(N, 1), threads)
        if rc != 0:
            raise RuntimeError(f"{fn_name} failed with code {rc}")
        return C, D

    def gemm_f32(self, A: np.ndarray, B: np.ndarray, rows: Optional[Sequence[int]] = None,
                 threads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        """(C, D) in fp64 for fp32 operands; ``rows`` restricts to those rows of C."""
        return self._call("oracle_gemm_f32", np.float32, A, B, rows, threads)

    def gemm_bf16(self, A_bits: np.ndarray, B_bits: np.ndarray,
                  rows: Optional[Sequence[int]] = None,
                  threads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        """(C, D) in fp64 for bf16 operands given as raw uint16 patterns."""
        return self._call("oracle_gemm_bf16", np.uint16, A_bits, B_bits, rows, threads)

    @staticmethod
    def _stored(x: np.ndarray, dtype) -> Tuple[np.ndarray, int, int, int]:
        """(array, batch, batch stride, row stride) of a 2-D or 3-D operand as
        stored; a 2-D operand is one matrix reused by every product."""
        if x.dtype != dtype:
            raise TypeError(f"expected {np.dtype(dtype)}, got {x.dtype}")
        if x.ndim == 2:
            x = x[None]
            bstride_zero = True
        elif x.ndim == 3:
            bstride_zero = False
        else:
            raise ValueError("operands must be 2-D or 3-D")
        if x.size and x.shape[2] > 1 and x.strides[2] != x.itemsize:
            x = np.ascontiguousarray(x)
        if x.size and x.shape[1] > 1 and (x.strides[1] < 0 or x.strides[1] % x.itemsize):
            x = np.ascontiguousarray(x)
        if x.size and x.shape[0] > 1 and (x.strides[0] < 0 or x.strides[0] % x.itemsize):
            x = np.ascontiguousarray(x)
        ld = x.strides[1] // x.itemsize if x.shape[1] > 1 else max(1, x.shape[2])
        ld = max(ld, x.shape[2], 1)
        sb = 0 if (bstride_zero or x.shape[0] <= 1) else x.strides[0] // x.itemsize
        return x, x.shape[0], sb, ld

    def gemm_batched(self, A: np.ndarray, B: np.ndarray, transa: bool = False,
                     transb: bool = False, threads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        """(C, D) in fp64 for C_b = op(A_b) op(B_b), b over the batch.

        A and B are given as stored: A is M x K (K x M when ``transa``), B is
        K x N (N x K when ``transb``); float32, uint16 bf16 patterns or float16.  A
        3-D operand is a batch (any batch stride, 0 included, e.g. from
        numpy.broadcast_to); a 2-D one is reused by every product.  The result
        is (batch, M, N), or (M, N) when both operands are 2-D."""
        dtype = A.dtype
        if dtype not in (np.float32, np.uint16, np.float16) or B.dtype != dtype:
            raise TypeError("operands must both be float32, both uint16 (bf16 patterns) or both "
                            f"float16, got {A.dtype}, {B.dtype}")
        kind = {np.dtype(np.float32): 0, np.dtype(np.uint16): 1, np.dtype(np.float16): 2}[dtype]
        two_d = A.ndim == 2 and B.ndim == 2
        A3, ba, sa, lda = self._stored(A, dtype)
        B3, bb, sb, ldb = self._stored(B, dtype)
        if A.ndim == 3 and B.ndim == 3 and ba != bb:
            raise ValueError(f"batch sizes differ: {ba} and {bb}")
        batch = ba if A.ndim == 3 else bb
        M, K = (A3.shape[2], A3.shape[1]) if transa else (A3.shape[1], A3.shape[2])
        K2, N = (B3.shape[2], B3.shape[1]) if transb else (B3.shape[1], B3.shape[2])
        if K != K2:
            raise ValueError(f"inner dimensions differ: {K} and {K2}")
        C = np.zeros((batch, M, N), dtype=np.float64)
        D = np.zeros((batch, M, N), dtype=np.float64)
        ptr = lambda a: a.ctypes.data if a.size else None  # noqa: E731
        rc = self.lib.oracle_gemm_batched(kind, int(transa), int(transb), M, N, K,
                                          ptr(A3), lda, sa, ptr(B3), ldb, sb, batch,
                                          ptr(C), ptr(D), max(N, 1), threads)
        if rc != 0:
            raise RuntimeError(f"oracle_gemm_batched failed with code {rc}")
        return (C[0], D[0]) if two_d else (C, D)

    def gemm_f16(self, A: np.ndarray, B: np.ndarray, rows: Optional[Sequence[int]] = None,
                 threads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        """(C, D) in fp64 for fp16 operands (numpy float16 arrays; the oracle
        decodes their bit patterns itself)."""
        return self._call("oracle_gemm_f16", np.float16, A, B, rows, threads)

    def _decode(self, fn, bits):
        bits = np.ascontiguousarray(bits, dtype=np.uint16).reshape(-1)
        out = np.empty(bits.shape, dtype=np.float64)
        if bits.size:
            fn(bits.ctypes.data, out.ctypes.data, bits.size)
        return out

    def gemm_fp8_batched(self, A: np.ndarray, B: np.ndarray, fmt_a: int = 0, fmt_b: int = 0,
                         transa: bool = False, transb: bool = False,
                         threads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        """(C, D) in fp64 for 8-bit operands given as uint8 patterns (format
        0: e4m3, 1: e5m2), laid out as for gemm_batched."""
        two_d = A.ndim == 2 and B.ndim == 2
        A3, ba, sa, lda = self._stored(A, np.uint8)
        B3, bb, sb, ldb = self._stored(B, np.uint8)
        if A.ndim == 3 and B.ndim == 3 and ba != bb:
            raise ValueError(f"batch sizes differ: {ba} and {bb}")
        batch = ba if A.ndim == 3 else bb
        M, K = (A3.shape[2], A3.shape[1]) if transa else (A3.shape[1], A3.shape[2])
        K2, N = (B3.shape[2], B3.shape[1]) if transb else (B3.shape[1], B3.shape[2])
        if K != K2:
            raise ValueError(f"inner dimensions differ: {K} and {K2}")
        C = np.zeros((batch, M, N), dtype=np.float64)
        D = np.zeros((batch, M, N), dtype=np.float64)
        ptr = lambda a: a.ctypes.data if a.size else None  # noqa: E731
        rc = self.lib.oracle_gemm_fp8_batched(fmt_a, fmt_b, int(transa), int(transb), M, N, K,
                                              ptr(A3), lda, sa, ptr(B3), ldb, sb, batch,
                                              ptr(C), ptr(D), max(N, 1), threads)
        if rc != 0:
            raise RuntimeError(f"oracle_gemm_fp8_batched failed with code {rc}")
        return (C[0], D[0]) if two_d else (C, D)

    def gemm_mxfp8(self, A: np.ndarray, SA: np.ndarray, Bt: np.ndarray, SB: np.ndarray,
                   fmt_a: int = 0, fmt_b: int = 0, threads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        """(C, D) in fp64 for 8-bit operands with MX block scales: A (M x K)
        and Bt (N x K) uint8 patterns, SA (K/32 x >= M) and SB (K/32 x >= N)
        uint8 E8M0 scales, the scale of block kb of row i of A at SA[kb, i]
        (rows of the scale arrays may be padded)."""
        A = np.asarray(A, dtype=np.uint8)
        Bt = np.asarray(Bt, dtype=np.uint8)
        M, K = A.shape
        N, K2 = Bt.shape
        if K != K2:
            raise ValueError(f"inner dimensions differ: {K} and {K2}")
        SA = np.asarray(SA, dtype=np.uint8)
        SB = np.asarray(SB, dtype=np.uint8)
        for S_, n in ((SA, M), (SB, N)):
            if S_.ndim != 2 or S_.shape[1] < n or S_.shape[0] * 32 < K or \
                    (S_.shape[1] > 1 and S_.strides[1] != 1):
                raise ValueError("scales must be (blocks of K) x (rows) uint8, unit column stride")
        lda = A.strides[0] if M > 1 else max(K, 1)
        ldb = Bt.strides[0] if N > 1 else max(K, 1)
        if (K > 1 and (A.strides[1] != 1 or Bt.strides[1] != 1)):
            raise ValueError("operands need unit stride along K")
        C = np.zeros((M, N), dtype=np.float64)
        D = np.zeros((M, N), dtype=np.float64)
        ptr = lambda a: a.ctypes.data if a.size else None  # noqa: E731
        ld_sa = SA.strides[0] if SA.shape[0] > 1 else SA.shape[1]
        ld_sb = SB.strides[0] if SB.shape[0] > 1 else SB.shape[1]
        rc = self.lib.oracle_gemm_mxfp8(fmt_a, fmt_b, M, N, K, ptr(A), lda, ptr(SA), ld_sa,
                                        ptr(Bt), ldb, ptr(SB), ld_sb, ptr(C), ptr(D), max(N, 1),
                                        threads)
        if rc != 0:
            raise RuntimeError(f"oracle_gemm_mxfp8 failed with code {rc}")
        return C, D

    def decode_e8m0(self, bits: np.ndarray) -> np.ndarray:
        bits = np.ascontiguousarray(bits, dtype=np.uint8).reshape(-1)
        out = np.empty(bits.shape, dtype=np.float64)
        if bits.size:
            self.lib.oracle_decode_e8m0(bits.ctypes.data, out.ctypes.data, bits.size)
        return out

    def decode_fp8(self, fmt: int, bits: np.ndarray) -> np.ndarray:
        bits = np.ascontiguousarray(bits, dtype=np.uint8).reshape(-1)
        out = np.empty(bits.shape, dtype=np.float64)
        if bits.size:
            self.lib.oracle_decode_fp8(fmt, bits.ctypes.data, out.ctypes.data, bits.size)
        return out

    def decode_bf16(self, bits: np.ndarray) -> np.ndarray:
        return self._decode(self.lib.oracle_decode_bf16, bits)

    def decode_f16(self, bits: np.ndarray) -> np.ndarray:
        return self._decode(self.lib.oracle_decode_f16, bits)


def load(path: str = _LIB_PATH) -> Oracle:
    """The default oracle build, compiled on first use if it is missing."""
    global _lib
    if _lib is None or _lib.path != path:
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
            build(path)
        _lib = Oracle(path)
    return _lib


def gemm_f32(A, B, rows=None, threads=0):
    return load().gemm_f32(A, B, rows, threads)


def gemm_bf16(A_bits, B_bits, rows=None, threads=0):
    return load().gemm_bf16(A_bits, B_bits, rows, threads)


def gemm_f16(A, B, rows=None, threads=0):
    return load().gemm_f16(A, B, rows, threads)


def gemm_fp8_batched(A, B, fmt_a=0, fmt_b=0, transa=False, transb=False, threads=0):
    return load().gemm_fp8_batched(A, B, fmt_a, fmt_b, transa, transb, threads)


def gemm_mxfp8(A, SA, Bt, SB, fmt_a=0, fmt_b=0, threads=0):
    return load().gemm_mxfp8(A, SA, Bt, SB, fmt_a, fmt_b, threads)


def gemm_batched(A, B, transa=False, transb=False, threads=0):
    return load().gemm_batched(A, B, transa, transb, threads)


def normalized_error(c: np.ndarray, c_ref: np.ndarray, d: np.ndarray):
    """The correctness gate's statistic: max_ij |c_ij - C_ij| / D_ij.

    Returns (e, (i, j) of the worst entry, count of entries above 1e-5).
    A non-finite c gives e = inf.  Where D_ij = 0 every product is zero, so the
    only correct value is exactly C_ij (= 0): any other value gives e = inf.
    """
    c = np.asarray(c, dtype=np.float64)
    if c.shape != c_ref.shape or c.shape != d.shape:
        raise ValueError(f"shape mismatch {c.shape} {c_ref.shape} {d.shape}")
    if c.size == 0:
        return 0.0, (0, 0), 0
    diff = np.abs(c - c_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(d > 0, diff / np.where(d > 0, d, 1.0),
                         np.where(diff == 0, 0.0, np.inf))
    ratio = np.where(np.isfinite(c), ratio, np.inf)
    idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    return float(ratio[idx]), (int(idx[0]), int(idx[1])), int(np.count_nonzero(ratio > 1e-5))


# Gate on the normalized error for both the fp32 and the bf16 path.
GATE = 5e-4
