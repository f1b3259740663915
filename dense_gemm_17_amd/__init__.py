"""Python binding of libmi355gemm (C = A·B on MI355X / gfx950).

Argument marshalling only: every step of the product runs in the library's
HIP kernels.  PyTorch supplies device memory and the stream.  The names match
the C-ABI in include/mi355gemm.h.  If the shared library has not been built
the import fails: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmi355gemm.so")

F32 = 0
BF16 = 1
HIP_SUCCESS = 0
HIP_ERROR_INVALID_VALUE = 1


class GemmError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what} failed with hipError {code}")
        self.code = code


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python dense_gemm_17_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    sig = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp]
    for name in ("gemm_f32", "gemm_bf16_f32acc"):
        getattr(lib, name).argtypes = sig
        getattr(lib, name).restype = ci
    lib.gemm_kernel_count.argtypes = []
    lib.gemm_kernel_count.restype = ci
    lib.gemm_kernel_name.argtypes = [ci]
    lib.gemm_kernel_name.restype = ctypes.c_char_p
    lib.gemm_kernel_dtype.argtypes = [ci]
    lib.gemm_kernel_dtype.restype = ci
    lib.gemm_plan.argtypes = [ci, i64, i64, i64, ctypes.c_size_t, i64, ctypes.c_size_t, i64,
                              ctypes.c_size_t, i64]
    lib.gemm_plan.restype = ci
    lib.gemm_force_kernel.argtypes = [ci]
    lib.gemm_force_kernel.restype = ci
    lib.gemm_last_kernel.argtypes = []
    lib.gemm_last_kernel.restype = ci
    lib.gemm_build_info.argtypes = []
    lib.gemm_build_info.restype = ctypes.c_char_p
    return lib


lib = _load()

# Every symbol include/mi355gemm.h declares.
EXPORTS = ("gemm_f32", "gemm_bf16_f32acc", "gemm_kernel_count", "gemm_kernel_name",
           "gemm_kernel_dtype", "gemm_plan", "gemm_force_kernel", "gemm_last_kernel",
           "gemm_build_info")


# ---- raw entry points (pointers and sizes, same names as the C-ABI) --------

def gemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream) -> int:
    return lib.gemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_bf16_f32acc(M, N, K, A, lda, B, ldb, C, ldc, stream) -> int:
    return lib.gemm_bf16_f32acc(M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_kernel_count() -> int:
    return lib.gemm_kernel_count()


def gemm_kernel_name(kid: int) -> str:
    return lib.gemm_kernel_name(kid).decode()


def gemm_kernel_dtype(kid: int) -> int:
    return lib.gemm_kernel_dtype(kid)


def gemm_plan(dtype, M, N, K, A=1 << 40, lda=None, B=2 << 40, ldb=None, C=3 << 40,
              ldc=None) -> int:
    """Kernel id the table picks (pure host call); pointers matter by alignment."""
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return lib.gemm_plan(dtype, M, N, K, A, lda, B, ldb, C, ldc)


def gemm_force_kernel(kid: int) -> int:
    return lib.gemm_force_kernel(kid)


def gemm_last_kernel() -> int:
    return lib.gemm_last_kernel()


def gemm_build_info() -> str:
    return lib.gemm_build_info().decode()


def kernel_id(name: str) -> int:
    for i in range(gemm_kernel_count()):
        if gemm_kernel_name(i) == name:
            return i
    raise KeyError(name)


def kernel_names():
    return [gemm_kernel_name(i) for i in range(gemm_kernel_count())]


# ---- tensor-level call -----------------------------------------------------

def _current_raw_stream(dev: int) -> int:
    get = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if get is not None:
        return get(dev)
    return torch.cuda.current_stream(dev).cuda_stream


def _ld(t: torch.Tensor) -> int:
    rows, cols = t.shape
    if rows > 1 and cols > 0:
        return t.stride(0)
    return max(cols, 1)


def gemm(a: torch.Tensor, b: torch.Tensor, out: Optional[torch.Tensor] = None,
         stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """out = a @ b for 2-D device tensors (fp32·fp32 or bf16·bf16 -> fp32).

    Rows may be padded (any row stride), columns must be unit-stride.  The
    call is asynchronous on `stream` (default: the current stream of a's
    device)."""
    if a.dim() != 2 or b.dim() != 2:
        raise ValueError("gemm takes 2-D tensors")
    if a.dtype != b.dtype or a.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"operands must both be float32 or both bfloat16, got {a.dtype}, {b.dtype}")
    if a.device.type != "cuda" or b.device != a.device:
        raise ValueError("operands must be on the same GPU")
    M, K = a.shape
    K2, N = b.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {tuple(a.shape)} @ {tuple(b.shape)}")
    for name, t in (("a", a), ("b", b)):
        if t.shape[1] > 1 and t.stride(1) != 1:
            raise ValueError(f"{name} must have unit column stride")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a.device)
    elif (out.dtype != torch.float32 or out.shape != (M, N) or out.device != a.device
          or (N > 1 and out.stride(1) != 1)):
        raise ValueError("out must be a float32 (M, N) tensor with unit column stride on a's GPU")
    fn = lib.gemm_f32 if a.dtype == torch.float32 else lib.gemm_bf16_f32acc
    dev = a.get_device()
    # The raw handle of the current stream, without building a Stream object
    # (a few microseconds per call, which is the whole kernel time of the
    # smallest products).
    raw = stream.cuda_stream if stream is not None else _current_raw_stream(dev)
    # The library launches on the calling thread's current HIP device.
    if dev != torch.cuda.current_device():
        with torch.cuda.device(dev):
            rc = fn(M, N, K, a.data_ptr(), _ld(a), b.data_ptr(), _ld(b),
                    out.data_ptr(), _ld(out), raw)
    else:
        rc = fn(M, N, K, a.data_ptr(), _ld(a), b.data_ptr(), _ld(b),
                out.data_ptr(), _ld(out), raw)
    if rc != HIP_SUCCESS:
        raise GemmError(rc, "gemm_f32" if a.dtype == torch.float32 else "gemm_bf16_f32acc")
    return out
