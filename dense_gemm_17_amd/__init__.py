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
# MI355GEMM_LIBRARY names another build of the same library (the host
# sanitizer build the CPU tests load); by default the in-tree one.
LIB_PATH = os.environ.get("MI355GEMM_LIBRARY") or os.path.join(_HERE, "libmi355gemm.so")

F32 = 0
BF16 = 1
F16 = 2
FP8 = 3
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
    for name in ("gemm_f32", "gemm_bf16_f32acc", "gemm_f16_f32acc"):
        getattr(lib, name).argtypes = sig
        getattr(lib, name).restype = ci
    bsig = [ci, ci, i64, i64, i64, vp, i64, i64, vp, i64, i64, vp, i64, i64, i64, vp]
    for name in ("gemm_f32_batched", "gemm_bf16_f32acc_batched", "gemm_f16_f32acc_batched"):
        getattr(lib, name).argtypes = bsig
        getattr(lib, name).restype = ci
    sz = ctypes.c_size_t
    wsig = bsig[:-1] + [vp, sz, vp]
    for name in ("gemm_f32_batched_ws", "gemm_bf16_f32acc_batched_ws",
                 "gemm_f16_f32acc_batched_ws"):
        getattr(lib, name).argtypes = wsig
        getattr(lib, name).restype = ci
    lib.gemm_fp8_f32acc.argtypes = [ci, ci] + sig
    lib.gemm_fp8_f32acc.restype = ci
    lib.gemm_fp8_f32acc_batched.argtypes = [ci, ci, i64, i64, i64, vp, i64, i64, vp, i64, i64,
                                            vp, i64, i64, i64, vp]
    lib.gemm_fp8_f32acc_batched.restype = ci
    lib.gemm_workspace_size.argtypes = [ci, ci, ci, i64, i64, i64, i64]
    lib.gemm_workspace_size.restype = sz
    lib.gemm_plan_batched.argtypes = [ci, ci, ci, i64, i64, i64, sz, i64, i64, sz, i64, i64,
                                      sz, i64, i64, i64]
    lib.gemm_plan_batched.restype = ci
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
    lib.gemm_null_launch.argtypes = [vp]
    lib.gemm_null_launch.restype = ci
    lib.gemm_mxfp8_f32acc.argtypes = [ci, ci, i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64,
                                      vp, i64, vp]
    lib.gemm_mxfp8_f32acc.restype = ci
    lib.gemm_plan_mxfp8.argtypes = [i64, i64, i64, sz, i64, sz, i64, sz, i64, sz, i64, sz, i64]
    lib.gemm_plan_mxfp8.restype = ci
    lib.attention_fwd_f32.argtypes = [i64, i64, i64, i64, ci, ctypes.c_float] + \
        [vp, i64, i64, i64] * 4 + [vp, vp]
    lib.attention_fwd_f32.restype = ci
    lib.attention_force_kernel.argtypes = [ci]
    lib.attention_force_kernel.restype = ci
    lib.attention_last_kernel.argtypes = []
    lib.attention_last_kernel.restype = ci
    lib.gemm_batched_noalloc.argtypes = [ci] + bsig
    lib.gemm_batched_noalloc.restype = ci
    return lib


lib = _load()

# Every symbol include/mi355gemm.h declares.
EXPORTS = ("gemm_f32", "gemm_bf16_f32acc", "gemm_f16_f32acc", "gemm_f32_batched",
           "gemm_bf16_f32acc_batched", "gemm_f16_f32acc_batched", "gemm_f32_batched_ws",
           "gemm_bf16_f32acc_batched_ws", "gemm_f16_f32acc_batched_ws", "gemm_fp8_f32acc",
           "gemm_fp8_f32acc_batched", "gemm_workspace_size",
           "gemm_kernel_count", "gemm_kernel_name", "gemm_kernel_dtype", "gemm_plan",
           "gemm_plan_batched", "gemm_force_kernel", "gemm_last_kernel", "gemm_build_info",
           "gemm_null_launch", "gemm_batched_noalloc", "attention_fwd_f32",
           "gemm_mxfp8_f32acc", "gemm_plan_mxfp8", "attention_force_kernel",
           "attention_last_kernel")


# ---- raw entry points (pointers and sizes, same names as the C-ABI) --------

def gemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream) -> int:
    return lib.gemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_bf16_f32acc(M, N, K, A, lda, B, ldb, C, ldc, stream) -> int:
    return lib.gemm_bf16_f32acc(M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_f16_f32acc(M, N, K, A, lda, B, ldb, C, ldc, stream) -> int:
    return lib.gemm_f16_f32acc(M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_fp8_f32acc(fmt_a, fmt_b, M, N, K, A, lda, Bt, ldb, C, ldc, stream) -> int:
    return lib.gemm_fp8_f32acc(fmt_a, fmt_b, M, N, K, A, lda, Bt, ldb, C, ldc, stream)


def gemm_fp8_f32acc_batched(fmt_a, fmt_b, M, N, K, A, lda, stride_a, Bt, ldb, stride_b, C, ldc,
                            stride_c, batch, stream) -> int:
    return lib.gemm_fp8_f32acc_batched(fmt_a, fmt_b, M, N, K, A, lda, stride_a, Bt, ldb,
                                       stride_b, C, ldc, stride_c, batch, stream)


def gemm_f16_f32acc_batched(transa, transb, M, N, K, A, lda, stride_a, B, ldb, stride_b, C,
                            ldc, stride_c, batch, stream) -> int:
    return lib.gemm_f16_f32acc_batched(transa, transb, M, N, K, A, lda, stride_a, B, ldb,
                                       stride_b, C, ldc, stride_c, batch, stream)


def gemm_f32_batched(transa, transb, M, N, K, A, lda, stride_a, B, ldb, stride_b, C, ldc,
                     stride_c, batch, stream) -> int:
    return lib.gemm_f32_batched(transa, transb, M, N, K, A, lda, stride_a, B, ldb, stride_b,
                                C, ldc, stride_c, batch, stream)


def gemm_bf16_f32acc_batched(transa, transb, M, N, K, A, lda, stride_a, B, ldb, stride_b, C,
                             ldc, stride_c, batch, stream) -> int:
    return lib.gemm_bf16_f32acc_batched(transa, transb, M, N, K, A, lda, stride_a, B, ldb,
                                        stride_b, C, ldc, stride_c, batch, stream)


def gemm_batched_noalloc(dtype, transa, transb, M, N, K, A, lda, stride_a, B, ldb, stride_b, C,
                         ldc, stride_c, batch, stream) -> int:
    return lib.gemm_batched_noalloc(dtype, transa, transb, M, N, K, A, lda, stride_a, B, ldb,
                                    stride_b, C, ldc, stride_c, batch, stream)


def gemm_workspace_size(dtype, transa, transb, M, N, K, batch=1) -> int:
    return lib.gemm_workspace_size(dtype, int(transa), int(transb), M, N, K, batch)


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


def gemm_plan_batched(dtype, transa, transb, M, N, K, batch, A=1 << 40, lda=None, stride_a=None,
                      B=2 << 40, ldb=None, stride_b=None, C=3 << 40, ldc=None,
                      stride_c=None) -> int:
    """gemm_plan for a batch of products with optionally transposed factors;
    unset leading dimensions and strides are those of packed storage."""
    lda = (M if transa else K) if lda is None else lda
    ldb = (K if transb else N) if ldb is None else ldb
    ldc = N if ldc is None else ldc
    stride_a = M * K if stride_a is None else stride_a
    stride_b = K * N if stride_b is None else stride_b
    stride_c = M * N if stride_c is None else stride_c
    return lib.gemm_plan_batched(dtype, int(transa), int(transb), M, N, K, A, lda, stride_a,
                                 B, ldb, stride_b, C, ldc, stride_c, batch)


def gemm_force_kernel(kid: int) -> int:
    return lib.gemm_force_kernel(kid)


def gemm_last_kernel() -> int:
    return lib.gemm_last_kernel()


def gemm_build_info() -> str:
    return lib.gemm_build_info().decode()


def gemm_null_launch(stream) -> int:
    return lib.gemm_null_launch(stream)


def gemm_mxfp8_f32acc(fmt_a, fmt_b, M, N, K, A, lda, scale_a, ld_scale_a, Bt, ldb, scale_b,
                      ld_scale_b, C, ldc, stream) -> int:
    return lib.gemm_mxfp8_f32acc(fmt_a, fmt_b, M, N, K, A, lda, scale_a, ld_scale_a, Bt, ldb,
                                 scale_b, ld_scale_b, C, ldc, stream)


def gemm_plan_mxfp8(M, N, K, A, lda, scale_a, ld_scale_a, Bt, ldb, scale_b, ld_scale_b, C,
                    ldc) -> int:
    return lib.gemm_plan_mxfp8(M, N, K, A, lda, scale_a, ld_scale_a, Bt, ldb, scale_b,
                               ld_scale_b, C, ldc)


def gemm_mx(a: torch.Tensor, scale_a: torch.Tensor, b: torch.Tensor, scale_b: torch.Tensor,
            out: Optional[torch.Tensor] = None,
            stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """out = (a with its MX block scales) @ (b with its MX block scales), fp32.

    a is an (M, K) 8-bit float tensor (e4m3 or e5m2) with unit stride along
    K; b is (K, N), the transposed view of a row-major (N, K) 8-bit tensor
    (``w.t()``).  scale_a is a uint8 (K/32, M') tensor, M' >= M, holding the
    E8M0 scale of block kb of row i at scale_a[kb, i]; scale_b likewise
    (K/32, N') for the rows of b's storage.  Rows of the scale tensors may be
    padded; their pitch (the width for a single row) is a multiple of 4."""
    if a.dtype not in FP8_FORMAT or b.dtype not in FP8_FORMAT:
        raise TypeError("operands must be float8_e4m3fn or float8_e5m2")
    if scale_a.dtype != torch.uint8 or scale_b.dtype != torch.uint8:
        raise TypeError("scales must be uint8 E8M0 patterns")
    M, K = a.shape
    K2, N = b.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {tuple(a.shape)} @ {tuple(b.shape)}")
    if (K > 1 and (a.stride(1) != 1 or b.stride(0) != 1)):
        raise ValueError("a needs unit stride along K and b must be a transposed row-major tensor")
    for t, n in ((scale_a, M), (scale_b, N)):
        if t.dim() != 2 or t.shape[0] != K // 32 or t.shape[1] < n or \
                (t.shape[1] > 1 and t.stride(1) != 1) or t.device != a.device:
            raise ValueError("scales must be (K/32, >= rows) uint8 tensors with unit column stride")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a.device)
    dev = a.get_device()
    raw = stream.cuda_stream if stream is not None else _current_raw_stream(dev)
    lda = a.stride(0) if M > 1 else max(K, 16)
    ldb = b.stride(1) if N > 1 else max(K, 16)
    lsa = scale_a.stride(0) if scale_a.shape[0] > 1 else scale_a.shape[1]
    lsb = scale_b.stride(0) if scale_b.shape[0] > 1 else scale_b.shape[1]
    _launch(lib.gemm_mxfp8_f32acc, "gemm_mxfp8_f32acc", dev,
            (FP8_FORMAT[a.dtype], FP8_FORMAT[b.dtype], M, N, K, a.data_ptr(), lda,
             scale_a.data_ptr(), lsa, b.data_ptr(), ldb, scale_b.data_ptr(), lsb, out.data_ptr(),
             _ld(out), raw))
    return out


def attention_fwd_f32(B, H, S, D, causal, scale, Q, q_sb, q_sh, q_ss, K, k_sb, k_sh, k_ss,
                      V, v_sb, v_sh, v_ss, O, o_sb, o_sh, o_ss, lse, stream) -> int:
    return lib.attention_fwd_f32(B, H, S, D, causal, scale, Q, q_sb, q_sh, q_ss, K, k_sb, k_sh,
                                 k_ss, V, v_sb, v_sh, v_ss, O, o_sb, o_sh, o_ss, lse, stream)


def attention_force_kernel(variant: int) -> int:
    return lib.attention_force_kernel(variant)


def attention_last_kernel() -> int:
    return lib.attention_last_kernel()


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = True,
              scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
              lse: Optional[torch.Tensor] = None,
              stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Fused attention forward: out = softmax(scale * q k^T [causal mask]) v
    per (sequence, head), fp32.  q, k, v and out are (B, H, S, D) float32
    tensors on one GPU with unit stride along D (views such as slices of a
    QKV projection buffer are read in place); scale defaults to 1/sqrt(D);
    lse, if given, is a contiguous (B, H, S) float32 tensor that receives
    log sum_j exp(s_ij).  Asynchronous on `stream` (default: the current
    stream of q's device)."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.float32 or t.dim() != 4 or t.device.type != "cuda":
            raise TypeError(f"{name} must be a 4-D float32 CUDA tensor")
        if t.shape != q.shape or t.device != q.device:
            raise ValueError("q, k and v must have one (B, H, S, D) shape on one GPU")
        if t.shape[3] > 1 and t.stride(3) != 1:
            raise ValueError(f"{name} needs unit stride along D")
    B, H, S, D = q.shape
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    if out is None:
        out = torch.empty((B, H, S, D), dtype=torch.float32, device=q.device)
    elif out.dtype != torch.float32 or out.shape != q.shape or out.device != q.device or \
            (D > 1 and out.stride(3) != 1):
        raise ValueError("out must be a float32 (B, H, S, D) tensor with unit stride along D")
    if lse is not None and (lse.dtype != torch.float32 or lse.shape != (B, H, S)
                            or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 (B, H, S) tensor on q's GPU")
    dev = q.get_device()
    raw = stream.cuda_stream if stream is not None else _current_raw_stream(dev)
    args = [B, H, S, D, int(bool(causal)), float(scale)]
    for t in (q, k, v, out):
        args += [t.data_ptr(), t.stride(0), t.stride(1), t.stride(2)]
    args += [lse.data_ptr() if lse is not None else None, raw]
    _launch(lib.attention_fwd_f32, "attention_fwd_f32", dev, args)
    return out


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


def _layout(t: torch.Tensor, name: str):
    """(transposed, leading dimension) of the last two dims of an operand: a
    unit stride along the columns is the stored layout, a unit stride along
    the rows is a transposed view (e.g. ``x.t()``)."""
    rows, cols = t.shape[-2], t.shape[-1]
    rs, cs = t.stride(-2), t.stride(-1)
    if rows == 0 or cols == 0:
        return False, max(cols, 1)
    if cols <= 1 or cs == 1:
        ld = rs if rows > 1 else max(cols, 1)
        if ld >= max(cols, 1):
            return False, ld
    if rows <= 1 or rs == 1:
        ld = cs if cols > 1 else max(rows, 1)
        if ld >= max(rows, 1):
            return True, ld
    raise ValueError(f"{name} needs a unit stride along its rows or its columns "
                     f"(got strides {tuple(t.stride())} for shape {tuple(t.shape)})")


# entry points (plain, batched) per operand type
_FN = {torch.float32: ("gemm_f32", "gemm_f32_batched"),
       torch.bfloat16: ("gemm_bf16_f32acc", "gemm_bf16_f32acc_batched"),
       torch.float16: ("gemm_f16_f32acc", "gemm_f16_f32acc_batched")}
_PLAIN = {dt: getattr(lib, names[0]) for dt, names in _FN.items()}
_CODE = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}
_BATCHED = {dt: getattr(lib, names[1]) for dt, names in _FN.items()}
# 8-bit float operand formats of gemm_fp8_f32acc*
FP8_FORMAT = {torch.float8_e4m3fn: 0, torch.float8_e5m2: 1}


def _batch_stride(t: torch.Tensor) -> int:
    return t.stride(0) if t.dim() == 3 and t.shape[0] > 1 else 0


def gemm(a: torch.Tensor, b: torch.Tensor, out: Optional[torch.Tensor] = None,
         stream: Optional[torch.cuda.Stream] = None,
         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out = a @ b on the GPU (fp32·fp32, bf16·bf16 or fp16·fp16 -> fp32, or
    8-bit floats: e4m3 / e5m2 in any pairing -> fp32).

    a is (M, K) or (batch, M, K), b is (K, N) or (batch, K, N); a 2-D operand
    is shared by every product of a batch, and a 3-D one may have any batch
    stride (0 included, as from ``expand``).  Each matrix needs a unit stride
    along its rows or its columns: rows may be padded, and a transposed view
    such as ``w.t()`` is read in place as a transposed factor.  The result is
    (M, N) for two 2-D operands, else (batch, M, N).  The call is asynchronous
    on `stream` (default: the current stream of a's device).  `workspace`
    (a device tensor of at least ``workspace_size(a, b)`` bytes) lets a
    single product with a small output split its K range over work-groups
    (the *_ws entry points); the caller keeps it alive until the stream has
    passed the call.  8-bit operands take one layout: a row-major, b the
    transposed view of a row-major (N, K) tensor (``w.t()``), K and the row
    pitches multiples of 16 bytes; they have no workspace variant."""
    if a.dtype in FP8_FORMAT or b.dtype in FP8_FORMAT:
        return _gemm_fp8(a, b, out, stream)
    if workspace is None and (a.dim() == 2 and b.dim() == 2 and (a.shape[1] <= 1 or a.stride(1) == 1)
                              and (b.shape[1] <= 1 or b.stride(1) == 1)):
        return _gemm_plain(a, b, out, stream)
    return _gemm_general(a, b, out, stream, workspace)


def workspace_size(a: torch.Tensor, b: torch.Tensor) -> int:
    """Bytes of workspace gemm(a, b, workspace=...) can use (0: none)."""
    if a.dim() != 2 or b.dim() != 2:
        return 0
    ta, _ = _layout(a, "a")
    tb, _ = _layout(b, "b")
    return gemm_workspace_size(_CODE[a.dtype], ta, tb, a.shape[0], b.shape[1], a.shape[1], 1)


def _check_operands(a, b):
    if a.dtype != b.dtype or a.dtype not in _FN:
        raise TypeError("operands must both be float32, both bfloat16 or both float16, "
                        f"got {a.dtype}, {b.dtype}")
    if a.device.type != "cuda" or b.device != a.device:
        raise ValueError("operands must be on the same GPU")


def _launch(fn, what, dev, args):
    # The library launches on the calling thread's current HIP device.
    if dev != torch.cuda.current_device():
        with torch.cuda.device(dev):
            rc = fn(*args)
    else:
        rc = fn(*args)
    if rc != HIP_SUCCESS:
        raise GemmError(rc, what)


def _gemm_plain(a, b, out, stream):
    """Two 2-D operands with unit column stride: the plain entry points (the
    short path: the smallest products take about as long as this call)."""
    _check_operands(a, b)
    M, K = a.shape
    K2, N = b.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {tuple(a.shape)} @ {tuple(b.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a.device)
    elif (out.dtype != torch.float32 or out.shape != (M, N) or out.device != a.device
          or (N > 1 and out.stride(1) != 1)):
        raise ValueError("out must be a float32 (M, N) tensor with unit column stride on a's GPU")
    dev = a.get_device()
    # The raw handle of the current stream, without building a Stream object
    # (a few microseconds per call, which is the whole kernel time of the
    # smallest products).
    raw = stream.cuda_stream if stream is not None else _current_raw_stream(dev)
    name = _FN[a.dtype][0]
    _launch(_PLAIN[a.dtype], name, dev,
            (M, N, K, a.data_ptr(), _ld(a), b.data_ptr(), _ld(b), out.data_ptr(), _ld(out), raw))
    return out


def _gemm_fp8(a, b, out, stream):
    """8-bit float operands: gemm_fp8_f32acc_batched (A as written, B
    transposed)."""
    if a.dtype not in FP8_FORMAT or b.dtype not in FP8_FORMAT:
        raise TypeError(f"8-bit operands must both be float8_e4m3fn or float8_e5m2, got "
                        f"{a.dtype}, {b.dtype}")
    if a.device.type != "cuda" or b.device != a.device:
        raise ValueError("operands must be on the same GPU")
    if a.dim() not in (2, 3) or b.dim() not in (2, 3):
        raise ValueError("gemm takes 2-D or 3-D tensors")
    M, K = a.shape[-2], a.shape[-1]
    K2, N = b.shape[-2], b.shape[-1]
    if K != K2:
        raise ValueError(f"inner dimensions differ: {tuple(a.shape)} @ {tuple(b.shape)}")
    if a.dim() == 3 and b.dim() == 3 and a.shape[0] != b.shape[0]:
        raise ValueError(f"batch sizes differ: {a.shape[0]} and {b.shape[0]}")
    # a: unit stride along K, rows lda bytes apart; b: the view of Bt (N x K)
    # with unit stride along K, rows of Bt ldb bytes apart.  A single row (or
    # K = 0) has no pitch of its own: a packed one is passed.
    if K > 1 and (a.stride(-1) != 1 or b.stride(-2) != 1):
        raise ValueError("8-bit operands: a must be row-major (M, K) and b the transposed view "
                         "of a row-major (N, K) tensor, e.g. w.t()")
    lda = a.stride(-2) if M > 1 else max(K, 16)
    ldb = b.stride(-1) if N > 1 else max(K, 16)
    if K == 0:
        lda = ldb = 16
    batched = a.dim() == 3 or b.dim() == 3
    batch = a.shape[0] if a.dim() == 3 else (b.shape[0] if b.dim() == 3 else 1)
    shape = (batch, M, N) if batched else (M, N)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=a.device)
    elif (out.dtype != torch.float32 or tuple(out.shape) != shape or out.device != a.device
          or (N > 1 and out.stride(-1) != 1)):
        raise ValueError(f"out must be a float32 {shape} tensor with unit column stride on a's GPU")
    ldc = out.stride(-2) if M > 1 else max(N, 1)
    dev = a.get_device()
    raw = stream.cuda_stream if stream is not None else _current_raw_stream(dev)
    _launch(lib.gemm_fp8_f32acc_batched, "gemm_fp8_f32acc_batched", dev,
            (FP8_FORMAT[a.dtype], FP8_FORMAT[b.dtype], M, N, K, a.data_ptr(), lda,
             _batch_stride(a), b.data_ptr(), ldb, _batch_stride(b), out.data_ptr(), ldc,
             _batch_stride(out), batch, raw))
    return out


def _gemm_general(a, b, out, stream, workspace=None):
    """Transposed views and batches: the *_batched entry points (*_ws with a
    workspace)."""
    if a.dim() not in (2, 3) or b.dim() not in (2, 3):
        raise ValueError("gemm takes 2-D or 3-D tensors")
    _check_operands(a, b)
    M, K = a.shape[-2], a.shape[-1]
    K2, N = b.shape[-2], b.shape[-1]
    if K != K2:
        raise ValueError(f"inner dimensions differ: {tuple(a.shape)} @ {tuple(b.shape)}")
    if a.dim() == 3 and b.dim() == 3 and a.shape[0] != b.shape[0]:
        raise ValueError(f"batch sizes differ: {a.shape[0]} and {b.shape[0]}")
    batched = a.dim() == 3 or b.dim() == 3
    batch = a.shape[0] if a.dim() == 3 else (b.shape[0] if b.dim() == 3 else 1)
    ta, lda = _layout(a, "a")
    tb, ldb = _layout(b, "b")
    shape = (batch, M, N) if batched else (M, N)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=a.device)
    elif (out.dtype != torch.float32 or tuple(out.shape) != shape or out.device != a.device
          or (N > 1 and out.stride(-1) != 1)):
        raise ValueError(f"out must be a float32 {shape} tensor with unit column stride on a's GPU")
    ldc = out.stride(-2) if M > 1 else max(N, 1)
    dev = a.get_device()
    raw = stream.cuda_stream if stream is not None else _current_raw_stream(dev)
    if workspace is not None:
        if workspace.device != a.device:
            raise ValueError("workspace must be on the operands' GPU")
        name = _FN[a.dtype][1] + "_ws"
        fn = getattr(lib, name)
        args = (int(ta), int(tb), M, N, K, a.data_ptr(), lda, _batch_stride(a), b.data_ptr(),
                ldb, _batch_stride(b), out.data_ptr(), ldc, _batch_stride(out), batch,
                workspace.data_ptr(), workspace.numel() * workspace.element_size(), raw)
    elif not batched and not ta and not tb:
        name, fn = _FN[a.dtype][0], _PLAIN[a.dtype]
        args = (M, N, K, a.data_ptr(), lda, b.data_ptr(), ldb, out.data_ptr(), ldc, raw)
    else:
        name, fn = _FN[a.dtype][1], _BATCHED[a.dtype]
        args = (int(ta), int(tb), M, N, K, a.data_ptr(), lda, _batch_stride(a), b.data_ptr(),
                ldb, _batch_stride(b), out.data_ptr(), ldc, _batch_stride(out), batch, raw)
    _launch(fn, name, dev, args)
    return out
