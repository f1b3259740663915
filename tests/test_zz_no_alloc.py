"""The no-allocation entry point (gemm_batched_noalloc) against the one it
varies (gemm_*_batched_ws with a caller's workspace), through the C-ABI.

Both split K over work-groups the same way, so their outputs must agree bit
for bit; both are also held to the oracle's 5e-4 gate.  Two calls in a row
on each element type, the second with a smaller product, check that the
library's fixed scratch array carries nothing from one call into the next;
a third call splits nothing and must equal the plain batched call.
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
CODE = {"f32": g.F32, "bf16": g.BF16, "f16": g.F16}
WS_FN = {"f32": g.lib.gemm_f32_batched_ws, "bf16": g.lib.gemm_bf16_f32acc_batched_ws,
         "f16": g.lib.gemm_f16_f32acc_batched_ws}
PLAIN_FN = {"f32": g.lib.gemm_f32_batched, "bf16": g.lib.gemm_bf16_f32acc_batched,
            "f16": g.lib.gemm_f16_f32acc_batched}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def operands(dtype, M, N, K, seed):
    """A weight gradient X^T dY: X stored K x M (A transposed), dY stored
    K x N (B as written)."""
    gen = workloads.generator(seed)
    X = workloads.draw((K, M), ("normal", 1.0), gen).to(workloads.TORCH_DTYPE[dtype])
    dY = workloads.draw((K, N), ("normal", 1.0), gen).to(workloads.TORCH_DTYPE[dtype])
    return X, dY


def call(fn_kind, dtype, M, N, K, Xd, dYd, C, ws=None):
    stream = torch.cuda.current_stream().cuda_stream
    args = (1, 0, M, N, K, Xd.data_ptr(), M, M * K, dYd.data_ptr(), N, K * N,
            C.data_ptr(), N, M * N, 1)
    if fn_kind == "noalloc":
        rc = g.lib.gemm_batched_noalloc(CODE[dtype], *args, stream)
    elif fn_kind == "ws":
        rc = WS_FN[dtype](*args, ws.data_ptr(), ws.numel() * ws.element_size(), stream)
    else:
        rc = PLAIN_FN[dtype](*args, stream)
    assert rc == 0, f"{fn_kind} returned {rc}"


def oracle_check(dtype, X, dY, C):
    Cref, D = oracle.gemm_batched(workloads.as_numpy_operand(X), workloads.as_numpy_operand(dY),
                                  True, False)
    e, at, _ = oracle.normalized_error(C.cpu().numpy(), Cref, D)
    assert e <= oracle.GATE, f"normalized error {e} at {at}"
    return e


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_noalloc_matches_workspace_entry(dtype):
    # first the GPT's QKV weight gradient (384 x 1152 over 16384 tokens: a
    # 16-way split, 28 MB of partials), then a smaller product (256 x 384
    # over 4096: a 16-way split, 6 MB) whose partials overwrite only part of
    # the first call's
    for (M, N, K, seed) in [(384, 1152, 16384, 70), (256, 384, 4096, 71)]:
        ws_bytes = g.gemm_workspace_size(CODE[dtype], 1, 0, M, N, K, 1)
        assert 0 < ws_bytes <= 32 << 20
        X, dY = operands(dtype, M, N, K, seed)
        Xd, dYd = X.to(DEV), dY.to(DEV)
        C_no = torch.full((M, N), float("nan"), device=DEV)
        C_ws = torch.full((M, N), float("nan"), device=DEV)
        ws = torch.empty(ws_bytes // 4, dtype=torch.float32, device=DEV)
        say(f"[noalloc] {dtype} {M}x{N}x{K}")
        call("noalloc", dtype, M, N, K, Xd, dYd, C_no)
        call("ws", dtype, M, N, K, Xd, dYd, C_ws, ws)
        torch.cuda.synchronize()
        assert torch.equal(C_no, C_ws), "no-allocation call differs from the workspace call"
        e = oracle_check(dtype, X, dY, C_no)
        say(f"[noalloc] {dtype} {M}x{N}x{K} equal to the workspace call, e={e:.3e}")


def test_noalloc_without_split_is_the_plain_call():
    # 2048 x 2048 fills the CUs with 128 x 128 tiles: nothing is split and
    # the call is exactly the plain batched one
    M = N = 2048
    K = 512
    assert g.gemm_workspace_size(g.F32, 1, 0, M, N, K, 1) == 0
    X, dY = operands("f32", M, N, K, 72)
    Xd, dYd = X.to(DEV), dY.to(DEV)
    C_no = torch.full((M, N), float("nan"), device=DEV)
    C_pl = torch.full((M, N), float("nan"), device=DEV)
    call("noalloc", "f32", M, N, K, Xd, dYd, C_no)
    call("plain", "f32", M, N, K, Xd, dYd, C_pl)
    torch.cuda.synchronize()
    assert torch.equal(C_no, C_pl)


def test_noalloc_refuses_bad_arguments():
    stream = torch.cuda.current_stream().cuda_stream
    x = torch.zeros(64, device=DEV)
    # 8-bit floats have no workspace variant; negative sizes; null operands
    assert g.lib.gemm_batched_noalloc(g.FP8, 0, 1, 4, 4, 16, x.data_ptr(), 16, 0,
                                      x.data_ptr(), 16, 0, x.data_ptr(), 4, 0, 1, stream) != 0
    assert g.lib.gemm_batched_noalloc(g.F32, 0, 0, -1, 4, 4, x.data_ptr(), 4, 0,
                                      x.data_ptr(), 4, 0, x.data_ptr(), 4, 0, 1, stream) != 0
    assert g.lib.gemm_batched_noalloc(g.F32, 1, 0, 384, 1152, 16384, 0, 384, 0,
                                      x.data_ptr(), 1152, 0, x.data_ptr(), 1152, 0, 1,
                                      stream) != 0
