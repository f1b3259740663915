"""GPU parity of the fused attention forward (attention_fwd_f32) against the
fp64 attention oracle, through the C-ABI.

The gate is the normalized error max |o - o_ref| / sum_j p_ij |v_jc| <=
5e-4 on every output element (the same bound the matrix products meet,
divided by the scale of the output's rounding error) and |lse - lse_ref| /
max(1, sm) <= 5e-4 on the log-sum-exp, sm being the softmax-weighted
magnitude of the scores (the scale of their fp32 rounding error).  Exact
checks where the arithmetic is exact: a key whose score dominates by more
than fp32's exponent range must give its value row bit for bit, and a
single visible key (the first query under the causal mask) its own value
row.  Shapes: the GPT's attention read in place from its QKV projection
buffer (64 sequences, 6 heads of 64, context 256, with and without the
causal mask), the context-2048 case, one sequence of the GPT (where the
keys are split over the waves), head width 128, and ragged lengths around
the 128- and 32-query and 64- and 32-key tiles, each on both kernels.
"""
import math
import sys

import numpy as np
import pytest
import torch

import dense_gemm_17_amd as g
import workloads
from oracle import attention as att

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GATE = 5e-4


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class Forced:
    """Force one of the attention kernels (0: 128-query tiles, 1: keys split
    over the waves of 32-query work-groups) for the calls inside."""

    def __init__(self, variant):
        self.variant = variant

    def __enter__(self):
        assert g.attention_force_kernel(self.variant) == 0

    def __exit__(self, *exc):
        g.attention_force_kernel(-1)


def check(q, k, v, causal, scale=None, name="", variant=-1):
    """Run the kernel on CPU tensors q, k, v (B, H, S, D), compare with the
    oracle; returns the GPU output."""
    B, H, S, D = q.shape
    sc = 1.0 / math.sqrt(D) if scale is None else scale
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    lse = torch.full((B, H, S), float("nan"), device=DEV)
    with Forced(variant):
        O = g.attention(qd, kd, vd, causal=causal, scale=sc, lse=lse)
        O2 = g.attention(qd, kd, vd, causal=causal, scale=sc)
    torch.cuda.synchronize()
    if variant >= 0 and D == 64:
        assert g.attention_last_kernel() == variant
    assert torch.equal(O, O2), "not deterministic"
    Oref, DN, Lref, SM = att.attention_fwd(q.numpy(), k.numpy(), v.numpy(), causal, sc)
    e, at = att.normalized_error(O.cpu().numpy(), Oref, DN)
    el = att.lse_error(lse.cpu().numpy(), Lref, SM)
    say(f"[attn] {name} B={B} H={H} S={S} D={D} causal={causal} kernel={g.attention_last_kernel()} "
        f"e={e:.3e} at={at} lse_err={el:.3e}")
    assert e <= GATE, f"normalized error {e} at {at}"
    assert el <= GATE, f"log-sum-exp error {el}"
    return O


def rand(shape, seed, scale=1.0):
    return torch.randn(shape, generator=workloads.generator(seed)) * scale


@pytest.mark.parametrize("name", list(workloads.ATTENTION_WORKLOADS))
def test_workloads_in_place_from_qkv_buffer(name):
    w = workloads.ATTENTION_WORKLOADS[name]
    qkv = workloads.make_attention_qkv(w)
    Q, K, V = workloads.attention_views(w, qkv)
    qkvd = qkv.to(DEV)
    Qd, Kd, Vd = workloads.attention_views(w, qkvd)
    # output token-major (B*S) x (H*D), as the next projection reads it
    out = torch.full((w.B * w.S, w.H * w.D), float("nan"), device=DEV)
    Od = out.view(w.B, w.S, w.H, w.D).permute(0, 2, 1, 3)
    lse = torch.empty((w.B, w.H, w.S), device=DEV)
    g.attention(Qd, Kd, Vd, causal=w.causal, scale=w.scale, out=Od, lse=lse)
    torch.cuda.synchronize()
    Oref, DN, Lref, SM = att.attention_fwd(Q.numpy(), K.numpy(), V.numpy(), w.causal, w.scale)
    e, at = att.normalized_error(Od.cpu().numpy(), Oref, DN)
    el = att.lse_error(lse.cpu().numpy(), Lref, SM)
    say(f"[attn] {name} e={e:.3e} at={at} lse_err={el:.3e}")
    assert e <= GATE and el <= GATE


@pytest.mark.parametrize("S", [1, 2, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 200, 257, 385])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("variant", [0, 1, 2])
def test_ragged_lengths(S, causal, variant):
    B, H, D = 2, 3, 64
    check(rand((B, H, S, D), S), rand((B, H, S, D), S + 1000), rand((B, H, S, D), S + 2000),
          causal, name=f"ragged S={S}", variant=variant)


@pytest.mark.parametrize("causal", [False, True])
def test_single_sequence_default_kernel(causal):
    # one sequence of the GPT (6 heads, 256 tokens): too few 128-query
    # work-groups, so the table splits the keys over the waves
    B, H, S, D = 1, 6, 256, 64
    check(rand((B, H, S, D), 81), rand((B, H, S, D), 82), rand((B, H, S, D), 83), causal,
          name="one sequence")
    assert g.attention_last_kernel() == 1
    check(rand((B, H, 2048, D), 84), rand((B, H, 2048, D), 85), rand((B, H, 2048, D), 86), causal,
          name="one sequence of 2048", variant=1)


@pytest.mark.parametrize("S,want", [(256, 2), (128, 2), (384, 0), (1024, 0)])
def test_default_kernel_by_length(S, want):
    # enough work-groups for the CUs: 32-key tiles up to 256 tokens, 64-key
    # tiles beyond
    H, D = 6, 64
    B = -(-256 // (-(-S // 128) * H))          # 128-query work-groups >= CUs
    assert g.attention_force_kernel(-1) == 0
    check(rand((B, H, S, D), S + 90), rand((B, H, S, D), S + 91), rand((B, H, S, D), S + 92), True,
          name=f"default S={S}")
    assert g.attention_last_kernel() == want


@pytest.mark.parametrize("S", [1, 33, 96, 128, 130, 300])
@pytest.mark.parametrize("causal", [False, True])
def test_head_width_128(S, causal):
    B, H, D = 2, 2, 128
    check(rand((B, H, S, D), S + 7), rand((B, H, S, D), S + 1007), rand((B, H, S, D), S + 2007),
          causal, name=f"D=128 S={S}")


@pytest.mark.parametrize("variant", [0, 1, 2])
def test_large_scores_and_scale(variant):
    # scores of order 1000, far past fp32's exponential range: the running
    # maximum keeps every exponential finite
    B, H, S, D = 1, 2, 300, 64
    check(rand((B, H, S, D), 1, 10.0), rand((B, H, S, D), 2, 10.0), rand((B, H, S, D), 3),
          True, scale=1.0, name="large scores", variant=variant)
    check(rand((B, H, S, D), 1, 2.0), rand((B, H, S, D), 2, 2.0), rand((B, H, S, D), 3),
          False, scale=1.0, name="scores of order 30", variant=variant)
    check(rand((B, H, S, D), 4), rand((B, H, S, D), 5), rand((B, H, S, D), 6), False,
          scale=0.01, name="flat scores", variant=variant)


@pytest.mark.parametrize("variant", [0, 1, 2])
def test_dominant_key_is_exact(variant):
    # key j* scores 2^10 above every other key: every other exponential is
    # exactly 0 in fp32, so the output is the value row of j*, bit for bit
    B, H, S, D = 1, 1, 200, 64
    jstar = 77
    q = torch.zeros((B, H, S, D))
    k = torch.zeros((B, H, S, D))
    q[..., 0] = 1.0
    k[0, 0, jstar, 0] = 8192.0                 # scale 1/8: score 1024
    v = rand((B, H, S, D), 7)
    with Forced(variant):
        O = g.attention(q.to(DEV), k.to(DEV), v.to(DEV), causal=False, scale=0.125)
        torch.cuda.synchronize()
        assert torch.equal(O.cpu()[0, 0], v[0, 0, jstar].expand(S, D))
        Oc = g.attention(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, scale=0.125).cpu()
    # causal: queries from j* on see it; query 0 sees only key 0
    assert torch.equal(Oc[0, 0, jstar:], v[0, 0, jstar].expand(S - jstar, D))
    assert torch.equal(Oc[0, 0, 0], v[0, 0, 0])


@pytest.mark.parametrize("variant", [0, 1, 2])
def test_uniform_scores_give_the_mean(variant):
    B, H, S, D = 2, 2, 150, 64
    q = torch.zeros((B, H, S, D))
    k, v = rand((B, H, S, D), 8), rand((B, H, S, D), 9)
    O = check(q, k, v, True, name="uniform causal", variant=variant)
    mean = torch.cumsum(v.double(), dim=2) / torch.arange(1, S + 1).double().view(1, 1, S, 1)
    assert torch.allclose(O.cpu().double(), mean, rtol=0, atol=1e-5)


def test_key_value_permutation():
    # without the mask, permuting keys and values together leaves the output
    # unchanged up to the order of the sums
    B, H, S, D = 1, 2, 160, 64
    q, k, v = rand((B, H, S, D), 10), rand((B, H, S, D), 11), rand((B, H, S, D), 12)
    perm = torch.randperm(S, generator=workloads.generator(13))
    for variant in (0, 1, 2):
        O1 = check(q, k, v, False, name="perm a", variant=variant)
        O2 = check(q, k[:, :, perm], v[:, :, perm], False, name="perm b", variant=variant)
        assert torch.allclose(O1, O2, rtol=0, atol=1e-5)


def test_refused_arguments():
    B, H, S, D = 1, 1, 8, 64
    x = torch.zeros((B, H, S, D), device=DEV)
    o = torch.zeros((B, H, S, D), device=DEV)
    st = torch.cuda.current_stream().cuda_stream

    def call(D_=D, causal=1, scale=0.125, q=x, o_=o, qs=(S * D, S * D, D), os_=(S * D, S * D, D),
             lse=None):
        args = [B, H, S, D_, causal, scale, q.data_ptr(), *qs, x.data_ptr(), S * D, S * D, D,
                x.data_ptr(), S * D, S * D, D, o_.data_ptr(), *os_,
                lse.data_ptr() if lse is not None else None, st]
        return g.attention_fwd_f32(*args)

    assert call() == 0
    assert call(D_=96) != 0                      # head width not built
    assert call(causal=2) != 0
    assert call(scale=float("nan")) != 0 and call(scale=float("inf")) != 0
    assert call(o_=x) != 0                       # output over an input
    assert call(qs=(S * D, S * D, 2)) != 0       # stride not a multiple of 4
    assert call(os_=(0, 0, 0)) != 0 or S == 1    # output rows on top of each other
    xb = torch.zeros(B * H * S * D + 4, device=DEV)
    assert call(q=xb[1:]) != 0                   # misaligned
    lse = torch.zeros((B, H, S), device=DEV)
    assert call(lse=lse) == 0
    torch.cuda.synchronize()
    assert g.attention_fwd_f32(0, H, S, D, 1, 0.1, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0,
                               None, st) == 0    # empty: nothing to do
