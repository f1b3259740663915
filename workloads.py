"""Seeded synthetic inputs for the GEMM workloads.

This module is shared by the tests, the smoke check and the benchmark, on both
sides of the parity check (HIP library and CPU oracle).  It draws operands and
holds none of the product's arithmetic.

Recipe (every workload): one CPU ``torch.Generator`` seeded with 1234 — the
seed the hackathon write-up on devpost ("Tools") gives for its synthetic
tensors — draws A first, then B, in fp32:
  * ``uniform``   rand * 2 - 1            (i.i.d. on [-1, 1))
  * ``normal``    randn * sigma
  * bf16 inputs   the fp32 draw rounded to bf16 (round to nearest even)
The same bytes are copied to the GPU and handed to the oracle.

Workload sizes come from the pages' subject: square 4096 and 8192 products
(the kernel ladder of "Bare Metal Bard", page 1, first paragraph), the
projection shapes of the 10.8M-parameter, 6-layer, d_model 384 character GPT
of the same page (second paragraph) at 16384 tokens, and skinny or ragged
shapes that exercise the launch- and bandwidth-bound regimes that the devpost
write-up ("What we built") routes through a dispatch table.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, List, Tuple

import torch

SEED = 1234


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dtype: str                    # "f32", "bf16" or "f16" (inputs); output is always fp32
    dist_a: Tuple[str, float] = ("uniform", 1.0)
    dist_b: Tuple[str, float] = ("uniform", 1.0)
    note: str = ""

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def in_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def algorithmic_bytes(self) -> int:
        """Each operand read once and C written once."""
        s = self.in_bytes
        return s * (self.M * self.K + self.K * self.N) + 4 * self.M * self.N


_ACT = ("normal", 1.0)      # GPT activations
_WGT = ("normal", 0.02)     # GPT weights

WORKLOADS: Dict[str, Workload] = {w.name: w for w in [
    Workload("f32_256", 256, 256, 256, "f32", note="small square; oracle in well under a second"),
    Workload("f32_4096", 4096, 4096, 4096, "f32", note="square fp32"),
    Workload("f32_8192", 8192, 8192, 8192, "f32", note="square fp32 at the headline size"),
    Workload("gpt_qkv", 16384, 1152, 384, "f32", _ACT, _WGT, note="GPT QKV projection"),
    Workload("gpt_mlp_up", 16384, 1536, 384, "f32", _ACT, _WGT, note="GPT MLP up"),
    Workload("gpt_mlp_down", 16384, 384, 1536, "f32", _ACT, _WGT, note="GPT MLP down"),
    Workload("bf16_8192", 8192, 8192, 8192, "bf16", ("normal", 1.0), ("normal", 1.0),
             note="bf16 in / fp32 accumulate at the headline size"),
    Workload("skinny_1x8960x1536", 1, 8960, 1536, "f32", note="one-row product (decode-like)"),
    Workload("skinny_7x4096x4096", 7, 4096, 4096, "f32", note="seven-row product"),
    Workload("ragged_1000x3000x777", 1000, 3000, 777, "f32", note="ragged, K not a multiple of 4"),
    Workload("ragged_4097x4095x1023", 4097, 4095, 1023, "f32", note="ragged in every dimension"),
    # beyond the listed configurations: the GPT projections in bf16 (the same
    # draws rounded), where 256 x 256 tiles leave CUs idle
    Workload("bf16_gpt_qkv", 16384, 1152, 384, "bf16", _ACT, _WGT,
             note="GPT QKV projection, bf16 operands"),
    Workload("bf16_gpt_mlp_down", 16384, 384, 1536, "bf16", _ACT, _WGT,
             note="GPT MLP down, bf16 operands"),
    # fp16 operands (the same draws rounded to binary16) at the headline size
    Workload("f16_8192", 8192, 8192, 8192, "f16", ("normal", 1.0), ("normal", 1.0),
             note="fp16 in / fp32 accumulate at the headline size"),
]}

# Groups of the workload list as the parity tests and the benchmark use them.
PARITY_WORKLOADS: List[str] = [
    "f32_256", "f32_4096", "gpt_qkv", "gpt_mlp_up", "gpt_mlp_down", "bf16_8192",
    "skinny_1x8960x1536", "skinny_7x4096x4096", "ragged_1000x3000x777",
    "ragged_4097x4095x1023", "f32_8192",
]


# Operand types: fp32, and bf16 or fp16 rounded from the fp32 draw (round to
# nearest even); the output is fp32 for all three.
TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def generator(seed: int = SEED) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def draw(shape, dist: Tuple[str, float], g: torch.Generator) -> torch.Tensor:
    kind, scale = dist
    if kind == "uniform":
        return torch.rand(shape, generator=g, dtype=torch.float32) * 2.0 - 1.0
    if kind == "normal":
        return torch.randn(shape, generator=g, dtype=torch.float32) * scale
    raise ValueError(f"unknown distribution {kind!r}")


def make_inputs(w: Workload, seed: int = SEED) -> Tuple[torch.Tensor, torch.Tensor]:
    """CPU tensors (A, B): fp32, or bf16 rounded from the fp32 draw."""
    g = generator(seed)
    A = draw((w.M, w.K), w.dist_a, g)
    B = draw((w.K, w.N), w.dist_b, g)
    return A.to(TORCH_DTYPE[w.dtype]), B.to(TORCH_DTYPE[w.dtype])


def small_int(shape, lo: int, hi: int, g: torch.Generator, dtype=torch.float32) -> torch.Tensor:
    """Integer-valued entries in [lo, hi], exactly representable in fp32/bf16."""
    return torch.randint(lo, hi + 1, shape, generator=g).to(dtype)


def bf16_bits(t: torch.Tensor):
    """Raw bf16 patterns of a CPU bf16 tensor as a numpy uint16 array."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view("uint16")


def as_numpy_operand(t: torch.Tensor):
    """numpy view of a CPU operand in the form the oracle takes."""
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    return t.contiguous().numpy()


# ---- transposed factors and strided batches --------------------------------
# The backward pass of the same GPT (gradients are products with one factor
# stored transposed: the input gradient dX = dY W^T reads the weight as
# stored, the weight gradient dW = X^T dY the activations as stored) and its
# attention (6 heads of width 64 over a context of 256, 64 sequences: 384
# per-head products).  Each product's operands are drawn in their stored
# layout, A first, then B, from the same seeded generator.


@dataclass(frozen=True)
class GeneralWorkload:
    name: str
    batch: int
    M: int
    N: int
    K: int
    ta: bool                      # A stored K x M
    tb: bool                      # B stored N x K
    dtype: str
    dist_a: Tuple[str, float] = ("normal", 1.0)
    dist_b: Tuple[str, float] = ("normal", 1.0)
    note: str = ""

    @property
    def flops(self) -> int:
        return 2 * self.batch * self.M * self.N * self.K

    @property
    def in_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def algorithmic_bytes(self) -> int:
        s = self.in_bytes
        return self.batch * (s * (self.M * self.K + self.K * self.N) + 4 * self.M * self.N)


GENERAL_WORKLOADS: Dict[str, GeneralWorkload] = {w.name: w for w in [
    GeneralWorkload("gpt_qkv_dx", 1, 16384, 384, 1152, False, True, "f32", _ACT, _WGT,
                    note="QKV input gradient dY W^T"),
    GeneralWorkload("gpt_qkv_dw", 1, 384, 1152, 16384, True, False, "f32", _ACT, _ACT,
                    note="QKV weight gradient X^T dY"),
    GeneralWorkload("gpt_mlp_down_dx", 1, 16384, 1536, 384, False, True, "f32", _ACT, _WGT,
                    note="MLP-down input gradient dY W^T"),
    GeneralWorkload("attn_scores", 384, 256, 256, 64, False, True, "f32",
                    note="per-head scores Q K^T"),
    GeneralWorkload("attn_pv", 384, 256, 64, 256, False, False, "f32",
                    note="per-head probabilities times values"),
    GeneralWorkload("bf16_gpt_qkv_dw", 1, 384, 1152, 16384, True, False, "bf16", _ACT, _ACT,
                    note="QKV weight gradient, bf16 operands"),
    GeneralWorkload("bf16_attn_scores", 384, 256, 256, 64, False, True, "bf16",
                    note="per-head scores, bf16 operands"),
]}


def make_general_inputs(w: GeneralWorkload, seed: int = SEED) -> Tuple[torch.Tensor, torch.Tensor]:
    """CPU tensors (A, B) in their stored layouts: A is (batch,) M x K or
    K x M when transposed, B is (batch,) K x N or N x K; 2-D when batch is 1."""
    g = generator(seed)
    lead = (w.batch,) if w.batch > 1 else ()
    A = draw(lead + ((w.K, w.M) if w.ta else (w.M, w.K)), w.dist_a, g)
    B = draw(lead + ((w.N, w.K) if w.tb else (w.K, w.N)), w.dist_b, g)
    return A.to(TORCH_DTYPE[w.dtype]), B.to(TORCH_DTYPE[w.dtype])


def general_views(w: GeneralWorkload, A: torch.Tensor, B: torch.Tensor):
    """The logical factors op(A), op(B) as views of the stored tensors."""
    return (A.transpose(-1, -2) if w.ta else A), (B.transpose(-1, -2) if w.tb else B)


# ---- a launch-bound sequence ------------------------------------------------
# The matrix products of one forward pass of the same GPT over a single
# sequence of 256 tokens (6 layers; per layer the QKV projection, the
# per-head scores Q K^T and probabilities x values over 6 heads of width 64,
# the attention output projection, MLP up and MLP down; then the output
# layer onto the 65-character vocabulary): 37 calls of at most 0.3 GFLOP
# each, the regime where the launches, not the kernels, set the time.
# Entries: (name, batch, M, N, K, A stored transposed, B stored transposed).
def gpt_forward_sequence(tokens: int = 256, layers: int = 6, d_model: int = 384,
                         heads: int = 6, vocab: int = 65):
    dh = d_model // heads
    seq = []
    for l in range(layers):
        seq += [(f"l{l}_qkv", 1, tokens, 3 * d_model, d_model, False, False),
                (f"l{l}_scores", heads, tokens, tokens, dh, False, True),
                (f"l{l}_pv", heads, tokens, dh, tokens, False, False),
                (f"l{l}_proj", 1, tokens, d_model, d_model, False, False),
                (f"l{l}_mlp_up", 1, tokens, 4 * d_model, d_model, False, False),
                (f"l{l}_mlp_down", 1, tokens, d_model, 4 * d_model, False, False)]
    seq.append(("lm_head", 1, tokens, vocab, d_model, False, False))
    return seq


# ---- 8-bit float operands ------------------------------------------------------
# Products with OCP 8-bit float operands (e4m3 / e5m2), the weight stored
# output-major (N x K), as FP8 inference keeps it.  The fp32 draws are
# rounded to the format (round to nearest even, saturating to the largest
# finite value where torch's conversion does): N(0, 1) activations and
# weights, well inside both formats' range.
FP8_TORCH = {0: torch.float8_e4m3fn, 1: torch.float8_e5m2}


@dataclass(frozen=True)
class Fp8Workload:
    name: str
    M: int
    N: int
    K: int
    fa: int                       # format of A: 0 e4m3, 1 e5m2
    fb: int                       # format of B
    batch: int = 1
    note: str = ""
    dtype: str = "fp8"

    @property
    def flops(self) -> int:
        return 2 * self.batch * self.M * self.N * self.K

    @property
    def algorithmic_bytes(self) -> int:
        """Each operand read once (1 byte per element), C written once (fp32)."""
        return self.batch * (self.M * self.K + self.N * self.K + 4 * self.M * self.N)


FP8_WORKLOADS: Dict[str, Fp8Workload] = {w.name: w for w in [
    Fp8Workload("fp8_e4m3_8192", 8192, 8192, 8192, 0, 0,
                note="e4m3 x e4m3 at the headline size"),
    Fp8Workload("fp8_e5m2_e4m3_8192", 8192, 8192, 8192, 1, 0,
                note="e5m2 x e4m3 (gradient x weight pairing) at the headline size"),
    Fp8Workload("fp8_gpt_qkv", 16384, 1152, 384, 0, 0, note="GPT QKV projection, e4m3"),
    Fp8Workload("fp8_gpt_mlp_down", 16384, 384, 1536, 0, 0, note="GPT MLP down, e4m3"),
    Fp8Workload("fp8_skinny_1x8960x1536", 1, 8960, 1536, 0, 0,
                note="one-row product through e4m3 weights (decode-like)"),
    Fp8Workload("fp8_skinny_4x8192x8192", 4, 8192, 8192, 0, 0,
                note="four-row product through e4m3 weights"),
    Fp8Workload("fp8_skinny_16x8192x8192", 16, 8192, 8192, 0, 0,
                note="sixteen-row product through e4m3 weights"),
]}


def make_fp8_inputs(w: Fp8Workload, seed: int = SEED) -> Tuple[torch.Tensor, torch.Tensor]:
    """CPU tensors (A, Bt): A (batch, M, K) or (M, K) and Bt (N, K), the
    transposed right factor, as 8-bit floats rounded from N(0, 1) draws."""
    g = generator(seed)
    shape_a = (w.batch, w.M, w.K) if w.batch > 1 else (w.M, w.K)
    A = draw(shape_a, ("normal", 1.0), g).to(FP8_TORCH[w.fa])
    Bt = draw((w.N, w.K), ("normal", 1.0), g).to(FP8_TORCH[w.fb])
    return A, Bt


def fp8_bits(t: torch.Tensor):
    """Raw 8-bit patterns of a CPU 8-bit float tensor as a numpy uint8 array."""
    return t.contiguous().view(torch.uint8).numpy()


# ---- fused attention forward ---------------------------------------------------
# The GPT's attention ("Bare Metal Bard", page 1, second and third paragraphs:
# 6 heads of width 64 over a context of 256, 64 sequences; the fused kernel
# let the same model train at a context of 2048).  Q, K and V are read where
# the QKV projection leaves them: one (B*S) x (3*H*D) fp32 buffer, token-major,
# the Q block of each token's row first, then K, then V, each H heads of D;
# the output is written token-major, (B*S) x (H*D), as the attention output
# projection reads it.  Entries are N(0, 1): with the 1/sqrt(D) scale the
# scores are of order one, so the softmax is neither flat nor one-hot.


@dataclass(frozen=True)
class AttentionWorkload:
    name: str
    B: int
    H: int
    S: int
    D: int
    causal: bool
    note: str = ""
    dtype: str = "f32"

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def pairs(self) -> int:
        """(query, key) pairs scored per head: S^2, or S(S+1)/2 with the
        causal mask."""
        return self.S * (self.S + 1) // 2 if self.causal else self.S * self.S

    @property
    def flops(self) -> int:
        """Two products per scored pair, each of D multiply-adds: 4 D flops
        per pair (the exponentials are not counted)."""
        return 4 * self.B * self.H * self.pairs * self.D

    @property
    def algorithmic_bytes(self) -> int:
        """Q, K, V read once, O written once (fp32), plus the log-sum-exp."""
        return 4 * self.B * self.H * self.S * (4 * self.D + 1)


ATTENTION_WORKLOADS: Dict[str, AttentionWorkload] = {w.name: w for w in [
    AttentionWorkload("attn_gpt_causal", 64, 6, 256, 64, True,
                      note="the GPT's attention: 64 sequences, 6 heads of 64, context 256"),
    AttentionWorkload("attn_gpt_full", 64, 6, 256, 64, False,
                      note="the same without the causal mask"),
    AttentionWorkload("attn_2048_causal", 8, 6, 2048, 64, True,
                      note="context 2048, 8 sequences"),
]}


def make_attention_qkv(w: AttentionWorkload, seed: int = SEED) -> torch.Tensor:
    """The QKV projection's output, (B*S) x (3*H*D) fp32, N(0, 1)."""
    return draw((w.B * w.S, 3 * w.H * w.D), ("normal", 1.0), generator(seed))


def attention_views(w: AttentionWorkload, qkv: torch.Tensor):
    """Q, K, V as (B, H, S, D) views of the projection buffer (no copy)."""
    t = qkv.view(w.B, w.S, 3, w.H, w.D)
    return tuple(t[:, :, i].permute(0, 2, 1, 3) for i in range(3))
