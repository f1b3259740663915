"""Attention forward, the plain definition in fp64 — TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module; the product path never does.

"Bare Metal Bard" (page 1, third paragraph) trains its GPT with a fused,
FlashAttention-style forward kernel: the score matrix is never stored, each
score tile stays in registers and a running maximum and sum are carried
from tile to tile.  That streaming form reaches, up to rounding, the plain
result of scaled dot-product attention, so this oracle is that definition
written out, one (sequence, head) at a time, with no tiling and no running
statistics:

    s_ij   = scale * sum_c q_ic k_jc        for keys j < S (j <= i if causal)
    p_ij   = exp(s_ij - max_j s_ij) / sum_j exp(s_ij - max_j s_ij)
    o_ic   = sum_j p_ij v_jc
    lse_i  = max_j s_ij + log sum_j exp(s_ij - max_j s_ij)   (= log sum_j e^{s_ij})

Causal masking (a key never after its query) is the reading for a GPT, a
decoder that predicts each character from the ones before it.  Beside the
output it returns the magnitude sum dn_ic = sum_j p_ij |v_jc|, the scale of
the output's rounding error that the correctness gate divides by, and the
weighted score magnitude sm_i = sum_j p_ij * |scale| * sum_c |q_ic k_jc|, the
scale of the rounding error of the scores and so of the log-sum-exp (a
score computed in fp32 is off by about D * 2^-24 of its magnitude sum).

fp32 inputs are widened to fp64 exactly; products of two fp32 values are
exact in fp64; numpy's fp64 matrix product serves as the inner-product step
and numpy's exp and log as the exponential and logarithm.  Pinned by
``tests/test_attention_oracle.py``: closed forms (uniform scores give the mean
of the visible values; one dominant key selects its value row; a single key
gives its value row and its score as lse; two keys give the logistic
weights), invariance under permuting the keys together with the values,
agreement with scipy's softmax and logsumexp, and brute force in plain
Python on tiny shapes; planted mistakes (``MUTANTS``) each fail a pin.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

# Planted mistakes for the oracle's own sensitivity tests (None: the oracle
# as written).  Set only by tests, on the CPU.
MUTANTS = ("NO_SCALE", "MASK_DIAGONAL", "SOFTMAX_OVER_QUERIES", "NO_MAX_SHIFT", "VALUES_FROM_K")
_mutant: Optional[str] = None


def plant(mutant: Optional[str]) -> None:
    global _mutant
    if mutant is not None and mutant not in MUTANTS:
        raise ValueError(f"unknown attention-oracle mutant {mutant!r}")
    _mutant = mutant


def _one_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool, scale: float):
    """One (sequence, head): q, k, v are S x D fp64.  Returns o, dn (S x D),
    lse and sm (S)."""
    S = q.shape[0]
    s = q @ k.T
    if _mutant != "NO_SCALE":
        s = s * scale
    if causal:
        j_after_i = np.triu(np.ones((S, S), dtype=bool), k=0 if _mutant == "MASK_DIAGONAL" else 1)
        s = np.where(j_after_i, -np.inf, s)
    axis = 0 if _mutant == "SOFTMAX_OVER_QUERIES" else 1
    m = np.max(s, axis=axis, keepdims=True)
    if _mutant == "NO_MAX_SHIFT":
        m = np.zeros_like(m)
    e = np.exp(s - m)
    l = np.sum(e, axis=axis, keepdims=True)
    p = e / l
    vv = k if _mutant == "VALUES_FROM_K" else v
    o = p @ vv
    dn = p @ np.abs(vv)
    lse = (m + np.log(l)).reshape(-1) if axis == 1 else np.full(S, np.nan)
    sm = np.sum(p * (abs(scale) * (np.abs(q) @ np.abs(k).T)), axis=1)
    return o, dn, lse, sm


def attention_fwd(Q: np.ndarray, K: np.ndarray, V: np.ndarray, causal: bool,
                  scale: float) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """Q, K, V: float32 arrays of shape (B, H, S, D) (any strides).  Returns
    (O, dn, lse, sm) in fp64: O and dn of shape (B, H, S, D), lse and sm
    (B, H, S)."""
    if not (Q.shape == K.shape == V.shape) or Q.ndim != 4:
        raise ValueError("Q, K and V must share one (B, H, S, D) shape")
    B, H, S, D = Q.shape
    O = np.zeros((B, H, S, D))
    DN = np.zeros((B, H, S, D))
    L = np.zeros((B, H, S))
    SM = np.zeros((B, H, S))
    sc = float(np.float32(scale))
    for b in range(B):
        for h in range(H):
            o, dn, lse, sm = _one_head(Q[b, h].astype(np.float64), K[b, h].astype(np.float64),
                                       V[b, h].astype(np.float64), causal, sc)
            O[b, h], DN[b, h], L[b, h], SM[b, h] = o, dn, lse, sm
    return O, DN, L, SM


def lse_error(lse: np.ndarray, lse_ref: np.ndarray, sm: np.ndarray) -> float:
    """max |lse - lse_ref| / max(1, sm): the log-sum-exp's error against the
    scale of the score rounding (at least 1, the scale of the exponential's
    and logarithm's own rounding); non-finite values fail."""
    lse = np.asarray(lse, dtype=np.float64)
    if lse.size == 0:
        return 0.0
    if not np.all(np.isfinite(lse)):
        return float("inf")
    return float(np.max(np.abs(lse - lse_ref) / np.maximum(1.0, sm)))


def normalized_error(o: np.ndarray, o_ref: np.ndarray, dn: np.ndarray):
    """max |o - o_ref| / dn over every element (dn = sum_j p_ij |v_jc|), with
    an exact match required where dn is 0 and any non-finite o failing;
    returns (error, index of the worst element)."""
    o = np.asarray(o, dtype=np.float64)
    if not np.all(np.isfinite(o)):
        bad = np.argwhere(~np.isfinite(o))[0]
        return float("inf"), tuple(int(x) for x in bad)
    diff = np.abs(o - o_ref)
    zero = dn == 0
    if np.any(zero & (diff != 0)):
        bad = np.argwhere(zero & (diff != 0))[0]
        return float("inf"), tuple(int(x) for x in bad)
    ratio = np.where(zero, 0.0, diff / np.where(zero, 1.0, dn))
    if ratio.size == 0:
        return 0.0, ()
    at = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    return float(ratio[at]), tuple(int(x) for x in at)
