"""Pins of the attention oracle against facts that do not come from it.

The oracle (oracle/attention.py) is scaled dot-product attention written out
in fp64 ("Bare Metal Bard", page 1, third paragraph, names the fused kernel
that computes it).  Each pin below is a closed form, an invariance, a
library routine or brute force in plain Python, chosen so that a plausible
mistake (a missing scale, the diagonal masked, the softmax over the wrong
axis, no max shift, values read from the wrong tensor) fails at least one
of them; the planted-mutant test checks exactly that.
"""
import math

import numpy as np
import pytest
import scipy.special

from oracle import attention as att

TOL = 1e-12


def rnd(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def close(a, b, tol=TOL):
    return np.allclose(a, b, rtol=tol, atol=tol)


# --------------------------------------------------------------------------
# pins, written as functions so the mutant test can re-run them
# --------------------------------------------------------------------------

def pin_uniform_scores():
    # Q = 0: every visible key gets the same score, so o_i is the mean of
    # the visible value rows and lse_i = log(number of visible keys)
    B, H, S, D = 1, 2, 9, 5
    Q = np.zeros((B, H, S, D), np.float32)
    K, V = rnd((B, H, S, D), 1), rnd((B, H, S, D), 2)
    for causal in (False, True):
        O, DN, L, SM = att.attention_fwd(Q, K, V, causal, 0.125)
        for h in range(H):
            for i in range(S):
                n = i + 1 if causal else S
                mean = [math.fsum(float(V[0, h, j, c]) for j in range(n)) / n for c in range(D)]
                assert close(O[0, h, i], mean)
                assert close(L[0, h, i], math.log(n))
                absmean = [math.fsum(abs(float(V[0, h, j, c])) for j in range(n)) / n
                           for c in range(D)]
                assert close(DN[0, h, i], absmean)
                assert SM[0, h, i] == 0.0            # every score is exactly 0


def pin_dominant_key():
    # key 3 scores 200 above every other key for every query: its weight is
    # 1 - O(e^-200) and the output is its value row (to fp64 rounding);
    # causal rows before 3 do not see it
    B, H, S, D = 1, 1, 8, 4
    Q = np.zeros((B, H, S, D), np.float32)
    K = np.zeros((B, H, S, D), np.float32)
    Q[..., 0] = 1.0
    K[0, 0, 3, 0] = 1600.0                     # scale 1/8: score 200
    V = rnd((B, H, S, D), 3)
    O, _, L, _ = att.attention_fwd(Q, K, V, False, 0.125)
    for i in range(S):
        assert close(O[0, 0, i], V[0, 0, 3])
        assert close(L[0, 0, i], 200.0)
    O, _, L, _ = att.attention_fwd(Q, K, V, True, 0.125)
    for i in range(3, S):
        assert close(O[0, 0, i], V[0, 0, 3]) and close(L[0, 0, i], 200.0)
    for i in range(3):                          # uniform over keys 0..i
        assert close(O[0, 0, i], V[0, 0, :i + 1].astype(np.float64).mean(axis=0))


def pin_single_key_and_two_keys():
    # S = 1: the only key has weight 1: o = v, lse = its score
    q, k, v = rnd((1, 1, 1, 6), 4), rnd((1, 1, 1, 6), 5), rnd((1, 1, 1, 6), 6)
    O, _, L, SM = att.attention_fwd(q, k, v, False, 0.3)
    assert np.array_equal(O[0, 0, 0], v[0, 0, 0].astype(np.float64))
    s = 0.30000001192092896 * math.fsum(float(a) * float(b) for a, b in zip(q[0, 0, 0], k[0, 0, 0]))
    assert close(L[0, 0, 0], s)
    assert close(SM[0, 0, 0], 0.30000001192092896 * math.fsum(
        abs(float(a) * float(b)) for a, b in zip(q[0, 0, 0], k[0, 0, 0])))
    # S = 2, non-causal: the weights are the logistic function of the
    # score difference
    q, k, v = rnd((1, 1, 2, 3), 7), rnd((1, 1, 2, 3), 8), rnd((1, 1, 2, 3), 9)
    O, _, _, _ = att.attention_fwd(q, k, v, False, 0.5)
    for i in range(2):
        s0 = 0.5 * math.fsum(float(a) * float(b) for a, b in zip(q[0, 0, i], k[0, 0, 0]))
        s1 = 0.5 * math.fsum(float(a) * float(b) for a, b in zip(q[0, 0, i], k[0, 0, 1]))
        p0 = 1.0 / (1.0 + math.exp(s1 - s0))
        want = p0 * v[0, 0, 0].astype(np.float64) + (1 - p0) * v[0, 0, 1].astype(np.float64)
        assert close(O[0, 0, i], want)


def pin_key_permutation():
    # without a mask the keys form a set: permuting keys and values together
    # leaves every output unchanged
    B, H, S, D = 2, 2, 11, 7
    Q, K, V = rnd((B, H, S, D), 10), rnd((B, H, S, D), 11), rnd((B, H, S, D), 12)
    perm = np.random.default_rng(13).permutation(S)
    O, DN, L, SM = att.attention_fwd(Q, K, V, False, 0.4)
    O2, DN2, L2, SM2 = att.attention_fwd(Q, K[:, :, perm], V[:, :, perm], False, 0.4)
    assert close(O, O2) and close(DN, DN2) and close(L, L2) and close(SM, SM2)


def pin_scipy():
    # scipy's own softmax and logsumexp of independently formed scores
    B, H, S, D = 1, 3, 13, 8
    Q, K, V = rnd((B, H, S, D), 14, 2.0), rnd((B, H, S, D), 15, 2.0), rnd((B, H, S, D), 16)
    for causal in (False, True):
        O, _, L, _ = att.attention_fwd(Q, K, V, causal, 0.35)
        for h in range(H):
            s = np.einsum("id,jd->ij", Q[0, h].astype(np.float64),
                          K[0, h].astype(np.float64)) * float(np.float32(0.35))
            if causal:
                s[np.triu_indices(S, 1)] = -np.inf
            assert close(O[0, h], scipy.special.softmax(s, axis=1) @ V[0, h].astype(np.float64))
            assert close(L[0, h], scipy.special.logsumexp(s, axis=1))


def pin_brute_force():
    # plain Python, element by element, on tiny shapes (both mask modes)
    for (S, D, causal, seed) in [(1, 1, False, 17), (3, 2, True, 18), (4, 3, False, 19),
                                 (5, 4, True, 20)]:
        Q, K, V = rnd((1, 1, S, D), seed), rnd((1, 1, S, D), seed + 100), rnd((1, 1, S, D), seed + 200)
        scale = 0.7
        O, DN, L, SM = att.attention_fwd(Q, K, V, causal, scale)
        sc = float(np.float32(scale))
        for i in range(S):
            keys = range(i + 1) if causal else range(S)
            s = {j: sc * math.fsum(float(Q[0, 0, i, c]) * float(K[0, 0, j, c]) for c in range(D))
                 for j in keys}
            m = max(s.values())
            w = {j: math.exp(s[j] - m) for j in keys}
            tot = math.fsum(w.values())
            for c in range(D):
                o = math.fsum(w[j] * float(V[0, 0, j, c]) for j in keys) / tot
                dn = math.fsum(w[j] * abs(float(V[0, 0, j, c])) for j in keys) / tot
                assert close(O[0, 0, i, c], o) and close(DN[0, 0, i, c], dn)
            assert close(L[0, 0, i], m + math.log(tot))
            sm = math.fsum(w[j] * sc * math.fsum(abs(float(Q[0, 0, i, c]) * float(K[0, 0, j, c]))
                                                 for c in range(D)) for j in keys) / tot
            assert close(SM[0, 0, i], sm)


def pin_large_scores():
    # scores far beyond exp's range: the max shift keeps every weight finite
    B, H, S, D = 1, 1, 6, 3
    Q, K, V = rnd((B, H, S, D), 21, 40.0), rnd((B, H, S, D), 22, 40.0), rnd((B, H, S, D), 23)
    O, DN, L, _ = att.attention_fwd(Q, K, V, False, 1.0)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    s = Q[0, 0].astype(np.float64) @ K[0, 0].astype(np.float64).T
    assert close(L[0, 0], scipy.special.logsumexp(s, axis=1))


PINS = [pin_uniform_scores, pin_dominant_key, pin_single_key_and_two_keys, pin_key_permutation,
        pin_scipy, pin_brute_force, pin_large_scores]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    att.plant(None)
    pin()


@pytest.mark.parametrize("mutant", att.MUTANTS)
def test_planted_mutant_fails_a_pin(mutant):
    caught = []
    att.plant(mutant)
    try:
        for pin in PINS:
            try:
                with np.errstate(all="ignore"):
                    pin()
            except (AssertionError, FloatingPointError):
                caught.append(pin.__name__)
    finally:
        att.plant(None)
    assert caught, f"mutant {mutant} passed every pin"


def test_lse_error_statistic():
    ref = np.array([1.0, 2.0, 3.0])
    sm = np.array([0.5, 10.0, 0.0])
    assert att.lse_error(ref.copy(), ref, sm) == 0.0
    assert att.lse_error(ref + np.array([1e-3, 0, 0]), ref, sm) == pytest.approx(1e-3)
    assert att.lse_error(ref + np.array([0, 1e-2, 0]), ref, sm) == pytest.approx(1e-3)
    assert att.lse_error(np.array([1.0, np.inf, 3.0]), ref, sm) == math.inf


def test_normalized_error_statistic():
    ref = np.array([[1.0, 2.0], [0.0, -3.0]])
    dn = np.array([[2.0, 4.0], [0.0, 3.0]])
    assert att.normalized_error(ref.copy(), ref, dn) == (0.0, (0, 0))
    o = ref.copy()
    o[0, 1] += 1.0
    assert att.normalized_error(o, ref, dn) == (0.25, (0, 1))
    o = ref.copy()
    o[1, 0] = 1e-30                      # dn = 0 demands an exact match
    assert att.normalized_error(o, ref, dn)[0] == math.inf
    o = ref.copy()
    o[1, 1] = np.nan
    assert att.normalized_error(o, ref, dn)[0] == math.inf
