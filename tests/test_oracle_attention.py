"""Pins of the attention oracle (oracle/attention.py) to things other than itself: brute force
with exactly rounded sums, closed forms (zero queries, the first causal row, a dominant key),
grouped-query attention as multi-head attention with repeated K/V heads, invariance under a
permutation of the keys, rows that sum to one, empty causal rows, and the checker rejecting a
mask that is off by one.  CPU only."""
import math

import numpy as np
import pytest

from oracle import attention as att
from oracle import check as ck
from tiled_matmul_amd import synth


def qkv(B, Hq, Hkv, Lq, Lk, d, seed, sigma=1.0):
    Q = synth.normal(B * Hq * Lq, d, seed, sigma).reshape(B, Hq, Lq, d)
    K = synth.normal(B * Hkv * Lk, d, seed + 1, sigma).reshape(B, Hkv, Lk, d)
    V = synth.normal(B * Hkv * Lk, d, seed + 2).reshape(B, Hkv, Lk, d)
    return Q, K, V


def brute(Q, K, V, scale, causal):
    q, k, v = (att.bf16_to_f64(x) for x in (Q, K, V))
    B, Hq, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    O = np.zeros(q.shape)
    LSE = np.full((B, Hq, Lq), -math.inf)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            for i in range(Lq):
                js = [j for j in range(Lk) if not causal or j <= i + Lk - Lq]
                if not js:
                    continue
                s = [scale * math.fsum(q[b, h, i, c] * k[b, g, j, c] for c in range(d)) for j in js]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                tot = math.fsum(e)
                for c in range(d):
                    O[b, h, i, c] = math.fsum(e[t] * v[b, g, j, c] for t, j in enumerate(js)) / tot
                LSE[b, h, i] = m + math.log(tot)
    return O, LSE


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Lq,Lk", [(5, 5), (3, 7), (6, 4)])
def test_brute_force(causal, Lq, Lk):
    Q, K, V = qkv(2, 4, 2, Lq, Lk, 8, 900 + Lq + Lk)
    O, LSE, PV, _ = att.attention(Q, K, V, 0.35, causal)
    Ob, Lb = brute(Q, K, V, 0.35, causal)
    assert np.allclose(O.reshape(Ob.shape), Ob, rtol=0, atol=1e-12)
    both = np.isneginf(LSE.reshape(Lb.shape)) & np.isneginf(Lb)
    with np.errstate(invalid="ignore"):
        assert np.all(both | (np.abs(LSE.reshape(Lb.shape) - Lb) < 1e-12))


def test_zero_queries_give_the_mean_of_the_allowed_values():
    B, Hq, Hkv, L, d = 1, 2, 1, 6, 4
    _, K, V = qkv(B, Hq, Hkv, L, L, d, 910)
    Q = np.zeros((B, Hq, L, d), np.uint16)
    O, LSE, _, _ = att.attention(Q, K, V, 1.0, causal=True)
    v = att.bf16_to_f64(V)[0, 0]
    for i in range(L):
        assert np.allclose(O[0, i], v[:i + 1].mean(axis=0), atol=1e-15)
        assert abs(LSE[0, i] - math.log(i + 1)) < 1e-15
    O, LSE, _, _ = att.attention(Q, K, V, 1.0, causal=False)
    assert np.allclose(O[1], v.mean(axis=0)[None, :], atol=1e-15)


def test_first_causal_row_is_the_first_value_and_a_dominant_key_wins():
    Q, K, V = qkv(1, 1, 1, 4, 4, 8, 920)
    O, LSE, _, _ = att.attention(Q, K, V, 0.5, causal=True)
    v = att.bf16_to_f64(V)[0, 0]
    q, k = att.bf16_to_f64(Q)[0, 0], att.bf16_to_f64(K)[0, 0]
    assert np.array_equal(O[0, 0], v[0])
    assert LSE[0, 0] == 0.5 * float(q[0] @ k[0])
    # scale 60 on a score gap of order 1: the largest key takes all the weight in fp64
    Qd = np.zeros((1, 1, 1, 8))
    Kd = np.zeros((1, 1, 5, 8))
    Kd[0, 0, 3, 0] = 20.0
    Qd[0, 0, 0, 0] = 1.0
    Vd = np.ones((1, 1, 5, 8)) * np.arange(5)[None, None, :, None]   # value row j is all j
    O, _, _, _ = att.attention(Qd, Kd, Vd, 60.0, False)
    assert abs(O[0, 0, 0] - 3.0) < 1e-12


def test_gqa_equals_mha_with_repeated_heads():
    Q, K, V = qkv(2, 8, 2, 9, 11, 16, 930)
    O, LSE, _, _ = att.attention(Q, K, V, 0.25, causal=True)
    Kr, Vr = np.repeat(K, 4, axis=1), np.repeat(V, 4, axis=1)
    O2, LSE2, _, _ = att.attention(Q, Kr, Vr, 0.25, causal=True)
    assert np.array_equal(O, O2) and np.array_equal(LSE, LSE2)


def test_key_permutation_invariance_without_mask():
    Q, K, V = qkv(1, 2, 2, 7, 13, 8, 940)
    perm = np.random.default_rng(0).permutation(13)
    O, LSE, _, _ = att.attention(Q, K, V, 0.3, causal=False)
    O2, LSE2, _, _ = att.attention(Q, K[:, :, perm], V[:, :, perm], 0.3, causal=False)
    assert np.allclose(O, O2, atol=1e-12) and np.allclose(LSE, LSE2, atol=1e-12)


def test_rows_sum_to_one_and_empty_rows():
    Q, K, _ = qkv(1, 1, 1, 6, 4, 8, 950)
    ones = np.ones((1, 1, 4, 8))
    O, LSE, PV, _ = att.attention(Q, K, ones, 0.4, causal=True)   # Lq > Lk: rows 0, 1 empty
    assert np.all(O[0, :2] == 0) and np.all(np.isneginf(LSE[0, :2]))
    assert np.allclose(O[0, 2:], 1.0, atol=1e-15) and np.allclose(PV[0, 2:], 1.0, atol=1e-15)


def test_rows_and_heads_subsets():
    Q, K, V = qkv(2, 4, 2, 8, 8, 8, 960)
    O, LSE, _, _ = att.attention(Q, K, V, 0.3, causal=True)
    O2, LSE2, _, _ = att.attention(Q, K, V, 0.3, causal=True, heads=[(1, 3), (0, 1)], rows=[7, 0, 4])
    assert np.array_equal(O2[0], O[7][[7, 0, 4]]) and np.array_equal(O2[1], O[1][[7, 0, 4]])
    assert np.array_equal(LSE2[0], LSE[7][[7, 0, 4]])


def test_checker_accepts_rounding_and_rejects_an_off_by_one_mask():
    Q, K, V = qkv(1, 2, 1, 64, 64, 32, 970)
    O, LSE, PV, SM = att.attention(Q, K, V, 0.2, causal=True)
    r = ck.check_attention(O.astype(np.float32), O, PV, SM, 64, ck.OUT_FP32, LSE.astype(np.float32), LSE)
    assert r["ok"], r
    # a mask that lets each query see one key too many
    Ow, Lw, _, _ = att.attention(Q, np.concatenate([K, K[:, :, :1]], 2), np.concatenate([V, V[:, :, :1]], 2), 0.2, causal=True)
    # Lk + 1 keys, bottom-right aligned: row i sees keys 0 .. i + 1
    r = ck.check_attention(Ow.astype(np.float32), O, PV, SM, 64, ck.OUT_FP32)
    assert not r["ok"]


# --- SMAG, the score magnitude the attention tolerance is written in -------------------------

def brute_smag(Q, K, scale, causal):
    """SMAG[b][h][i] = d |scale| max_j sum_c |Q_ic K_jc| + max_j |scale sum_c Q_ic K_jc| over
    the allowed keys j, with exactly rounded sums (pure-Python loops)."""
    q, k = att.bf16_to_f64(Q), att.bf16_to_f64(K)
    B, Hq, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    out = np.zeros((B, Hq, Lq))
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            for i in range(Lq):
                js = [j for j in range(Lk) if not causal or j <= i + Lk - Lq]
                if not js:
                    continue
                mag = max(math.fsum(abs(q[b, h, i, c] * k[b, g, j, c]) for c in range(d)) for j in js)
                s = max(abs(math.fsum(q[b, h, i, c] * k[b, g, j, c] for c in range(d))) for j in js)
                out[b, h, i] = d * abs(scale) * mag + abs(scale) * s
    return out


@pytest.mark.parametrize("causal,Lq,Lk", [(False, 5, 7), (True, 6, 4), (True, 5, 5)])
def test_smag_equals_its_definition(causal, Lq, Lk):
    Q, K, V = qkv(1, 4, 2, Lq, Lk, 8, 930 + Lq)
    _, _, _, SMAG = att.attention(Q, K, V, -0.3, causal)
    ref = brute_smag(Q, K, -0.3, causal).reshape(SMAG.shape)
    assert np.allclose(SMAG, ref, rtol=2.0 ** -45, atol=0.0)


def test_smag_pin_rejects_planted_mistakes(monkeypatch):
    """The pin above fails on plausible mistakes planted in the oracle: the d factor dropped,
    the scale's sign kept (negative scale), masked keys counted."""
    Q, K, V = qkv(1, 2, 1, 6, 4, 8, 940)
    scale = -0.3
    ref = brute_smag(Q, K, scale, True).reshape(2, 6)
    good = att.score_magnitude

    def variant(Qr, Kg, S, scale, allowed, factor):
        Sa = scale * (np.abs(Qr) @ np.abs(Kg).T)
        if allowed is not None:
            Sa = np.where(allowed, Sa, 0.0)
        return factor * Sa.max(axis=1, initial=0.0) + np.where(np.isfinite(S), np.abs(S), 0.0).max(axis=1, initial=0.0)

    def no_d(Qr, Kg, S, scale, allowed=None):
        return variant(Qr, Kg, S, abs(scale), allowed, 1)

    def signed_scale(Qr, Kg, S, scale, allowed=None):
        return variant(Qr, Kg, S, scale, allowed, Qr.shape[-1])

    def mask_ignored(Qr, Kg, S, scale, allowed=None):
        return good(Qr, Kg, S, scale, None)

    for mutant in (no_d, signed_scale, mask_ignored):
        monkeypatch.setattr(att, "score_magnitude", mutant)
        _, _, _, SMAG = att.attention(Q, K, V, scale, True)
        assert not np.allclose(SMAG, ref, rtol=2.0 ** -45, atol=0.0), mutant.__name__
    monkeypatch.setattr(att, "score_magnitude", good)
