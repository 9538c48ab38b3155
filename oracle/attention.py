"""CPU oracle for the fused attention forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use
it; it shares no code with the product path (``tiled_matmul_amd``).

What it computes.  The page "Modern GPU Programming for MLSys：深度解读" (its outline of the
book's Part IV, Flash Attention 4) and the page "Jak okiełznać Blackwella bez szaleństwa od
CUDA" (section "Co znajdziesz w tym samouczku") describe an attention kernel built from the
GEMM techniques: softmax between two matrix products, online-softmax rescaling, causal
masking and grouped-query attention.  The online rescaling is a way of evaluating the softmax
block by block; the result it reaches is the plain definition, which is what this oracle
writes out (in binary64, the whole score row at once):

    S[i][j]  = scale * sum_c Q[b,h,i,c] K[b,g(h),j,c]          g(h) = h / (Hq / Hkv)   (GQA)
    S[i][j]  = -inf  where causal and j > i + (Lk - Lq)                 (bottom-right aligned)
    P[i][j]  = exp(S[i][j] - max_j S[i][j]) / sum_j exp(S[i][j] - max_j S[i][j])
    O[b,h,i] = sum_j P[i][j] V[b,g(h),j,:]
    LSE[b,h,i] = max_j S + log(sum_j exp(S - max_j S))   (natural log; -inf for an empty row)

A row with no allowed key (causal with Lq > Lk) has O = 0.  Inputs are bf16 bit patterns
(uint16), decoded exactly; Q, K, V are [B][H][L][d] arrays.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(h) -> np.ndarray:
    h = np.asarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def attention(Q, K, V, scale: float, causal: bool, heads=None, rows=None):
    """(O, LSE, PV, SMAG) in binary64.  Q: [B][Hq][Lq][d], K, V: [B][Hkv][Lk][d] (bf16 bits or
    floats).  ``heads``: optional list of (b, h) pairs to compute (default all); ``rows``:
    optional list of query rows (default all).  Returns arrays shaped [n_heads][n_rows][d]
    (O, and PV = P |V|, the magnitude the acceptance bound is written in) and
    [n_heads][n_rows] (LSE; SMAG = d scale max_j sum_c |Q_ic K_jc| + max_j |S_ij|, the
    magnitude the scores' rounding error is written in)."""
    def f64(x):
        x = np.asarray(x)
        return bf16_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)
    Q, K, V = f64(Q), f64(K), f64(V)
    B, Hq, Lq, d = Q.shape
    _, Hkv, Lk, _ = K.shape
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    heads = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else list(heads)
    rows = np.arange(Lq) if rows is None else np.asarray(rows)
    O = np.zeros((len(heads), len(rows), d))
    PV = np.zeros((len(heads), len(rows), d))
    LSE = np.full((len(heads), len(rows)), -np.inf)
    SMAG = np.zeros((len(heads), len(rows)))
    for n, (b, h) in enumerate(heads):
        g = h // group
        S = scale * (Q[b, h, rows] @ K[b, g].T)                       # [rows][Lk]
        if causal:
            allowed = np.arange(Lk)[None, :] <= (rows[:, None] + (Lk - Lq))
            S = np.where(allowed, S, -np.inf)
        m = S.max(axis=1, keepdims=True)
        ok = np.isfinite(m[:, 0])
        E = np.where(ok[:, None], np.exp(S - np.where(ok[:, None], m, 0.0)), 0.0)
        l = E.sum(axis=1, keepdims=True)
        P = np.where(ok[:, None], E / np.where(l > 0, l, 1.0), 0.0)
        O[n] = P @ V[b, g]
        PV[n] = P @ np.abs(V[b, g])
        LSE[n] = np.where(ok, m[:, 0] + np.log(np.where(ok, l[:, 0], 1.0)), -np.inf)
        SMAG[n] = score_magnitude(Q[b, h, rows], K[b, g], S, scale, allowed if causal else None)
    return O, LSE, PV, SMAG


def score_magnitude(Qr, Kg, S, scale: float, allowed=None) -> np.ndarray:
    """SMAG of each query row: d |scale| max_j sum_c |Q_ic K_jc| + max_j |S_ij| over the
    allowed keys j (0 for a row with none): the score magnitudes that the fp32 error of a
    score, accumulated over d products and then scaled, is bounded by."""
    d = Qr.shape[-1]
    Sa = abs(scale) * (np.abs(Qr) @ np.abs(Kg).T)
    if allowed is not None:
        Sa = np.where(allowed, Sa, 0.0)
    return d * Sa.max(axis=1, initial=0.0) + np.where(np.isfinite(S), np.abs(S), 0.0).max(axis=1, initial=0.0)
