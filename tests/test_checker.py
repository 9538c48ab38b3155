"""The acceptance checker must reject plausible wrong results.  Each mistake is planted in
the oracle's computation on the CPU (a dropped K tail, swapped rows, a row pitch off by one,
truncation instead of round-to-nearest-even), then checked against the correct oracle
result.  Integer-valued inputs make the correct result exact, so the bitwise check catches
every mistake; the random-value bound is shown to be the looser acceptance gate.  No GPU."""
import numpy as np
import pytest

import oracle
from oracle import check as ck
from tiled_matmul_amd import synth


@pytest.fixture(scope="module")
def case():
    M, N, K = 40, 48, 260
    A = synth.integers(M, K + 4, 1, ld=K + 4)   # pitch K+4, padding NaN
    B = synth.integers(N, K, 2)
    A[:, K:] = synth.integers(M, 4, 99)         # finite padding for the pitch mutation
    C, Mag = oracle.gemm(A, B, K=K)
    return A, B, K, C, Mag


def test_correct_result_passes(case):
    A, B, K, C, Mag = case
    assert ck.check_exact(C.astype(np.float32), C, ck.OUT_FP32)["ok"]
    assert ck.check(C.astype(np.float32), C, Mag, K, ck.OUT_FP32)["ok"]
    rb = oracle.round_bf16(C)
    assert ck.check_exact(rb, rb, ck.OUT_BF16)["ok"]
    assert ck.check(rb, C, Mag, K, ck.OUT_BF16)["ok"]


def test_dropped_k_tail_fails(case):
    A, B, K, C, Mag = case
    Cw, _ = oracle.gemm(np.ascontiguousarray(A[:, :K - 4]), np.ascontiguousarray(B[:, :K - 4]))
    assert not ck.check_exact(Cw.astype(np.float32), C, ck.OUT_FP32)["ok"]


def test_swapped_rows_fail(case):
    A, B, K, C, Mag = case
    Cw = C.copy()
    Cw[[3, 4]] = Cw[[4, 3]]
    assert not ck.check_exact(Cw.astype(np.float32), C, ck.OUT_FP32)["ok"]
    assert not ck.check(Cw.astype(np.float32), C, Mag, K, ck.OUT_FP32)["ok"]


def test_pitch_off_by_one_fails(case):
    A, B, K, C, Mag = case
    flat = A.reshape(-1)
    M, lda = A.shape
    Aw = np.lib.stride_tricks.as_strided(flat, shape=(M, K), strides=((lda - 1) * 2, 2))
    Cw, _ = oracle.gemm(np.ascontiguousarray(Aw), B)
    assert not ck.check_exact(Cw.astype(np.float32), C, ck.OUT_FP32)["ok"]


def test_truncation_instead_of_rne_fails(case):
    A, B, K, C, Mag = case
    f = C.astype(np.float32).view(np.uint32)
    truncated = (f >> 16).astype(np.uint16)
    assert not ck.check_exact(truncated, oracle.round_bf16(C), ck.OUT_BF16)["ok"]


def test_nan_fails():
    C = np.ones((2, 2))
    Cg = np.ones((2, 2), np.float32)
    Cg[1, 1] = np.nan
    assert not ck.check(Cg, C, np.ones((2, 2)), 1, ck.OUT_FP32)["ok"]


def test_bound_is_loose_for_random_values():
    """At K=4100 with U[-1,1] a dropped tail of 4 products is usually inside the bound:
    this is why the integer-exact cases are the bug detector."""
    A, B = synth.uniform(16, 4100, 5), synth.uniform(16, 4100, 6)
    C, Mag = oracle.gemm(A, B)
    Cw, _ = oracle.gemm(np.ascontiguousarray(A[:, :4096]), np.ascontiguousarray(B[:, :4096]))
    r = ck.check(Cw.astype(np.float32), C, Mag, 4100, ck.OUT_FP32)
    assert 0 < r["n_fail"] < r["n"]
