"""Pins of the CPU oracle against facts fixed outside it (closed forms, brute force with
exact rationals, a textbook routine, IEEE format definitions).  No GPU.

Each pin is chosen so that a plausible mistake in the oracle fails it:
  * a dropped or duplicated product      -> all-ones (C == K), brute force
  * a wrong sign or a wrong |.| in Mag    -> brute force on mixed signs, Mag checks
  * a wrong index / transposed operand   -> identity and permutation closed forms with
                                            non-square, non-symmetric operands
  * a wrong row pitch                     -> padded-ld cases (padding holds NaN)
  * a wrong bf16 decode                   -> IEEE bit-pattern table
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tiled_matmul_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bits_of(values):
    """Exact bf16 bit patterns of values that are representable in bf16 (test helper)."""
    f = np.asarray(values, dtype=np.float32)
    b = f.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "value not representable in bf16"
    return (b >> 16).astype(np.uint16)


def random_exact_bf16(rng, shape, emin=-8, emax=8):
    """bf16 patterns with exponents in [emin, emax] and random sign/significand."""
    sign = rng.integers(0, 2, size=shape).astype(np.uint16) << 15
    exp = (rng.integers(emin, emax + 1, size=shape) + 127).astype(np.uint16) << 7
    man = rng.integers(0, 128, size=shape).astype(np.uint16)
    return sign | exp | man


def frac_of_bits(h):
    """Exact rational value of a normal bf16 pattern, computed from its fields."""
    h = int(h)
    s = -1 if h >> 15 else 1
    e = ((h >> 7) & 0xFF) - 127
    m = h & 0x7F
    return s * Fraction(128 + m, 128) * (Fraction(2) ** e)


def test_decode_ieee_table(oracle_lib):
    cases = {
        0x3F80: 1.0, 0xBF80: -1.0, 0x4000: 2.0, 0x3F81: 1.0 + 2.0 ** -7,
        0x4580: 4096.0, 0x0001: 2.0 ** -133, 0x0080: 2.0 ** -126,
        0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127, 0x0000: 0.0, 0x7F80: np.inf,
        0xFF80: -np.inf, 0x3E80: 0.25, 0xC2F6: -123.0,
    }
    got = oracle.decode_bf16(np.array(list(cases), dtype=np.uint16))
    assert np.array_equal(got, np.array(list(cases.values())))
    neg0 = oracle.decode_bf16(np.array([0x8000], dtype=np.uint16))[0]
    assert neg0 == 0.0 and np.signbit(neg0)
    assert np.isnan(oracle.decode_bf16(np.array([0x7FC0], dtype=np.uint16))[0])


@pytest.mark.parametrize("M,N,K,seed", [(1, 1, 1, 0), (3, 5, 7, 1), (8, 8, 8, 2),
                                        (2, 7, 1, 3), (5, 3, 8, 4), (8, 1, 6, 5)])
def test_bruteforce_exact_rationals(oracle_lib, M, N, K, seed):
    rng = np.random.default_rng(seed)
    A = random_exact_bf16(rng, (M, K))
    B = random_exact_bf16(rng, (N, K))
    C, Mag = oracle.gemm(A, B)
    for i in range(M):
        for j in range(N):
            prods = [frac_of_bits(A[i, k]) * frac_of_bits(B[j, k]) for k in range(K)]
            exact = sum(prods, Fraction(0))
            mag = sum((abs(p) for p in prods), Fraction(0))
            # |exact sum| < 2^21 and every product is a multiple of 2^-32: exact in binary64
            assert Fraction(C[i, j]) == exact
            assert Fraction(Mag[i, j]) == mag


def test_numpy_textbook_crosscheck(oracle_lib):
    A, B = synth.normal(37, 300, 11), synth.normal(29, 300, 12)
    C, Mag = oracle.gemm(A, B)
    a = oracle.decode_bf16(A)
    b = oracle.decode_bf16(B)
    ref = a @ b.T
    assert np.all(np.abs(C - ref) <= 2 * 300 * 2.0 ** -53 * Mag)
    assert np.allclose(Mag, np.abs(a) @ np.abs(b).T, rtol=1e-14, atol=0)
    assert np.all(Mag >= np.abs(C))


def test_transpose_invariant(oracle_lib):
    A, B = synth.uniform(23, 64, 21), synth.uniform(17, 64, 22)
    C, M1 = oracle.gemm(A, B)
    Ct, M2 = oracle.gemm(B, A)
    assert np.array_equal(C, Ct.T) and np.array_equal(M1, M2.T)


def test_identity_closed_form(oracle_lib):
    K = 48
    I = bits_of(np.eye(K))
    B = synth.normal(19, K, 31)           # N = 19 != K
    C, _ = oracle.gemm(I, B)              # A = I  =>  C = B^T
    assert np.array_equal(C, oracle.decode_bf16(B).T)
    A = synth.normal(13, K, 32)
    C, _ = oracle.gemm(A, I)              # B = I  =>  C = A
    assert np.array_equal(C, oracle.decode_bf16(A))


def test_permutation_closed_form(oracle_lib):
    K = 40
    rng = np.random.default_rng(7)
    perm = rng.permutation(K)
    P = np.zeros((K, K))
    P[np.arange(K), perm] = 1.0           # row i of A is e_{perm[i]}
    B = synth.uniform(21, K, 41)
    C, _ = oracle.gemm(bits_of(P), B)
    b = oracle.decode_bf16(B)
    for i in range(K):
        assert np.array_equal(C[i], b[:, perm[i]])


def test_rank1_closed_form(oracle_lib):
    M, N, K = 9, 11, 300
    rng = np.random.default_rng(3)
    a = rng.integers(1, 16, M) * rng.choice([-1, 1], M)
    bb = rng.integers(1, 16, N) * rng.choice([-1, 1], N)
    x = rng.choice([-1, 1], K)
    y = rng.choice([-1, 1], K)
    A = bits_of(np.outer(a, x))
    B = bits_of(np.outer(bb, y))
    C, Mag = oracle.gemm(A, B)
    dot = int(np.dot(x, y))
    for i in range(M):
        for j in range(N):
            assert C[i, j] == a[i] * bb[j] * dot
            assert Mag[i, j] == abs(a[i] * bb[j]) * K


@pytest.mark.parametrize("K", [1, 64, 4100, 4112, 4120])
def test_all_ones(oracle_lib, K):
    ones = bits_of(np.ones((3, K)))
    C, Mag = oracle.gemm(ones, bits_of(np.ones((5, K))))
    assert np.all(C == K) and np.all(Mag == K)


def test_padded_ld_ignores_padding(oracle_lib):
    K = 100
    A = synth.uniform(6, K, 51, ld=K + 28)   # padding is NaN
    B = synth.uniform(7, K, 52, ld=K + 3)
    C, Mag = oracle.gemm(A, B, K=K)
    C2, _ = oracle.gemm(np.ascontiguousarray(A[:, :K]), np.ascontiguousarray(B[:, :K]))
    assert np.isfinite(C).all() and np.array_equal(C, C2)


def test_row_sampling_matches_full(oracle_lib):
    A, B = synth.normal(50, 70, 61), synth.normal(40, 70, 62)
    C, Mag = oracle.gemm(A, B)
    rows = [49, 0, 17, 17, 3]
    Cs, Ms = oracle.gemm(A, B, rows=rows)
    assert np.array_equal(Cs, C[rows]) and np.array_equal(Ms, Mag[rows])


def test_thread_count_does_not_change_result(oracle_lib):
    A, B = synth.normal(33, 257, 71), synth.normal(31, 257, 72)
    C1, _ = oracle.gemm(A, B, nthreads=1)
    C8, _ = oracle.gemm(A, B, nthreads=8)
    assert np.array_equal(C1, C8)


def test_degenerate_sizes(oracle_lib):
    C, Mag = oracle.gemm(np.zeros((4, 0), np.uint16), np.zeros((3, 0), np.uint16), K=0)
    assert C.shape == (4, 3) and np.all(C == 0) and np.all(Mag == 0)
    C, _ = oracle.gemm(np.zeros((0, 8), np.uint16), synth.uniform(3, 8, 1))
    assert C.shape == (0, 3)
    C, _ = oracle.gemm(synth.uniform(3, 8, 1), np.zeros((0, 8), np.uint16))
    assert C.shape == (3, 0)


def test_round_bf16_golden_table(oracle_lib):
    rows = []
    with open(os.path.join(GOLDEN, "bf16_rne_cases.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                v, bits = line.split()[:2]
                rows.append((float(v), int(bits, 16)))
    got = oracle.round_bf16([v for v, _ in rows])
    assert [int(g) for g in got] == [b for _, b in rows]


def test_round_bf16_matches_torch_on_fp32(oracle_lib):
    """On binary32 inputs one rounding to bf16 is torch's conversion (a library routine)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(1000),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),      # subnormal range
        np.array([3.3895314e38, -3.3895314e38, 3.4e38], dtype=np.float32),  # near overflow
        (np.arange(4096, 8192, dtype=np.float32)),                    # every tie near 4096
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_round_bf16_specials(oracle_lib):
    got = oracle.round_bf16([np.inf, -np.inf, 1e300, -0.0])
    assert [int(g) for g in got] == [0x7F80, 0xFF80, 0x7F80, 0x8000]
    assert (int(oracle.round_bf16([np.nan])[0]) & 0x7FFF) > 0x7F80
