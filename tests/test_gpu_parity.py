"""GPU parity: the HIP kernels, called through the C ABI, against the CPU oracle.

Two bars:
  * integer-valued inputs (|a|, |b| <= 4): every partial sum is an integer below 2^24, so
    fp32 accumulation is exact in any order; the GPU result must equal the oracle bitwise
    (fp32 out) or equal the oracle's round-to-nearest-even bf16 of it (bf16 out).  This
    catches any indexing, tail, pitch, swizzle or scheduling mistake.
  * the workloads' own value distributions: |C - C_ref| <= 4 K 2^-24 (|A||B|^T), plus
    2^-8 (|C_ref| + that) for bf16 output (oracle/check.py).
Full-size workloads are compared on sampled rows (tile-boundary rows plus seeded random
ones), which the oracle computes one by one.
"""
import numpy as np
import pytest

import oracle
from oracle import check as ck
import tiled_matmul_amd as tm
from tiled_matmul_amd import synth

from helpers import OUT_BF16, OUT_FP32, empty_out, out_to_host, run_gemm, to_device

pytestmark = pytest.mark.gpu

V = tm
ALL_TILED = [V.GEMM_VARIANT_SIMPLE, V.GEMM_VARIANT_MFMA, V.GEMM_VARIANT_PIPELINED,
             V.GEMM_VARIANT_PERSISTENT, V.GEMM_VARIANT_SPECIALIZED, V.GEMM_VARIANT_PINGPONG,
             V.GEMM_VARIANT_RING8, V.GEMM_VARIANT_RING4, V.GEMM_VARIANT_DTV, V.GEMM_VARIANT_ROLES,
             V.GEMM_VARIANT_AUTO]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield


def exact_expected(A, B, K, out_dtype, rows=None):
    C, _ = oracle.gemm(A, B, K=K, rows=rows)
    return C.astype(np.float32) if out_dtype == OUT_FP32 else oracle.round_bf16(C)


def assert_exact(got, A, B, K, out_dtype, rows=None, what=""):
    exp = exact_expected(A, B, K, out_dtype, rows)
    r = ck.check_exact(got, exp, out_dtype)
    assert r["ok"], f"{what}: {r}"


def assert_bound(got, A, B, K, out_dtype, rows=None, what=""):
    C, Mag = oracle.gemm(A, B, K=K, rows=rows)
    r = ck.check(got, C, Mag, K, out_dtype)
    assert r["ok"], f"{what}: {r}"
    return r


def sample_rows(M, tile=256, n_random=24, seed=0):
    rows = set()
    for b in range(0, M, tile):
        rows.update({b, b + 1, min(M - 1, b + tile - 1)})
    rows.update(np.random.default_rng(seed).integers(0, M, n_random).tolist())
    rows = sorted(r for r in rows if r < M)
    if len(rows) > 96:
        keep = np.random.default_rng(seed + 1).choice(len(rows), 96, replace=False)
        rows = sorted(rows[i] for i in keep) + [M - 1]
    return sorted(set(rows))


# ---------------------------------------------------------------------------------------
# Every variant, integer-exact, on shapes that span several tiles and have ragged tails.
# ---------------------------------------------------------------------------------------
SHAPES = [(128, 128, 128), (300, 200, 264), (257, 513, 136), (512, 384, 1024),
          (64, 1000, 8), (1, 77, 40), (33, 3, 520)]


@pytest.mark.parametrize("variant", ALL_TILED)
@pytest.mark.parametrize("out_dtype", [OUT_FP32, OUT_BF16])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_integer_exact_variants(variant, out_dtype, M, N, K):
    A = synth.integers(M, K, 11 + M)
    B = synth.integers(N, K, 12 + N)
    got = run_gemm(A, B, K, out_dtype, variant=variant)
    assert_exact(got, A, B, K, out_dtype, what=f"variant {variant} {M}x{N}x{K}")


@pytest.mark.parametrize("variant", [V.GEMM_VARIANT_GEMV, V.GEMM_VARIANT_AUTO])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 7, 9, 16])
@pytest.mark.parametrize("N,K", [(4096, 4096), (100, 264), (17, 8), (300, 1000), (33, 4360),
                                 (70, 8200)])
def test_integer_exact_gemv(variant, M, N, K):
    A = synth.integers(M, K, 21 + M)
    B = synth.integers(N, K, 22 + N)
    for out_dtype in (OUT_FP32, OUT_BF16):
        got = run_gemm(A, B, K, out_dtype, variant=variant)
        assert_exact(got, A, B, K, out_dtype, what=f"gemv {M}x{N}x{K}")


# ---------------------------------------------------------------------------------------
# Edge cases
# ---------------------------------------------------------------------------------------
def test_k_zero_writes_zeros():
    import torch
    for out_dtype in (OUT_FP32, OUT_BF16):
        C = empty_out(37, 50, out_dtype, fill=7)
        dummy = torch.zeros(8, dtype=torch.bfloat16, device="cuda")
        tm.gemm_bf16(37, 41, 0, dummy, 1, dummy, 1, C, 50, out_dtype)
        h = out_to_host(C, 37, 50, 50, out_dtype)
        assert np.all(h[:, :41] == 0) and np.all(h[:, 41:] == 7)


def test_empty_m_or_n_is_a_noop():
    import torch
    C = empty_out(4, 4, OUT_FP32, fill=5)
    dummy = torch.zeros(64, dtype=torch.bfloat16, device="cuda")
    tm.gemm_bf16(0, 4, 8, dummy, 8, dummy, 8, C, 4, OUT_FP32)
    tm.gemm_bf16(4, 0, 8, dummy, 8, dummy, 8, C, 4, OUT_FP32)
    assert np.all(out_to_host(C, 4, 4, 4, OUT_FP32) == 5)


@pytest.mark.parametrize("variant", ALL_TILED)
def test_padded_pitches(variant):
    M, N, K = 200, 300, 256
    A = synth.integers(M, K, 31, ld=K + 24)      # padding holds NaN: must never be read
    B = synth.integers(N, K, 32, ld=K + 8)
    got = run_gemm(A, B, K, OUT_FP32, variant=variant, ldc=N + 5)
    assert_exact(got, A, B, K, OUT_FP32, what="padded pitches")


# The skinny-M path (dot-product form for M <= 4, MFMA form above) with padded pitches whose
# padding holds NaN: K = 4360 spans two 4096-deep phases and ends mid 512-element chunk, so any
# read past K in W or X, or a wrong pitch, shows.
@pytest.mark.parametrize("variant", [V.GEMM_VARIANT_GEMV, V.GEMM_VARIANT_AUTO])
@pytest.mark.parametrize("M", [1, 3, 8, 16])
def test_gemv_padded_pitches(variant, M):
    N, K = 70, 4360
    A = synth.integers(M, K, 61 + M, ld=K + 24)
    B = synth.integers(N, K, 62 + M, ld=K + 8)
    for out_dtype in (OUT_FP32, OUT_BF16):
        got = run_gemm(A, B, K, out_dtype, variant=variant, ldc=N + 3)
        assert_exact(got, A, B, K, out_dtype, what=f"gemv padded pitches M={M}")
    rc, name, _, _ = tm.gemm_bf16_plan(variant, 1, M, N, K, 16, K + 24, 0, 16, K + 8, 0, 16, N + 3, 0, 0)
    assert rc == 0 and name == ("gemv_lds" if M <= 4 else "gemv")


# Ragged K (not a multiple of 8) and rows that are only 4- or 8-byte aligned: the pipelined
# kernels load whole 16-byte chunks below K rounded down to 8 and add the rest in one extra
# k step.  Pitch padding holds NaN, so a tail element read from beyond K would show.
RAGGED = [(130, 260, 77), (260, 129, 1027), (64, 64, 7), (300, 520, 100), (257, 300, 2053),
          (513, 257, 4)]
PIPE_VARIANTS = [V.GEMM_VARIANT_PIPELINED, V.GEMM_VARIANT_PERSISTENT,
                 V.GEMM_VARIANT_SPECIALIZED, V.GEMM_VARIANT_RING8, V.GEMM_VARIANT_RING4,
                 V.GEMM_VARIANT_AUTO]


@pytest.mark.parametrize("variant", PIPE_VARIANTS)
@pytest.mark.parametrize("M,N,K", RAGGED)
def test_ragged_k_and_4byte_rows(variant, M, N, K):
    lda = K + (K % 2)          # even: rows start on 4-byte boundaries
    ldb = K + 2 - (K % 2)
    A = synth.integers(M, K, 301 + K, ld=lda)
    B = synth.integers(N, K, 302 + K, ld=ldb)
    for out_dtype in (OUT_FP32, OUT_BF16):
        got = run_gemm(A, B, K, out_dtype, variant=variant, a_offset=2, b_offset=6)
        assert_exact(got, A, B, K, out_dtype, what=f"variant {variant} {M}x{N}x{K}")


@pytest.mark.parametrize("lda_pad", [1, 3, 4])
def test_unaligned_pitches_and_k(lda_pad):
    """Pitches and K that are not multiples of 8 (odd ldb with lda_pad 4: the general
    kernel; even pitches: the pipelined kernels with a ragged K tail)."""
    M, N, K = 130, 140, 100 + lda_pad
    A = synth.integers(M, K, 41, ld=K + lda_pad)
    B = synth.integers(N, K, 42, ld=K + 1)
    for out_dtype in (OUT_FP32, OUT_BF16):
        got = run_gemm(A, B, K, out_dtype)
        assert_exact(got, A, B, K, out_dtype, what=f"unaligned lda_pad={lda_pad}")


def test_misaligned_pointers():
    M, N, K = 150, 170, 128
    A = synth.integers(M, K, 51)
    B = synth.integers(N, K, 52)
    got = run_gemm(A, B, K, OUT_FP32, a_offset=1, b_offset=3)
    assert_exact(got, A, B, K, OUT_FP32, what="2-byte aligned operands")
    rc, name, _, _ = tm.gemm_bf16_plan(0, 1, M, N, K, 2, K, 0, 16, K, 0, 16, N, 0, 0)
    assert name == "mfma_128"


@pytest.mark.parametrize("K,expect_bits", [(4100, 0x4580), (4112, 0x4580), (4120, 0x4581),
                                           (4144, 0x4582), (1024, 0x4480)])
def test_all_ones_rounding(K, expect_bits):
    ones = np.full((64, K), 0x3F80, dtype=np.uint16)
    for variant in (V.GEMM_VARIANT_AUTO, V.GEMM_VARIANT_MFMA, V.GEMM_VARIANT_SIMPLE):
        got = run_gemm(ones, ones[:48], K, OUT_BF16, variant=variant)
        assert np.all(got == expect_bits), (variant, K, np.unique(got))
        got32 = run_gemm(ones, ones[:48], K, OUT_FP32, variant=variant)
        assert np.all(got32 == K)


def test_nan_propagates_to_its_row_only():
    M, N, K = 256, 256, 256
    A = synth.uniform(M, K, 61)
    B = synth.uniform(N, K, 62)
    A[7, 100] = 0x7FC0
    got = run_gemm(A, B, K, OUT_FP32)
    assert np.all(np.isnan(got[7]))
    assert np.isfinite(np.delete(got, 7, axis=0)).all()


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 4096), (3000, 5000, 4100)])
def test_identity_closed_form_full_size(M, N, K):
    """A = [I | 0] (row i is e_i): C[i][j] = B[j][i] exactly, no oracle needed."""
    A = np.zeros((M, K), dtype=np.uint16)
    A[np.arange(M), np.arange(M)] = 0x3F80
    B = synth.uniform(N, K, 71)
    for out_dtype in (OUT_FP32, OUT_BF16):
        got = run_gemm(A, B, K, out_dtype)
        exp = B[:, :M].T
        if out_dtype == OUT_FP32:
            exp = ck.bf16_bits_to_f64(exp).astype(np.float32)
        r = ck.check_exact(got, exp, out_dtype)
        assert r["ok"], r


def test_permutation_closed_form():
    K = 512
    perm = np.random.default_rng(3).permutation(K)
    A = np.zeros((K, K), dtype=np.uint16)
    A[np.arange(K), perm] = 0x3F80
    B = synth.normal(384, K, 81)
    got = run_gemm(A, B, K, OUT_FP32)
    exp = ck.bf16_bits_to_f64(B[:, perm].T).astype(np.float32)
    assert ck.check_exact(got, exp, OUT_FP32)["ok"]


def test_deterministic():
    A, B = synth.normal(1024, 2048, 91), synth.normal(768, 2048, 92)
    g1 = run_gemm(A, B, 2048, OUT_FP32)
    g2 = run_gemm(A, B, 2048, OUT_FP32)
    assert np.array_equal(g1.view(np.uint32), g2.view(np.uint32))


# ---------------------------------------------------------------------------------------
# Batched
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("variant", ALL_TILED)
def test_batched_integer_exact(variant):
    batch, M, N, K = 5, 130, 200, 136
    As = [synth.integers(M, K, 100 + b) for b in range(batch)]
    Bs = [synth.integers(N, K, 200 + b) for b in range(batch)]
    sA, sB, ldc = M * K + 8, N * K, N + 4
    sC = M * ldc + 12
    Abuf = np.zeros(batch * sA, np.uint16)
    Bbuf = np.zeros(batch * sB, np.uint16)
    for b in range(batch):
        Abuf[b * sA:b * sA + M * K] = As[b].reshape(-1)
        Bbuf[b * sB:b * sB + N * K] = Bs[b].reshape(-1)
    A, B = to_device(Abuf), to_device(Bbuf)
    C = empty_out(1, sC, OUT_FP32, batch=batch)
    tm.gemm_bf16_variant(variant, batch, M, N, K, A, K, sA, B, K, sB, C, ldc, sC, OUT_FP32)
    h = out_to_host(C, 1, sC, sC, OUT_FP32, batch=batch)
    for b in range(batch):
        got = h[b, 0, :M * ldc].reshape(M, ldc)[:, :N]
        assert_exact(got, As[b], Bs[b], K, OUT_FP32, what=f"batch item {b}")


# ---------------------------------------------------------------------------------------
# The workloads at their full sizes, through gemm_bf16 / gemm_bf16_strided_batched (the
# launch the bench times).
# ---------------------------------------------------------------------------------------
def workload_run(name, out_dtype=None, integer=False):
    w = synth.WORKLOADS[name]
    out_dtype = w["out"] if out_dtype is None else out_dtype
    M, N, K = w["M"], w["N"], w["K"]
    if integer:
        sa, sb = synth.seeds(w["cfg"])
        A, B = synth.integers(M, K, sa), synth.integers(N, K, sb)
    else:
        A, B = synth.make_operands(name)
    Ad, Bd = to_device(A), to_device(B)
    C = empty_out(M, N, out_dtype)
    tm.gemm_bf16(M, N, K, Ad, K, Bd, K, C, N, out_dtype)
    return A, B, out_to_host(C, M, N, N, out_dtype)


@pytest.mark.parametrize("name", ["single_tile_128", "gemv_m1", "gemv_m16"])
def test_workload_full_oracle(name):
    A, B, got = workload_run(name)
    K, out_dtype = synth.WORKLOADS[name]["K"], synth.WORKLOADS[name]["out"]
    assert_bound(got, A, B, K, out_dtype, what=name)
    A, B, got = workload_run(name, integer=True)
    assert_exact(got, A, B, K, out_dtype, what=name + " integer")


@pytest.mark.parametrize("name", ["square_4096", "irregular_3000x5000x4100",
                                  "ffn_up_8192x14336x4096", "ffn_down_8192x4096x14336"])
def test_workload_sampled_rows(name):
    w = synth.WORKLOADS[name]
    K, out_dtype = w["K"], w["out"]
    rows = sample_rows(w["M"])
    A, B, got = workload_run(name)
    r = assert_bound(got[rows], A, B, K, out_dtype, rows=rows, what=name)
    print(f"{name}: rows={len(rows)} max_err_over_bound={r['max_err_over_bound']:.3g}")
    assert np.isfinite(got).all()
    A, B, got = workload_run(name, integer=True)
    assert_exact(got[rows], A, B, K, out_dtype, rows=rows, what=name + " integer")


# The kernel with A in registers: K not a multiple of the 64-deep block (the last block
# partly past K) and an odd block count (the loop runs one block of zeros), rows of A and B
# beyond M and N, padded pitches with NaN between rows.
@pytest.mark.parametrize("M,N,K", [(256, 256, 64), (300, 520, 72), (520, 300, 200), (257, 1000, 4104),
                                   (1024, 768, 3000), (40, 24, 8)])
def test_dtv_block_tails(M, N, K):
    A = synth.integers(M, K, 401 + K, ld=K + 16)
    B = synth.integers(N, K, 402 + K, ld=K + 8)
    for out_dtype in (OUT_FP32, OUT_BF16):
        got = run_gemm(A, B, K, out_dtype, variant=V.GEMM_VARIANT_DTV, ldc=N + 4)
        assert_exact(got, A, B, K, out_dtype, what=f"dtv {M}x{N}x{K}")


# The same kernel at the full sizes of the large workloads (sampled rows).
@pytest.mark.parametrize("name", ["square_4096", "ffn_up_8192x14336x4096", "ffn_down_8192x4096x14336"])
def test_dtv_workload_sampled_rows(name):
    w = synth.WORKLOADS[name]
    M, N, K, out_dtype = w["M"], w["N"], w["K"], w["out"]
    rows = sample_rows(M)
    for integer in (False, True):
        if integer:
            sa, sb = synth.seeds(w["cfg"])
            A, B = synth.integers(M, K, sa), synth.integers(N, K, sb)
        else:
            A, B = synth.make_operands(name)
        got = run_gemm(A, B, K, out_dtype, variant=V.GEMM_VARIANT_DTV)
        if integer:
            assert_exact(got[rows], A, B, K, out_dtype, rows=rows, what=name + " dtv integer")
        else:
            assert_bound(got[rows], A, B, K, out_dtype, rows=rows, what=name + " dtv")
            assert np.isfinite(got).all()


@pytest.mark.parametrize("integer", [False, True])
@pytest.mark.parametrize("out_dtype", [OUT_FP32, OUT_BF16])
def test_workload_batched(out_dtype, integer):
    """All 64 items of the batched workload at its full shape through
    gemm_bf16_strided_batched (the launch the bench times), C filled with NaN first: every item
    against the oracle within the bound on the workload's values, and bitwise on integers."""
    name = "batched_64x256x256x1024"
    w = synth.WORKLOADS[name]
    batch, M, N, K = w["batch"], w["M"], w["N"], w["K"]
    if integer:
        sa, sb = synth.seeds(w["cfg"])
        pairs = [(synth.integers(M, K, sa + 2 * b), synth.integers(N, K, sb + 2 * b)) for b in range(batch)]
    else:
        pairs = [synth.make_operands(name, item=b) for b in range(batch)]
    A = to_device(np.stack([p[0] for p in pairs]))
    B = to_device(np.stack([p[1] for p in pairs]))
    C = empty_out(M, N, out_dtype, batch=batch, fill=float("nan") if out_dtype == OUT_FP32 else -1)
    tm.gemm_bf16_strided_batched(batch, M, N, K, A, K, M * K, B, K, N * K, C, N, M * N, out_dtype)
    h = out_to_host(C, M, N, N, out_dtype, batch=batch)
    for b in range(batch):
        if integer:
            assert_exact(h[b], pairs[b][0], pairs[b][1], K, out_dtype, what=f"item {b}")
        else:
            assert_bound(h[b], pairs[b][0], pairs[b][1], K, out_dtype, what=f"item {b}")
