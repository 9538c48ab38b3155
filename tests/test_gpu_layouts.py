"""GPU parity of the MN-major operand layouts (gemm_bf16_layout) against the CPU oracle.

The oracle takes K-major operands; the MN-major device copies are the transposes of the same
bf16 arrays (padding columns hold NaN, so a kernel that reads them fails the check).
Integer-valued inputs make every partial sum exact in fp32, so the GPU must match the
oracle bitwise (fp32 out) or the oracle's round-to-nearest-even bf16 (bf16 out).
"""
import numpy as np
import pytest

import oracle
from oracle import check as ck
import tiled_matmul_amd as tm
from tiled_matmul_amd import synth

from helpers import OUT_BF16, OUT_FP32, empty_out, out_to_host, to_device

pytestmark = pytest.mark.gpu

KM, MN = tm.GEMM_LAYOUT_K_MAJOR, tm.GEMM_LAYOUT_MN_MAJOR
LAYOUTS = [(KM, MN), (MN, KM), (MN, MN)]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield


def mn_major(X, ld=None):
    """K-major bits (rows x K) -> the MN-major array (K x ld), padding columns NaN."""
    rows, K = X.shape
    ld = rows if ld is None else ld
    out = np.full((K, ld), synth.PAD_BITS, dtype=np.uint16)
    out[:, :rows] = X.T
    return out


def run_layout(A, B, la, lb, out_dtype, variant=tm.GEMM_VARIANT_AUTO, lda=None, ldb=None,
               a_offset=0, b_offset=0):
    """One GEMM through gemm_bf16_layout; A (M x K) and B (N x K) are K-major bits and are
    laid out as asked on the device."""
    (M, K), (N, _) = A.shape, B.shape
    kpitch = K + K % 2   # K-major pitch: even (rows 4-byte aligned), the pad column NaN
    Ad = mn_major(A, lda) if la == MN else synth_pad(A, kpitch if lda is None else lda)
    Bd = mn_major(B, ldb) if lb == MN else synth_pad(B, kpitch if ldb is None else ldb)
    Ag, Bg = to_device(Ad, a_offset), to_device(Bd, b_offset)
    C = empty_out(M, N, out_dtype)
    tm.gemm_bf16_layout(la, lb, variant, 1, M, N, K, Ag, Ad.shape[1], 0, Bg, Bd.shape[1], 0,
                        C, N, 0, out_dtype)
    return out_to_host(C, M, N, N, out_dtype)


def synth_pad(X, ld):
    out = np.full((X.shape[0], ld), synth.PAD_BITS, dtype=np.uint16)
    out[:, :X.shape[1]] = X
    return out


def assert_exact(got, A, B, out_dtype, rows=None, what=""):
    C, _ = oracle.gemm(A, B, rows=rows)
    exp = C.astype(np.float32) if out_dtype == OUT_FP32 else oracle.round_bf16(C)
    r = ck.check_exact(got, exp, out_dtype)
    assert r["ok"], f"{what}: {r}"


def plan_name(A, B, la, lb, variant):
    (M, K), (N, _) = A.shape, B.shape
    lda = M if la == MN else K + K % 2
    ldb = N if lb == MN else K + K % 2
    return tm.gemm_bf16_layout_plan(la, lb, variant, 1, M, N, K, 256, lda, 0, 256, ldb, 0, 256,
                                    N, 0, 0)[1]


# Shapes whose MN extents are multiples of 8 (the ring kernel takes every layout), with
# ragged tiles, a K tail within a block, K < 8 and K not a multiple of 8.
RING_SHAPES = [(128, 128, 128), (264, 520, 1000), (512, 384, 1027), (64, 1000, 8), (256, 256, 4),
               (136, 72, 77), (520, 264, 300)]


@pytest.mark.parametrize("la,lb", LAYOUTS)
@pytest.mark.parametrize("variant", [tm.GEMM_VARIANT_AUTO, tm.GEMM_VARIANT_RING4,
                                     tm.GEMM_VARIANT_SIMPLE])
@pytest.mark.parametrize("M,N,K", RING_SHAPES)
def test_layout_integer_exact(la, lb, variant, M, N, K):
    A = synth.integers(M, K, 501 + M + K)
    B = synth.integers(N, K, 502 + N + K)
    if variant == tm.GEMM_VARIANT_AUTO:
        assert plan_name(A, B, la, lb, variant) == "ring4_256"
    for out_dtype in (OUT_FP32, OUT_BF16):
        got = run_layout(A, B, la, lb, out_dtype, variant)
        assert_exact(got, A, B, out_dtype, what=f"layouts {la}{lb} variant {variant} {M}x{N}x{K}")


# MN extents that are not multiples of 8: AUTO falls back to the general kernel.
@pytest.mark.parametrize("la,lb", LAYOUTS)
@pytest.mark.parametrize("M,N,K", [(300, 200, 264), (33, 77, 40), (257, 130, 1001)])
def test_layout_general_fallback(la, lb, M, N, K):
    A = synth.integers(M, K, 511 + M)
    B = synth.integers(N, K, 512 + N)
    expect_ring = (la == KM or M % 8 == 0) and (lb == KM or N % 8 == 0)
    name = plan_name(A, B, la, lb, tm.GEMM_VARIANT_AUTO)
    assert name == ("ring4_256" if expect_ring else "simple_64"), name
    for out_dtype in (OUT_FP32, OUT_BF16):
        got = run_layout(A, B, la, lb, out_dtype)
        assert_exact(got, A, B, out_dtype, what=f"layouts {la}{lb} {M}x{N}x{K} ({name})")


@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_layout_padded_pitches_and_offsets(la, lb):
    """Pitches beyond the extent (padding holds NaN and must never be read) and operands that
    start 4 bytes into an allocation."""
    M, N, K = 264, 136, 520
    A = synth.integers(M, K, 521)
    B = synth.integers(N, K, 522)
    lda = (M + 24) if la == MN else (K + 10)
    ldb = (N + 8) if lb == MN else (K + 2)
    got = run_layout(A, B, la, lb, OUT_FP32, lda=lda, ldb=ldb, a_offset=2, b_offset=6)
    assert_exact(got, A, B, OUT_FP32, what=f"padded layouts {la}{lb}")


@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_layout_batched(la, lb):
    batch, M, N, K = 3, 136, 264, 200
    As = [synth.integers(M, K, 530 + b) for b in range(batch)]
    Bs = [synth.integers(N, K, 540 + b) for b in range(batch)]
    Ad = [mn_major(a) if la == MN else a for a in As]
    Bd = [mn_major(b) if lb == MN else b for b in Bs]
    sA, sB = Ad[0].size + 8, Bd[0].size + 16
    Abuf = np.zeros(batch * sA, np.uint16)
    Bbuf = np.zeros(batch * sB, np.uint16)
    for b in range(batch):
        Abuf[b * sA:b * sA + Ad[b].size] = Ad[b].reshape(-1)
        Bbuf[b * sB:b * sB + Bd[b].size] = Bd[b].reshape(-1)
    C = empty_out(M, N, OUT_FP32, batch=batch)
    tm.gemm_bf16_layout(la, lb, tm.GEMM_VARIANT_AUTO, batch, M, N, K, to_device(Abuf),
                        Ad[0].shape[1], sA, to_device(Bbuf), Bd[0].shape[1], sB, C, N, M * N,
                        OUT_FP32)
    h = out_to_host(C, M, N, N, OUT_FP32, batch=batch)
    for b in range(batch):
        assert_exact(h[b], As[b], Bs[b], OUT_FP32, what=f"batch item {b}")


def test_layout_k_zero():
    import torch
    C = empty_out(40, 48, OUT_FP32, fill=3)
    dummy = torch.zeros(64, dtype=torch.bfloat16, device="cuda")
    tm.gemm_bf16_layout(MN, MN, 0, 1, 40, 48, 0, dummy, 40, 0, dummy, 48, 0, C, 48, 0, OUT_FP32)
    assert np.all(out_to_host(C, 40, 48, 48, OUT_FP32) == 0)


def test_layout_unsupported_variant_raises():
    A = synth.integers(64, 64, 1)
    with pytest.raises(tm.GemmError) as e:
        run_layout(A, A, KM, MN, OUT_FP32, variant=tm.GEMM_VARIANT_SPECIALIZED)
    assert e.value.status == tm.GEMM_ERR_UNSUPPORTED


@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_layout_full_size_sampled(la, lb):
    """4096^3 in each layout (C = A B for MN-major B): sampled rows against the oracle, with
    the square workload's values (within the bound) and with integers (bitwise)."""
    M = N = K = 4096
    rows = sorted({0, 1, 255, 256, 2047, 4095} | set(np.random.default_rng(5).integers(0, M, 10).tolist()))
    A, B = synth.make_operands("square_4096")
    got = run_layout(A, B, la, lb, OUT_FP32)
    C, Mag = oracle.gemm(A, B, rows=rows)
    r = ck.check(got[rows], C, Mag, K, OUT_FP32)
    assert r["ok"], r
    Ai, Bi = synth.integers(M, K, 551), synth.integers(N, K, 552)
    got = run_layout(Ai, Bi, la, lb, OUT_BF16)
    assert_exact(got[rows], Ai, Bi, OUT_BF16, rows=rows, what=f"4096^3 layouts {la}{lb}")
