"""GPU parity of split K (gemm_bf16_splitk) against the CPU oracle.

Integer-valued inputs keep every partial sum, and the sum of the partials, exact in fp32, so
the split result must equal the oracle bitwise (fp32 out) or the oracle's round-to-nearest-
even bf16 (bf16 out), for every split count.  Normal-valued inputs check the bound and that
a split run is deterministic.  Workspaces start filled with NaN: the result must not depend
on what they hold.
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
BIG = 1 << 62


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield


def workspace(nbytes):
    import torch
    return torch.full((max(nbytes, 16) // 4 + 4,), float("nan"), dtype=torch.float32, device="cuda")


def device_operand(X, layout):
    """K-major bits (rows x K) -> device array in `layout` (K-major pitch even, pad NaN)."""
    rows, K = X.shape
    if layout == MN:
        return np.ascontiguousarray(X.T)
    out = np.full((rows, K + K % 2), synth.PAD_BITS, dtype=np.uint16)
    out[:, :K] = X
    return out


def run_splitk(A, B, splits, out_dtype, la=KM, lb=KM, ldc=None, c_offset=0):
    """Split-K GEMM of K-major bit arrays A (M x K), B (N x K) into C with pitch ldc (default
    N) starting c_offset elements into its buffer.  Returns (C host, S)."""
    (M, K), (N, _) = A.shape, B.shape
    ldc = N if ldc is None else ldc
    Ad, Bd = device_operand(A, la), device_operand(B, lb)
    Ag, Bg = to_device(Ad), to_device(Bd)
    Cbuf = empty_out(M, ldc, out_dtype, fill=7)
    C = Cbuf[c_offset:]
    rc, S, kname, _ = tm.gemm_bf16_splitk_plan(la, lb, splits, 1, M, N, K, Ag, Ad.shape[1], 0, Bg,
                                               Bd.shape[1], 0, C, ldc, 0, out_dtype, 1 << 12, BIG)
    assert rc == 0, tm.gemm_bf16_status_string(rc)
    need = S * M * N * 4
    tm.gemm_bf16_splitk(la, lb, splits, 1, M, N, K, Ag, Ad.shape[1], 0, Bg, Bd.shape[1], 0, C,
                        ldc, 0, out_dtype, workspace(need), need)
    import torch
    torch.cuda.synchronize()
    h = Cbuf.cpu().numpy()
    h = (h if out_dtype == OUT_FP32 else h.view(np.uint16))[c_offset:c_offset + M * ldc]
    h = h.reshape(M, ldc)
    assert np.all(h[:, N:] == 7), "row padding of C was written"
    return np.ascontiguousarray(h[:, :N]), S


def assert_exact(got, A, B, out_dtype, rows=None, what=""):
    C, _ = oracle.gemm(A, B, rows=rows)
    exp = C.astype(np.float32) if out_dtype == OUT_FP32 else oracle.round_bf16(C)
    r = ck.check_exact(got, exp, out_dtype)
    assert r["ok"], f"{what}: {r}"


# (M, N, K): aligned K, a K tail inside the last block (K % 64 != 0), a K tail that is not a
# multiple of 8 (the element-wise tail step, in the last range only), ragged M and N.
# N = 130: the reduction's one-element-per-thread form (N % 4 != 0).
SHAPES = [(256, 256, 1024), (264, 136, 1027), (520, 264, 1000), (128, 256, 4100), (136, 72, 77),
          (200, 130, 2100)]


@pytest.mark.parametrize("splits", [1, 2, 3, 7])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_splitk_integer_exact(M, N, K, splits):
    A = synth.integers(M, K, 601 + M + K)
    B = synth.integers(N, K, 602 + N + K)
    for out_dtype in (OUT_FP32, OUT_BF16):
        got, S = run_splitk(A, B, splits, out_dtype)
        assert S == min(splits, -(-K // 64))
        assert_exact(got, A, B, out_dtype, what=f"{M}x{N}x{K} splits {splits}")


@pytest.mark.parametrize("ldc_pad,c_offset", [(2, 0), (0, 1), (6, 3)])
def test_splitk_output_pitch_and_alignment(ldc_pad, c_offset):
    """C rows with padding, and C not 16-byte aligned: the reduction's scalar-store forms."""
    M, N, K = 264, 136, 1027
    A = synth.integers(M, K, 681)
    B = synth.integers(N, K, 682)
    for out_dtype in (OUT_FP32, OUT_BF16):
        got, S = run_splitk(A, B, 3, out_dtype, ldc=N + ldc_pad, c_offset=c_offset)
        assert_exact(got, A, B, out_dtype, what=f"ldc {N + ldc_pad} offset {c_offset}")


@pytest.mark.parametrize("la,lb", [(KM, MN), (MN, KM), (MN, MN)])
@pytest.mark.parametrize("M,N,K", [(264, 520, 1000), (136, 72, 1027)])
def test_splitk_layouts_integer_exact(la, lb, M, N, K):
    A = synth.integers(M, K, 611 + M)
    B = synth.integers(N, K, 612 + N)
    for out_dtype in (OUT_FP32, OUT_BF16):
        got, S = run_splitk(A, B, 3, out_dtype, la, lb)
        assert S == 3
        assert_exact(got, A, B, out_dtype, what=f"layouts {la}{lb} {M}x{N}x{K}")


def test_splitk_batched():
    import torch
    batch, M, N, K, S = 3, 136, 264, 2000, 5
    As = [synth.integers(M, K, 620 + b) for b in range(batch)]
    Bs = [synth.integers(N, K, 630 + b) for b in range(batch)]
    sA, sB = M * K + 8, N * K + 16
    Abuf = np.zeros(batch * sA, np.uint16)
    Bbuf = np.zeros(batch * sB, np.uint16)
    for b in range(batch):
        Abuf[b * sA:b * sA + M * K] = As[b].reshape(-1)
        Bbuf[b * sB:b * sB + N * K] = Bs[b].reshape(-1)
    C = empty_out(M, N, OUT_FP32, batch=batch, fill=7)
    nbytes = S * batch * M * N * 4
    tm.gemm_bf16_splitk(KM, KM, S, batch, M, N, K, to_device(Abuf), K, sA, to_device(Bbuf), K, sB,
                        C, N, M * N, OUT_FP32, workspace(nbytes), nbytes)
    torch.cuda.synchronize()
    h = out_to_host(C, M, N, N, OUT_FP32, batch=batch)
    for b in range(batch):
        assert_exact(h[b], As[b], Bs[b], OUT_FP32, what=f"batch item {b}")


def test_splitk_deterministic_and_within_bound():
    """Normal values (the FFN weights' distributions): two runs give the same bits, the
    result is within the bound, and it matches the unsplit kernel within the bound too."""
    M, N, K = 256, 512, 8192
    A = synth.normal(M, K, 641)
    B = synth.normal(N, K, 642, sigma=0.02)
    C_ref, Mag = oracle.gemm(A, B)
    for out_dtype in (OUT_FP32, OUT_BF16):
        got1, S = run_splitk(A, B, 0, out_dtype)
        got2, _ = run_splitk(A, B, 0, out_dtype)
        assert S > 1
        assert np.array_equal(got1.view(np.uint32 if out_dtype == OUT_FP32 else np.uint16),
                              got2.view(np.uint32 if out_dtype == OUT_FP32 else np.uint16))
        r = ck.check(got1, C_ref, Mag, K, out_dtype)
        assert r["ok"], r


def test_splitk_one_range_is_the_plain_call():
    """S == 1 (no workspace at all) gives exactly gemm_bf16_layout's bits."""
    M, N, K = 300, 260, 520
    A, B = synth.uniform(M, K, 651), synth.uniform(N, K, 652)
    Ag, Bg = to_device(device_operand(A, KM)), to_device(device_operand(B, KM))
    ld = K + K % 2
    C1 = empty_out(M, N, OUT_FP32)
    C2 = empty_out(M, N, OUT_FP32)
    tm.gemm_bf16_splitk(KM, KM, 1, 1, M, N, K, Ag, ld, 0, Bg, ld, 0, C1, N, 0, OUT_FP32, None, 0)
    tm.gemm_bf16_layout(KM, KM, 0, 1, M, N, K, Ag, ld, 0, Bg, ld, 0, C2, N, 0, OUT_FP32)
    h1, h2 = out_to_host(C1, M, N, N, OUT_FP32), out_to_host(C2, M, N, N, OUT_FP32)
    assert np.array_equal(h1.view(np.uint32), h2.view(np.uint32))


def test_splitk_small_workspace_is_rejected_and_launches_nothing():
    M, N, K = 256, 256, 1024
    A = synth.integers(M, K, 661)
    Ag, Bg = to_device(A), to_device(A)
    C = empty_out(M, N, OUT_FP32, fill=7)
    nbytes = 2 * M * N * 4 - 16
    with pytest.raises(tm.GemmError) as e:
        tm.gemm_bf16_splitk(KM, KM, 2, 1, M, N, K, Ag, K, 0, Bg, K, 0, C, N, 0, OUT_FP32,
                            workspace(nbytes), nbytes)
    assert e.value.status == tm.GEMM_ERR_ARG
    assert np.all(out_to_host(C, M, N, N, OUT_FP32) == 7)


@pytest.mark.parametrize("name,M,N,K,sigma_b,out_dtype", [
    ("long_k_1024x1024x16384", 1024, 1024, 16384, 1.0, OUT_FP32),
    ("ffn_down_256x4096x14336", 256, 4096, 14336, 0.02, OUT_BF16),
])
def test_splitk_long_k_sampled(name, M, N, K, sigma_b, out_dtype):
    """Shapes with few tiles and a long K, in the automatic split count: sampled rows of C
    against the oracle (within the bound), and integers (bitwise)."""
    rows = sorted({0, 1, 255, M - 1} | set(np.random.default_rng(7).integers(0, M, 6).tolist()))
    A = synth.normal(M, K, 671)
    B = synth.normal(N, K, 672, sigma=sigma_b)
    got, S = run_splitk(A, B, 0, out_dtype)
    assert S == 16
    C, Mag = oracle.gemm(A, B, rows=rows)
    r = ck.check(got[rows], C, Mag, K, out_dtype)
    assert r["ok"], r
    Ai, Bi = synth.integers(M, K, 673, lo=-2, hi=2), synth.integers(N, K, 674, lo=-2, hi=2)
    got, _ = run_splitk(Ai, Bi, 0, out_dtype)
    assert_exact(got[rows], Ai, Bi, out_dtype, rows=rows, what=name)
