"""The largest row pitches the planner accepts: every K-major kernel addresses a tile's rows
with 32-bit offsets from a 64-bit tile base, so the planner admits pitches up to the point where
one tile's rows span 2^31 bytes, while the operand itself may be much larger.  At pitches just
below each kernel's limit (operands of 2.5-5 GB, NaN between the rows), integer inputs must
match the oracle bitwise.  (Every offset was checked against its resource on the host first:
at these pitches a tile's last row starts below 2^31 bytes from the tile's base.)"""
import numpy as np
import pytest

import tiled_matmul_amd as tm
from tiled_matmul_amd import synth

from helpers import OUT_FP32, OUT_BF16, empty_out, out_to_host
from test_gpu_parity import assert_exact

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.empty_cache()


def strided(bits, ld):
    """A device bf16 buffer of rows x ld elements: the first K of each row from `bits`, the
    rest the bf16 NaN pattern."""
    import torch
    rows, K = bits.shape
    t = torch.full((rows, ld), 0x7FC0, dtype=torch.int16, device="cuda")
    t[:, :K] = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()
    return t.view(torch.bfloat16).reshape(-1)


# (variant, rows per tile that bound the pitch): 256-row tiles (ring, specialised, ping-pong,
# A-in-registers, fixed roles); 128-row tiles (persistent and pipelined at M = 300, the general
# MFMA kernel, which addresses with 64-bit pointers and has no limit of its own)
TILED = [(tm.VARIANTS[n], r) for n, r in [("ring4", 256), ("ring8", 256), ("specialized", 256),
                                           ("pingpong", 256), ("dtv", 256), ("roles", 256),
                                           ("persistent", 128), ("pipelined", 128), ("mfma", 128)]]


@pytest.mark.parametrize("variant,rows", TILED)
def test_tiled_kernels_at_the_largest_pitch(variant, rows):
    import torch
    M, N, K = 300, 264, 64
    ld = ((1 << 31) // (2 * rows) - 1) // 8 * 8   # the largest multiple of 8 below the limit
    A, B = synth.integers(M, K, 971), synth.integers(N, K, 972)
    dA, dB = strided(A, ld), strided(B, ld)
    for od in (OUT_FP32, OUT_BF16):
        rc = tm.gemm_bf16_plan(variant, 1, M, N, K, dA, ld, 0, dB, ld, 0, dA, N, 0, od, 256)
        assert rc[0] == 0, (variant, rc)
        C = empty_out(M, N, od, fill=float("nan") if od == OUT_FP32 else -1)
        tm.gemm_bf16_variant(variant, 1, M, N, K, dA, ld, 0, dB, ld, 0, C, N, 0, od)
        assert_exact(out_to_host(C, M, N, N, od), A, B, K, od, what=f"variant {variant} ld {ld}")
    del dA, dB
    torch.cuda.empty_cache()


def test_skinny_m_at_the_largest_pitch():
    import torch
    M, N, K = 16, 40, 1024
    ld = ((1 << 31) // (2 * 16) - 1) // 8 * 8
    A, B = synth.integers(M, K, 973), synth.integers(N, K, 974)
    dA, dB = strided(A, ld), strided(B, ld)
    for m in (1, 5, 16):
        C = empty_out(m, N, OUT_FP32, fill=float("nan"))
        tm.gemm_bf16(m, N, K, dA, ld, dB, ld, C, N, OUT_FP32)
        assert_exact(out_to_host(C, m, N, N, OUT_FP32), A[:m], B, K, OUT_FP32, what=f"skinny M={m} ld {ld}")
    del dA, dB
    torch.cuda.empty_cache()


def test_largest_batch():
    """The largest batch the ABI accepts (65535 items; one more is an argument error), tiny
    ragged GEMMs through gemm_bf16_strided_batched: 200 sampled items (the first and last
    included) against the oracle bitwise, and every item finite."""
    import torch
    batch, M, N, K = 65535, 20, 24, 40
    rng = np.random.default_rng(7)
    A = rng.integers(-4, 5, size=(batch, M, K), dtype=np.int8)
    B = rng.integers(-4, 5, size=(batch, N, K), dtype=np.int8)
    bits = lambda x: (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)   # exact for small ints
    dA = torch.from_numpy(bits(A).view(np.int16).reshape(-1)).cuda().view(torch.bfloat16)
    dB = torch.from_numpy(bits(B).view(np.int16).reshape(-1)).cuda().view(torch.bfloat16)
    C = empty_out(M, N, OUT_FP32, batch=batch, fill=float("nan"))
    rc = tm.gemm_bf16_plan(0, batch + 1, M, N, K, dA, K, M * K, dB, K, N * K, C, N, M * N, OUT_FP32, 256)
    assert rc[0] == tm.GEMM_ERR_ARG
    tm.gemm_bf16_strided_batched(batch, M, N, K, dA, K, M * K, dB, K, N * K, C, N, M * N, OUT_FP32)
    got = out_to_host(C, M, N, N, OUT_FP32, batch=batch)
    assert np.isfinite(got).all()
    items = sorted({0, batch - 1} | set(rng.integers(0, batch, 198).tolist()))
    for b in items:
        assert_exact(got[b], bits(A[b]), bits(B[b]), K, OUT_FP32, what=f"batch item {b}")
