"""gemm_bf16_streamk (stream-K with atomic work claiming) on MI355X against the oracle:
integer-valued inputs bitwise (every fp32 partial sum is exact, so the cut tiles' fixed-order
sums must equal the oracle exactly), the workloads' values under the bound, determinism, and
the counters left at zero after every call."""
import numpy as np
import pytest

import tiled_matmul_amd as tm
from tiled_matmul_amd import synth

from helpers import OUT_BF16, OUT_FP32, empty_out, out_to_host, to_device
from test_gpu_parity import assert_bound, assert_exact

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield


def run_streamk(mode, A_bits, B_bits, K, out_dtype, batch=1, ws=None, C=None):
    """One call; returns (C host, workspace tensor, plan)."""
    import torch
    if batch == 1:
        M, lda = A_bits.shape
        N, ldb = B_bits.shape
    else:
        _, M, lda = A_bits.shape
        _, N, ldb = B_bits.shape
    sA, sB, sC = (M * lda, N * ldb, M * N) if batch > 1 else (0, 0, 0)
    A, B = to_device(A_bits), to_device(B_bits)
    if C is None:
        C = empty_out(M, N, out_dtype, batch=batch, fill=float("nan") if out_dtype == OUT_FP32 else -1)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    plan = tm.gemm_bf16_streamk_plan(mode, batch, M, N, K, A, lda, sA, B, ldb, sB, C, N, sC, out_dtype, cus)
    assert plan[0] == 0, plan
    if ws is None:
        ws = torch.zeros(max(plan[1] // 4, 64), dtype=torch.int32, device="cuda")
    tm.gemm_bf16_streamk(mode, batch, M, N, K, A, lda, sA, B, ldb, sB, C, N, sC, out_dtype, ws, ws.numel() * 4)
    return out_to_host(C, M, N, N, out_dtype, batch=batch), ws, plan


def counters_zero(ws, plan):
    """Every word of the 16 KB counter region (claim and exit counters, the words that hand each
    workgroup's claims to its waves, the tiles' arrival counters) is zero again after the call."""
    import torch
    torch.cuda.synchronize()
    h = ws[:16384 // 4].cpu().numpy()
    nz = np.nonzero(h)[0]
    if nz.size:
        print("nonzero counter words:", nz[:20].tolist(), h[nz[:20]].tolist())
    return nz.size == 0


# (M, N, K, mode, what the plan must hold): more tiles than compute units with a remainder (the
# last wave as stream-K slots, ragged K included), fewer tiles than compute units cut along K
# (GEMM_STREAMK_ALL), data-parallel only, and K shorter than a slot.
CASES = [
    (4352, 4352, 512, tm.GEMM_STREAMK_AUTO, "cut"),        # 289 tiles: all cut, slots span 2-3 tiles
    (4352, 4352, 260, tm.GEMM_STREAMK_AUTO, "cut"),        # K mod 8 != 0: ragged tail in the last piece
    (6144, 6400, 136, tm.GEMM_STREAMK_AUTO, "hybrid"),     # 600 tiles: 256 whole + 344 cut
    (1000, 1000, 1000, tm.GEMM_STREAMK_ALL, "all"),        # 16 tiles cut into 4 pieces each
    (520, 264, 2056, tm.GEMM_STREAMK_ALL, "all"),          # 6 tiles, long K, ragged in M and N
    (300, 520, 1032, tm.GEMM_STREAMK_DP, "dp"),
    (600, 700, 136, tm.GEMM_STREAMK_ALL, "all"),           # 9 tiles, 3 K blocks: one piece per tile
]


@pytest.mark.parametrize("out_dtype", [OUT_FP32, OUT_BF16])
@pytest.mark.parametrize("M,N,K,mode,kind", CASES)
def test_streamk_integer_exact(M, N, K, mode, kind, out_dtype):
    lda = K + (K % 2)
    A = synth.integers(M, K, 700 + K, ld=lda)
    B = synth.integers(N, K, 701 + K, ld=lda)
    got, ws, plan = run_streamk(mode, A, B, K, out_dtype)
    _, _, dp, sk, slots, _ = plan
    if kind == "hybrid":
        assert dp == 256 and sk > 0
    elif kind == "cut":
        assert dp == 0 and sk == 289
    elif kind == "all":
        assert dp == 0 and sk > 0
    else:
        assert sk == 0
    assert_exact(got, A, B, K, out_dtype, what=f"streamk {kind} {M}x{N}x{K}")
    assert counters_zero(ws, plan)


def test_streamk_repeated_calls_share_a_workspace():
    """Three calls on one workspace (the counters each call leaves at zero are what the next one
    starts from), the second with another shape and mode."""
    A = synth.integers(1000, 1000, 711)
    B = synth.integers(1000, 1000, 712)
    A2 = synth.integers(4352, 264, 713)
    B2 = synth.integers(4352, 264, 714)
    import torch
    ws = torch.zeros((160 << 20) // 4, dtype=torch.int32, device="cuda")
    # the partials of the first call (after the 16 KB of counters) are what the later calls find
    # in the workspace
    g1, _, p1 = run_streamk(tm.GEMM_STREAMK_ALL, A, B, 1000, OUT_FP32, ws=ws)
    g2, _, p2 = run_streamk(tm.GEMM_STREAMK_AUTO, A2, B2, 264, OUT_FP32, ws=ws)
    g3, _, p3 = run_streamk(tm.GEMM_STREAMK_ALL, A, B, 1000, OUT_FP32, ws=ws)
    assert_exact(g1, A, B, 1000, OUT_FP32, what="first")
    assert_exact(g2, A2, B2, 264, OUT_FP32, what="second")
    assert np.array_equal(g1.view(np.uint32), g3.view(np.uint32))
    assert counters_zero(ws, p1) and counters_zero(ws, p2)


def test_streamk_batched():
    batch, M, N, K = 5, 520, 264, 1000
    A = np.stack([synth.integers(M, K, 720 + b) for b in range(batch)])
    B = np.stack([synth.integers(N, K, 730 + b) for b in range(batch)])
    for mode in (tm.GEMM_STREAMK_ALL, tm.GEMM_STREAMK_DP):
        got, ws, plan = run_streamk(mode, A, B, K, OUT_FP32, batch=batch)
        for b in range(batch):
            assert_exact(got[b], A[b], B[b], K, OUT_FP32, what=f"batch item {b} mode {mode}")
        assert counters_zero(ws, plan)


@pytest.mark.parametrize("mode", [tm.GEMM_STREAMK_AUTO, tm.GEMM_STREAMK_ALL])
def test_streamk_random_values_bound_and_determinism(mode):
    M, N, K = (4352, 4352, 1024) if mode == tm.GEMM_STREAMK_AUTO else (1000, 1000, 4096)
    A, B = synth.normal(M, K, 741), synth.normal(N, K, 742)
    g1, _, _ = run_streamk(mode, A, B, K, OUT_FP32)
    g2, _, _ = run_streamk(mode, A, B, K, OUT_FP32)
    assert np.array_equal(g1.view(np.uint32), g2.view(np.uint32))
    rows = sorted({0, 1, 255, 256, 511, M - 1} | set(np.random.default_rng(5).integers(0, M, 24).tolist()))
    assert_bound(g1[rows], A, B, K, OUT_FP32, rows=rows, what=f"streamk mode {mode}")


def test_streamk_errors():
    import torch
    A = to_device(synth.integers(512, 512, 1))
    C = empty_out(512, 512, OUT_FP32)
    rc, need = tm.gemm_bf16_streamk_plan(tm.GEMM_STREAMK_ALL, 1, 512, 512, 512, A, 512, 0, A, 512, 0, C, 512, 0,
                                         OUT_FP32)[:2]
    assert rc == 0 and need > 0
    ws = torch.zeros(need // 4 + 64, dtype=torch.int32, device="cuda")
    with pytest.raises(tm.GemmError) as e:
        tm.gemm_bf16_streamk(tm.GEMM_STREAMK_ALL, 1, 512, 512, 512, A, 512, 0, A, 512, 0, C, 512, 0, OUT_FP32,
                             ws, need - 4)
    assert e.value.status == tm.GEMM_ERR_ARG
    with pytest.raises(tm.GemmError) as e:
        tm.gemm_bf16_streamk(tm.GEMM_STREAMK_ALL, 1, 512, 512, 512, A, 512, 0, A, 512, 0, C, 512, 0, OUT_FP32,
                             ws.view(torch.int8)[4:], need)
    assert e.value.status == tm.GEMM_ERR_ARG
    with pytest.raises(tm.GemmError) as e:
        tm.gemm_bf16_streamk(tm.GEMM_STREAMK_ALL, 1, 512, 512, 512, A, 512, 0, A, 512, 0, C, 512, 0, OUT_FP32,
                             None, need)
    assert e.value.status == tm.GEMM_ERR_NULL


def test_streamk_workload_square_4352_sampled_rows():
    """The stream-K measurement's own workload at its full size (4352 x 4352 x 4096, 289 tiles,
    every tile cut in the automatic mode): sampled rows (every tile row, and rows either side of
    each tile boundary) under the bound on the workload's values, and bitwise on integers."""
    from test_gpu_parity import sample_rows
    name = "square_4352x4352x4096"
    w = synth.WORKLOADS[name]
    M, N, K, out_dtype = w["M"], w["N"], w["K"], w["out"]
    rows = sample_rows(M)
    A, B = synth.make_operands(name)
    got, ws, plan = run_streamk(tm.GEMM_STREAMK_AUTO, A, B, K, out_dtype)
    assert plan[3] == 289 and plan[2] == 0   # every tile cut
    assert np.isfinite(got).all()
    r = assert_bound(got[rows], A, B, K, out_dtype, rows=rows, what=name + " stream-K")
    print(f"{name}: rows={len(rows)} max_err_over_bound={r['max_err_over_bound']:.3g}")
    assert counters_zero(ws, plan)
    sa, sb = synth.seeds(w["cfg"])
    A, B = synth.integers(M, K, sa), synth.integers(N, K, sb)
    got, ws, plan = run_streamk(tm.GEMM_STREAMK_AUTO, A, B, K, out_dtype, ws=ws)
    assert_exact(got[rows], A, B, K, out_dtype, rows=rows, what=name + " stream-K integer")
    assert counters_zero(ws, plan)
