"""gemm_bf16_splitk_noalloc (split K with the library's static scratch) against
gemm_bf16_splitk with a caller workspace: bitwise equal for the same split count, on two
calls in a row, the second with a smaller problem; a request beyond the scratch is refused."""
import numpy as np
import pytest

import tiled_matmul_amd as tm
from tiled_matmul_amd import synth

from helpers import to_device, empty_out, out_to_host

pytestmark = pytest.mark.gpu


def _pair(M, N, K, splits, out_dtype, seed, batch=1):
    import torch
    A = synth.normal(batch * M, K, seed).reshape(batch, M, K)
    B = synth.normal(batch * N, K, seed + 1).reshape(batch, N, K)
    Ad, Bd = to_device(A), to_device(B)
    sA, sB, sC = (M * K, N * K, M * N) if batch > 1 else (0, 0, 0)
    rc, S, _, _ = tm.gemm_bf16_splitk_plan(0, 0, splits, batch, M, N, K, Ad, K, sA, Bd, K, sB, Ad, N, sC,
                                           out_dtype, 1 << 12, tm.GEMM_SCRATCH_BYTES)
    assert rc == 0
    ws = torch.empty(max(S * batch * M * N, 4), dtype=torch.float32, device="cuda")
    C1 = empty_out(M, N, out_dtype, batch=batch, fill=float("nan") if out_dtype == 0 else -1)
    C2 = empty_out(M, N, out_dtype, batch=batch, fill=float("nan") if out_dtype == 0 else -1)
    tm.gemm_bf16_splitk(0, 0, splits, batch, M, N, K, Ad, K, sA, Bd, K, sB, C1, N, sC, out_dtype, ws,
                        ws.numel() * 4)
    tm.gemm_bf16_splitk_noalloc(0, 0, splits, batch, M, N, K, Ad, K, sA, Bd, K, sB, C2, N, sC, out_dtype)
    h1 = out_to_host(C1, M, N, N, out_dtype, batch=batch)
    h2 = out_to_host(C2, M, N, N, out_dtype, batch=batch)
    return S, h1, h2


@pytest.mark.parametrize("out_dtype", [tm.GEMM_OUT_FP32, tm.GEMM_OUT_BF16])
def test_noalloc_matches_workspace_entry_point(out_dtype):
    # first call: the FFN down projection for 256 tokens with the automatic count (16 ranges,
    # 64 MiB of partials: the whole scratch); then a smaller, ragged one with 3 ranges
    for (M, N, K, splits, seed) in ((256, 4096, 14336, 0, 11), (264, 136, 1028, 3, 13)):
        S, h1, h2 = _pair(M, N, K, splits, out_dtype, seed)
        assert S > 1
        a = h1.view(np.uint32) if out_dtype == 0 else h1
        b = h2.view(np.uint32) if out_dtype == 0 else h2
        assert np.array_equal(a, b), (M, N, K, S)
        assert np.isfinite(h1.astype(np.float32) if out_dtype == 0 else h1.astype(np.float32)).all()


def test_noalloc_refuses_more_than_the_scratch():
    A = to_device(np.zeros((1024, 4096), np.uint16))
    B = to_device(np.zeros((4096, 4096), np.uint16))
    C = empty_out(1024, 4096, 0)
    # 8 ranges of 1024 x 4096 fp32 partials = 128 MiB > 64 MiB
    with pytest.raises(tm.GemmError) as e:
        tm.gemm_bf16_splitk_noalloc(0, 0, 8, 1, 1024, 4096, 4096, A, 4096, 0, B, 4096, 0, C, 4096, 0, 0)
    assert e.value.status == tm.GEMM_ERR_SCRATCH
