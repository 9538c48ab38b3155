"""The library's launches captured in a HIP graph (as bench.py captures the decode GEMV to time
it): every replay gives the same bits as the eager call, with the program's own eager work and
synchronizations between replays, for the skinny-M paths and a persistent tiled GEMM.  No
library call records a memset or allocates, so the graph holds only the kernels."""
import numpy as np
import pytest

import tiled_matmul_amd as tm
from tiled_matmul_amd import synth

from helpers import OUT_FP32, OUT_BF16, empty_out, out_to_host, to_device
from test_gpu_parity import assert_exact

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield


@pytest.mark.parametrize("M,N,K,out_dtype", [(1, 4096, 4096, OUT_FP32), (16, 4096, 4096, OUT_FP32),
                                             (3, 1000, 1032, OUT_BF16), (1000, 1200, 520, OUT_FP32)])
def test_graph_replays_match_the_eager_call(M, N, K, out_dtype):
    import torch
    A_bits, B_bits = synth.integers(M, K, 901 + M), synth.integers(N, K, 902 + M)
    A, B = to_device(A_bits), to_device(B_bits)
    C_eager = empty_out(M, N, out_dtype, fill=0)
    tm.gemm_bf16(M, N, K, A, K, B, K, C_eager, N, out_dtype)
    eager = out_to_host(C_eager, M, N, N, out_dtype)
    assert_exact(eager, A_bits, B_bits, K, out_dtype, what=f"eager {M}x{N}x{K}")

    C = empty_out(M, N, out_dtype, fill=0)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=s):
        tm.gemm_bf16(M, N, K, A, K, B, K, C, N, out_dtype)
    for rep in range(3):
        C.fill_(float("nan") if out_dtype == OUT_FP32 else -1)   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        got = out_to_host(C, M, N, N, out_dtype)
        assert np.array_equal(got.view(np.uint32 if out_dtype == OUT_FP32 else np.uint16),
                              eager.view(np.uint32 if out_dtype == OUT_FP32 else np.uint16)), f"replay {rep}"
