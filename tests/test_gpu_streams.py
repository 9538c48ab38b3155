"""Calls on two streams at once: the library launches on the stream it is given (torch's
current stream through the binding) and gemm_bf16 keeps no device state between calls, so two GEMMs
issued back to back on different streams, three times over, both match the oracle bitwise on
integer inputs."""
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


def test_two_streams_at_once():
    import torch
    shapes = [(2000, 1500, 1032, OUT_FP32), (8, 4096, 4096, OUT_BF16)]
    ins, outs = [], []
    for i, (M, N, K, od) in enumerate(shapes):
        A, B = synth.integers(M, K, 950 + i), synth.integers(N, K, 960 + i)
        ins.append((A, B, to_device(A), to_device(B)))
        outs.append(empty_out(M, N, od, fill=float("nan") if od == OUT_FP32 else -1))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        for (M, N, K, od), (_, _, dA, dB), C, s in zip(shapes, ins, outs, streams):
            with torch.cuda.stream(s):
                tm.gemm_bf16(M, N, K, dA, K, dB, K, C, N, od)
        torch.cuda.synchronize()
        for (M, N, K, od), (A, B, _, _), C in zip(shapes, ins, outs):
            assert_exact(out_to_host(C, M, N, N, od), A, B, K, od, what=f"stream call {rep}: {M}x{N}x{K}")
            C.fill_(float("nan") if od == OUT_FP32 else -1)
