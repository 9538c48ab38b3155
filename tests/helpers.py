"""Test helpers: moving bf16 bit patterns to and from the GPU, and running one GEMM through
the C ABI (via the ctypes binding) on torch-allocated device memory."""
import numpy as np

import tiled_matmul_amd as tm

OUT_FP32, OUT_BF16 = tm.GEMM_OUT_FP32, tm.GEMM_OUT_BF16


def to_device(bits: np.ndarray, offset_elems: int = 0):
    """uint16 bf16 patterns -> a cuda bfloat16 tensor.  ``offset_elems`` > 0 returns a view
    that starts that many elements into a fresh buffer (for misaligned-pointer cases)."""
    import torch
    flat = np.ascontiguousarray(bits).reshape(-1)
    buf = torch.empty(flat.size + offset_elems + 8, dtype=torch.int16, device="cuda")
    buf[offset_elems:offset_elems + flat.size].copy_(torch.from_numpy(flat.view(np.int16)))
    return buf.view(torch.bfloat16)[offset_elems:offset_elems + flat.size].view(bits.shape)


def empty_out(rows: int, ldc: int, out_dtype: int, batch: int = 1, fill=None):
    import torch
    dt = torch.float32 if out_dtype == OUT_FP32 else torch.int16
    t = torch.empty(batch * rows * ldc + 8, dtype=dt, device="cuda")
    if fill is not None:
        t.fill_(fill)
    return t


def out_to_host(C, rows: int, N: int, ldc: int, out_dtype: int, batch: int = 1):
    """Device output buffer -> (batch, rows, N) numpy (float32, or uint16 bf16 patterns)."""
    import torch
    torch.cuda.synchronize()
    h = C.cpu().numpy()
    n = batch * rows * ldc
    h = h[:n].reshape(batch, rows, ldc)[:, :, :N]
    if out_dtype == OUT_BF16:
        h = h.view(np.uint16)
    return h if batch > 1 else h[0]


def run_gemm(A_bits, B_bits, K, out_dtype, variant=tm.GEMM_VARIANT_AUTO, ldc=None,
             a_offset=0, b_offset=0, sentinel=None):
    """One GEMM through gemm_bf16_variant with A (M x lda) and B (N x ldb) bit arrays whose
    first K columns are the operands.  Returns the host copy of C (M x N)."""
    M, lda = A_bits.shape
    N, ldb = B_bits.shape
    ldc = N if ldc is None else ldc
    A = to_device(A_bits, a_offset)
    B = to_device(B_bits, b_offset)
    C = empty_out(M, ldc, out_dtype, fill=sentinel)
    tm.gemm_bf16_variant(variant, 1, M, N, K, A, lda, 0, B, ldb, 0, C, ldc, 0, out_dtype)
    return out_to_host(C, M, N, ldc, out_dtype)
