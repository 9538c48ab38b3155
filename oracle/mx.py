"""CPU oracle for the block-scaled 8-bit GEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use
it; it shares no code with the product path (``tiled_matmul_amd``), and the product never
imports it.

What it computes.  The page "Modern GPU Programming for MLSys：深度解读" (section "背景")
names low-precision block-scaled GEMM among the kernel families the book builds, without a
format; the reading taken is the OCP microscaling (MX) format: 8-bit float elements (E4M3 or
E5M2), and one E8M0 power-of-two scale per 32 consecutive k of a row.  The GEMM is the same
C = A * B^T as the bf16 one ([Notes] page, section "9 步优化"), on the scaled values:

    C[i][j] = sum_k (a(i,k) 2^(sa(i, k/32) - 127)) (b(j,k) 2^(sb(j, k/32) - 127))

Each element is decoded from its bit fields in binary64 (exact), multiplied by its block's
power of two (exact), and the dot products are taken with numpy's float64 matrix product (the
products are exact in binary64; the sum is rounded in binary64, far below the fp32 error the
GPU result is checked with).  Also returned: |A||B|^T of the scaled values and the
"exponent-field magnitude" F = sum_k 2^(ea + eb + sa + sb - 254) over the nonzero products
(ea, eb: the unbiased exponent fields of the two elements, 1 - bias for subnormals), which the
acceptance bound of the gfx950 scaled MFMA is written in (oracle/check.py, check_mx).
"""
from __future__ import annotations

import numpy as np

E4M3, E5M2 = 0, 1
_BIAS = {E4M3: 7, E5M2: 15}
_MBITS = {E4M3: 3, E5M2: 2}


def _fields(codes: np.ndarray, fmt: int):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    mb = _MBITS[fmt]
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> mb) & ((1 << (7 - mb)) - 1)
    m = c & ((1 << mb) - 1)
    return sign, e, m


def decode(codes, fmt: int) -> np.ndarray:
    """8-bit float codes -> binary64 values (OCP E4M3: no infinities, S.1111.111 NaN;
    E5M2: IEEE-style, exponent 31 is infinity (mantissa 0) or NaN)."""
    sign, e, m = _fields(codes, fmt)
    bias, mb = _BIAS[fmt], _MBITS[fmt]
    normal = sign * (1.0 + m / 2.0 ** mb) * np.exp2(e - bias)
    sub = sign * (m / 2.0 ** mb) * 2.0 ** (1 - bias)
    v = np.where(e == 0, sub, normal)
    if fmt == E4M3:
        v = np.where((e == 15) & (m == 7), np.nan, v)
    else:
        v = np.where(e == 31, np.where(m == 0, sign * np.inf, np.nan), v)
    return v


def exponent_field(codes, fmt: int) -> np.ndarray:
    """Unbiased exponent of each element's exponent field (1 - bias for zero/subnormal)."""
    _, e, _ = _fields(codes, fmt)
    return np.where(e == 0, 1 - _BIAS[fmt], e - _BIAS[fmt])


def decode_scale(s) -> np.ndarray:
    """E8M0 scale codes -> 2^(s - 127) (255 is NaN)."""
    s = np.asarray(s, dtype=np.uint8).astype(np.int64)
    return np.where(s == 255, np.nan, np.exp2(s - 127.0))


def scaled(codes, scales, fmt: int, K: int) -> np.ndarray:
    """Rows of an operand as binary64: element times its 32-block's scale (first K columns)."""
    v = decode(np.asarray(codes)[:, :K], fmt)
    s = decode_scale(np.asarray(scales)[:, :K // 32])
    return v * np.repeat(s, 32, axis=1)


def gemm(A, SA, B, SB, fa: int, fb: int, K: int | None = None, rows=None):
    """(C, Mag, F) for rows ``rows`` of C (all rows if None): C and Mag as in the module
    docstring, F the exponent-field magnitude.  A: M x lda codes, SA: M x lds scale codes;
    B, SB likewise (N rows)."""
    A, SA, B, SB = (np.asarray(x) for x in (A, SA, B, SB))
    K = A.shape[1] if K is None else K
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    if rows is not None:
        A, SA = A[rows], SA[rows]
    a = scaled(A, SA, fa, K)
    b = scaled(B, SB, fb, K)
    C = a @ b.T
    Mag = np.abs(a) @ np.abs(b).T
    F = exponent_magnitudes(A, SA, fa, K) @ exponent_magnitudes(B, SB, fb, K).T
    return C, Mag, F


def exponent_magnitudes(codes, scales, fmt: int, K: int) -> np.ndarray:
    """Per element of the first K columns: 2^(e + s - 127) (e: the element's unbiased
    exponent field, s: its 32-block's scale code), or 0 for a zero element.  The product of
    two rows of these, summed over k, is F."""
    codes = np.asarray(codes)[:, :K]
    v = decode(codes, fmt)
    s = np.repeat(decode_scale(np.asarray(scales)[:, :K // 32]), 32, axis=1)
    return np.where(v != 0, np.exp2(exponent_field(codes, fmt)) * s, 0.0)
