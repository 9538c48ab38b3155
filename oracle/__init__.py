"""CPU oracle for the tiled bf16 GEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this package.  The product path (``tiled_matmul_amd``) never imports it, and it
never imports the product path: the two share no code.  Inputs come from the seeded
generators in ``tiled_matmul_amd.synth`` only by way of the caller, who passes the same bf16
bit patterns to both sides.

The arithmetic lives in ``oracle/gemm_ref.c`` (plain C, built with gcc, OpenMP over output
rows): it decodes bf16 to binary64 and runs the i/j/k triple loop with k ascending, which is
the GEMM C = A * B^T that the page "读书笔记-《面向机器学习系统的现代 GPU 编程》" builds in
its section "9 步优化" (steps 1-3), plus the magnitude matrix |A| |B|^T that the acceptance
bound is written in.  This module is argument marshalling around that library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gemm_ref.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

# The exact gcc line; no -ffast-math and no -march=native (the library built here also runs
# on other hosts, and the k order / IEEE semantics must be kept).
BUILD_CMD = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
             "-o", _LIB_PATH, _SRC, "-lm"]


def build() -> str:
    """Compile oracle/gemm_ref.c into oracle/liboracle.so (always recompiles)."""
    global _lib
    subprocess.run(BUILD_CMD, check=True)
    _lib = None
    return _LIB_PATH


def default_threads() -> int:
    """Threads the oracle uses by default: the CPUs this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        return os.cpu_count() or 1


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_gemm_bf16.argtypes = [i64, i64, i64, p, i64, p, i64, p, p, i64, p, i64,
                                     ctypes.c_int]
    lib.oracle_gemm_bf16.restype = ctypes.c_int
    lib.oracle_round_bf16.argtypes = [ctypes.c_double]
    lib.oracle_round_bf16.restype = ctypes.c_uint16
    lib.oracle_round_bf16_array.argtypes = [p, p, i64]
    lib.oracle_round_bf16_array.restype = None
    lib.oracle_decode_bf16_array.argtypes = [p, p, i64]
    lib.oracle_decode_bf16_array.restype = None
    lib.oracle_version.restype = ctypes.c_int
    _lib = lib
    return lib


def _as_bits(x: np.ndarray) -> np.ndarray:
    if x.dtype != np.uint16:
        raise TypeError(f"bf16 operands are passed as uint16 bit patterns, got {x.dtype}")
    return x


def gemm(A: np.ndarray, B: np.ndarray, K: int | None = None, rows=None,
         nthreads: int | None = None, want_mag: bool = True):
    """C = A * B^T in binary64 and Mag = |A| |B|^T.

    ``A`` is an (M, lda) uint16 array of bf16 bit patterns whose first K columns are the
    operand (row pitch lda >= K); ``B`` likewise (N, ldb).  ``rows`` (optional) selects the
    rows of C to compute; the result then has len(rows) rows, in that order.
    Returns ``(C, Mag)`` as float64 arrays (Mag is None if ``want_mag`` is false).
    """
    A = np.ascontiguousarray(_as_bits(A))
    B = np.ascontiguousarray(_as_bits(B))
    if A.ndim != 2 or B.ndim != 2:
        raise ValueError("A and B must be 2-D")
    M, lda = A.shape
    N, ldb = B.shape
    if K is None:
        K = lda
        if ldb != K:
            raise ValueError("pass K explicitly when the row pitches differ")
    if K > lda or K > ldb:
        raise ValueError("K exceeds a row pitch")
    if rows is not None:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nout = rows.shape[0]
    else:
        nout = M
    C = np.zeros((nout, N), dtype=np.float64)
    Mag = np.zeros((nout, N), dtype=np.float64) if want_mag else None
    if nout == 0 or N == 0:
        return C, Mag
    lib = _load()
    rc = lib.oracle_gemm_bf16(
        M, N, K,
        A.ctypes.data if A.size else None, max(lda, 1),
        B.ctypes.data if B.size else None, max(ldb, 1),
        C.ctypes.data, Mag.ctypes.data if want_mag else None, N,
        rows.ctypes.data if rows is not None else None, nout,
        nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_gemm_bf16 rejected its arguments (rc={rc})")
    return C, Mag


def gemm_batched(A: np.ndarray, B: np.ndarray, K: int | None = None,
                 nthreads: int | None = None):
    """Independent GEMMs over a leading batch axis: A (batch, M, lda), B (batch, N, ldb)."""
    Cs, Ms = [], []
    for b in range(A.shape[0]):
        C, Mg = gemm(A[b], B[b], K=K, nthreads=nthreads)
        Cs.append(C)
        Ms.append(Mg)
    return np.stack(Cs), np.stack(Ms)


def round_bf16(x) -> np.ndarray:
    """Round binary64 values to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, dtype=np.uint16)
    if x.size:
        _load().oracle_round_bf16_array(x.ctypes.data, out.ctypes.data, x.size)
    return out


def decode_bf16(h) -> np.ndarray:
    """bf16 bit patterns -> binary64 values (exact), using the oracle's own decode."""
    h = np.ascontiguousarray(np.asarray(h, dtype=np.uint16))
    out = np.empty(h.shape, dtype=np.float64)
    if h.size:
        _load().oracle_decode_bf16_array(h.ctypes.data, out.ctypes.data, h.size)
    return out
