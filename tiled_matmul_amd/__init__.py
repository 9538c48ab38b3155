"""tiled_matmul_amd: a tiled bf16 GEMM, C = A * B^T with fp32 accumulation, for AMD Instinct
MI355X (gfx950), behind the C ABI of ``libgemm_bf16.so`` (``include/gemm_bf16.h``).

This module is the thin Python binding: the functions carry the C names and only marshal
arguments (ints, or tensors via ``data_ptr()``; streams via ``cuda_stream``).  Every step of
the computation runs in the library's HIP kernels; there is no Python or CPU fallback, and
loading fails loudly when the library has not been built (``__graft_entry__.build()`` or
``python -m tiled_matmul_amd.build``).

``matmul`` is a convenience wrapper over torch tensors that allocates the output.
"""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
# GEMM_BF16_LIB selects another build of the same library (e.g. one compiled with other
# tile-shape macros by tiled_matmul_amd.build.build_library(out=..., defines=...)).
LIB_PATH = os.environ.get("GEMM_BF16_LIB") or os.path.join(_HERE, "libgemm_bf16.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "gemm_bf16.h")
HEADERS = [HEADER, os.path.join(os.path.dirname(_HERE), "include", "gemm_mx.h"),
           os.path.join(os.path.dirname(_HERE), "include", "attention.h")]

GEMM_OK = 0
GEMM_ERR_ARG = 1
GEMM_ERR_NULL = 2
GEMM_ERR_DTYPE = 3
GEMM_ERR_ARCH = 4
GEMM_ERR_LAUNCH = 5
GEMM_ERR_UNSUPPORTED = 6
GEMM_ERR_SCRATCH = 7
GEMM_SCRATCH_BYTES = 64 << 20

GEMM_STREAMK_AUTO = 0
GEMM_STREAMK_DP = 1
GEMM_STREAMK_ALL = 2

GEMM_OUT_FP32 = 0
GEMM_OUT_BF16 = 1

GEMM_LAYOUT_K_MAJOR = 0
GEMM_LAYOUT_MN_MAJOR = 1

# Block-scaled 8-bit GEMM (include/gemm_mx.h)
GEMM_MX_E4M3 = 0
GEMM_MX_E5M2 = 1
GEMM_MX_VARIANT_AUTO = 0
GEMM_MX_VARIANT_SIMPLE = 1
GEMM_MX_VARIANT_RING = 2

# Attention forward (include/attention.h)
ATTN_VARIANT_AUTO = 0
ATTN_VARIANT_SIMPLE = 1
ATTN_VARIANT_MFMA = 2
ATTN_VARIANT_PIPE = 3

GEMM_VARIANT_AUTO = 0
GEMM_VARIANT_SIMPLE = 1
GEMM_VARIANT_MFMA = 2
GEMM_VARIANT_PIPELINED = 3
GEMM_VARIANT_PERSISTENT = 4
GEMM_VARIANT_SPECIALIZED = 5
GEMM_VARIANT_GEMV = 6
GEMM_VARIANT_PINGPONG = 7
GEMM_VARIANT_RING8 = 8
GEMM_VARIANT_RING4 = 9
GEMM_VARIANT_DTV = 10
GEMM_VARIANT_ROLES = 11

VARIANTS = {
    "auto": GEMM_VARIANT_AUTO, "simple": GEMM_VARIANT_SIMPLE, "mfma": GEMM_VARIANT_MFMA,
    "pipelined": GEMM_VARIANT_PIPELINED, "persistent": GEMM_VARIANT_PERSISTENT,
    "specialized": GEMM_VARIANT_SPECIALIZED, "gemv": GEMM_VARIANT_GEMV,
    "pingpong": GEMM_VARIANT_PINGPONG, "ring8": GEMM_VARIANT_RING8, "ring4": GEMM_VARIANT_RING4,
    "dtv": GEMM_VARIANT_DTV, "roles": GEMM_VARIANT_ROLES,
}


class GemmError(RuntimeError):
    """A nonzero status from the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {gemm_bf16_status_string(status)} (status {status})")


_lib = None
_i64, _vp, _int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run __graft_entry__.build() "
            "(or python -m tiled_matmul_amd.build) first")
    lib = ctypes.CDLL(LIB_PATH)
    batched = [_i64, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _int]
    lib.gemm_bf16.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _int, _vp]
    lib.gemm_bf16_strided_batched.argtypes = batched + [_vp]
    lib.gemm_bf16_variant.argtypes = [_int] + batched + [_vp]
    lib.gemm_bf16_validate.argtypes = batched
    lib.gemm_bf16_plan.argtypes = [_int] + batched + [_int, ctypes.POINTER(_int),
                                                      ctypes.POINTER(_i64), ctypes.POINTER(_int)]
    lib.gemm_bf16_layout.argtypes = [_int, _int, _int] + batched + [_vp]
    lib.gemm_bf16_layout_validate.argtypes = [_int, _int] + batched
    lib.gemm_bf16_layout_plan.argtypes = [_int, _int, _int] + batched + [
        _int, ctypes.POINTER(_int), ctypes.POINTER(_i64), ctypes.POINTER(_int)]
    lib.gemm_bf16_splitk.argtypes = [_int, _int, _int] + batched + [_vp, _i64, _vp]
    lib.gemm_bf16_splitk_noalloc.argtypes = [_int, _int, _int] + batched + [_vp]
    lib.gemm_bf16_streamk.argtypes = [_int] + batched + [_vp, _i64, _vp]
    lib.gemm_bf16_streamk_plan.argtypes = [_int] + batched + [
        _int, ctypes.POINTER(_i64), ctypes.POINTER(_int), ctypes.POINTER(_int), ctypes.POINTER(_int),
        ctypes.POINTER(_i64)]
    lib.gemm_bf16_splitk_plan.argtypes = [_int, _int, _int] + batched + [
        _vp, _i64, _int, ctypes.POINTER(_int), ctypes.POINTER(_int), ctypes.POINTER(_i64)]
    mx = [_int, _int, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _int]
    lib.gemm_mx.argtypes = mx + [_vp]
    lib.gemm_mx_variant.argtypes = [_int] + mx + [_vp]
    lib.gemm_mx_validate.argtypes = mx
    lib.gemm_mx_plan.argtypes = [_int] + mx + [_int, ctypes.POINTER(_int), ctypes.POINTER(_i64),
                                                ctypes.POINTER(_int)]
    at = [_i64, _i64, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp]
    lib.attention_fwd.argtypes = at + [_vp, ctypes.c_float, _int, _int, _vp]
    lib.attention_fwd_variant.argtypes = [_int] + at + [_vp, ctypes.c_float, _int, _int, _vp]
    lib.attention_fwd_validate.argtypes = at + [ctypes.c_float, _int, _int]
    lib.attention_fwd_plan.argtypes = [_int] + at + [ctypes.c_float, _int, _int, _int,
                                                     ctypes.POINTER(_int), ctypes.POINTER(_i64),
                                                     ctypes.POINTER(_int)]
    for f in ("gemm_mx", "gemm_mx_variant", "gemm_mx_validate", "gemm_mx_plan", "attention_fwd",
              "attention_fwd_variant", "attention_fwd_validate", "attention_fwd_plan"):
        getattr(lib, f).restype = _int
    for f in ("gemm_bf16", "gemm_bf16_strided_batched", "gemm_bf16_variant",
              "gemm_bf16_validate", "gemm_bf16_plan", "gemm_bf16_version", "gemm_bf16_layout",
              "gemm_bf16_layout_validate", "gemm_bf16_layout_plan", "gemm_bf16_splitk",
              "gemm_bf16_splitk_noalloc", "gemm_bf16_streamk", "gemm_bf16_streamk_plan",
              "gemm_bf16_splitk_plan"):
        getattr(lib, f).restype = _int
    lib.gemm_bf16_kernel_name.argtypes = [_int]
    lib.gemm_bf16_kernel_name.restype = ctypes.c_char_p
    lib.gemm_bf16_status_string.argtypes = [_int]
    lib.gemm_bf16_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def library():
    """The loaded ctypes library (raises if it is not built)."""
    return _load()


def declared_functions() -> list[str]:
    """Names of the functions include/gemm_bf16.h and include/gemm_mx.h declare."""
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*((?:gemm|attention)_\w*)\s*\(",
                                text, re.M))
    return sorted(names)


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        try:
            import torch
            if torch.cuda.is_available():
                return torch.cuda.current_stream().cuda_stream
        except ImportError:  # pragma: no cover
            pass
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(status: int, where: str):
    if status != GEMM_OK:
        raise GemmError(status, where)


def gemm_bf16(M, N, K, A, lda, B, ldb, C, ldc, out_dtype, stream=None):
    _check(_load().gemm_bf16(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, out_dtype,
                             _stream(stream)), "gemm_bf16")


def gemm_bf16_strided_batched(batch, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc,
                              strideC, out_dtype, stream=None):
    _check(_load().gemm_bf16_strided_batched(batch, M, N, K, _ptr(A), lda, strideA, _ptr(B),
                                             ldb, strideB, _ptr(C), ldc, strideC, out_dtype,
                                             _stream(stream)), "gemm_bf16_strided_batched")


def gemm_bf16_variant(variant, batch, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc,
                      strideC, out_dtype, stream=None):
    _check(_load().gemm_bf16_variant(variant, batch, M, N, K, _ptr(A), lda, strideA, _ptr(B),
                                     ldb, strideB, _ptr(C), ldc, strideC, out_dtype,
                                     _stream(stream)), "gemm_bf16_variant")


def gemm_bf16_validate(batch, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC,
                       out_dtype) -> int:
    return _load().gemm_bf16_validate(batch, M, N, K, _ptr(A), lda, strideA, _ptr(B), ldb,
                                      strideB, _ptr(C), ldc, strideC, out_dtype)


def gemm_bf16_plan(variant, batch, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC,
                   out_dtype, num_cus=0):
    """(status, kernel_name, workgroups, threads_per_workgroup)."""
    k, g, b = _int(0), _i64(0), _int(0)
    rc = _load().gemm_bf16_plan(variant, batch, M, N, K, _ptr(A), lda, strideA, _ptr(B), ldb,
                                strideB, _ptr(C), ldc, strideC, out_dtype, num_cus,
                                ctypes.byref(k), ctypes.byref(g), ctypes.byref(b))
    return rc, gemm_bf16_kernel_name(k.value), g.value, b.value


def gemm_bf16_layout(a_layout, b_layout, variant, batch, M, N, K, A, lda, strideA, B, ldb, strideB,
                     C, ldc, strideC, out_dtype, stream=None):
    _check(_load().gemm_bf16_layout(a_layout, b_layout, variant, batch, M, N, K, _ptr(A), lda,
                                    strideA, _ptr(B), ldb, strideB, _ptr(C), ldc, strideC,
                                    out_dtype, _stream(stream)), "gemm_bf16_layout")


def gemm_bf16_layout_validate(a_layout, b_layout, batch, M, N, K, A, lda, strideA, B, ldb,
                              strideB, C, ldc, strideC, out_dtype) -> int:
    return _load().gemm_bf16_layout_validate(a_layout, b_layout, batch, M, N, K, _ptr(A), lda,
                                             strideA, _ptr(B), ldb, strideB, _ptr(C), ldc,
                                             strideC, out_dtype)


def gemm_bf16_layout_plan(a_layout, b_layout, variant, batch, M, N, K, A, lda, strideA, B, ldb,
                          strideB, C, ldc, strideC, out_dtype, num_cus=0):
    """(status, kernel_name, workgroups, threads_per_workgroup)."""
    k, g, b = _int(0), _i64(0), _int(0)
    rc = _load().gemm_bf16_layout_plan(a_layout, b_layout, variant, batch, M, N, K, _ptr(A), lda,
                                       strideA, _ptr(B), ldb, strideB, _ptr(C), ldc, strideC,
                                       out_dtype, num_cus, ctypes.byref(k), ctypes.byref(g),
                                       ctypes.byref(b))
    return rc, gemm_bf16_kernel_name(k.value), g.value, b.value


def gemm_bf16_splitk(a_layout, b_layout, splits, batch, M, N, K, A, lda, strideA, B, ldb,
                     strideB, C, ldc, strideC, out_dtype, workspace, workspace_bytes,
                     stream=None):
    _check(_load().gemm_bf16_splitk(a_layout, b_layout, splits, batch, M, N, K, _ptr(A), lda,
                                    strideA, _ptr(B), ldb, strideB, _ptr(C), ldc, strideC,
                                    out_dtype, _ptr(workspace), workspace_bytes,
                                    _stream(stream)), "gemm_bf16_splitk")


def gemm_bf16_splitk_noalloc(a_layout, b_layout, splits, batch, M, N, K, A, lda, strideA, B, ldb,
                             strideB, C, ldc, strideC, out_dtype, stream=None):
    _check(_load().gemm_bf16_splitk_noalloc(a_layout, b_layout, splits, batch, M, N, K, _ptr(A), lda,
                                            strideA, _ptr(B), ldb, strideB, _ptr(C), ldc, strideC,
                                            out_dtype, _stream(stream)), "gemm_bf16_splitk_noalloc")


def gemm_bf16_streamk(mode, batch, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC,
                      out_dtype, workspace, workspace_bytes, stream=None):
    _check(_load().gemm_bf16_streamk(mode, batch, M, N, K, _ptr(A), lda, strideA, _ptr(B), ldb, strideB,
                                     _ptr(C), ldc, strideC, out_dtype, _ptr(workspace), workspace_bytes,
                                     _stream(stream)), "gemm_bf16_streamk")


def gemm_bf16_streamk_plan(mode, batch, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC,
                           out_dtype, num_cus=0):
    """(status, workspace bytes, whole tiles, cut tiles, stream-K slots, workgroups)."""
    ws, dp, sk, sl, gx = _i64(0), _int(0), _int(0), _int(0), _i64(0)
    rc = _load().gemm_bf16_streamk_plan(mode, batch, M, N, K, _ptr(A), lda, strideA, _ptr(B), ldb, strideB,
                                        _ptr(C), ldc, strideC, out_dtype, num_cus, ctypes.byref(ws),
                                        ctypes.byref(dp), ctypes.byref(sk), ctypes.byref(sl), ctypes.byref(gx))
    return rc, ws.value, dp.value, sk.value, sl.value, gx.value


def gemm_bf16_splitk_plan(a_layout, b_layout, splits, batch, M, N, K, A, lda, strideA, B, ldb,
                          strideB, C, ldc, strideC, out_dtype, workspace, workspace_bytes,
                          num_cus=0):
    """(status, splits, kernel_name, workgroups of the first launch)."""
    s, k, g = _int(0), _int(0), _i64(0)
    rc = _load().gemm_bf16_splitk_plan(a_layout, b_layout, splits, batch, M, N, K, _ptr(A), lda,
                                       strideA, _ptr(B), ldb, strideB, _ptr(C), ldc, strideC,
                                       out_dtype, _ptr(workspace), workspace_bytes, num_cus,
                                       ctypes.byref(s), ctypes.byref(k), ctypes.byref(g))
    return rc, s.value, gemm_bf16_kernel_name(k.value), g.value


def gemm_mx(a_format, b_format, M, N, K, A, lda, A_scale, lda_scale, B, ldb, B_scale, ldb_scale, C,
            ldc, out_dtype, stream=None):
    _check(_load().gemm_mx(a_format, b_format, M, N, K, _ptr(A), lda, _ptr(A_scale), lda_scale,
                           _ptr(B), ldb, _ptr(B_scale), ldb_scale, _ptr(C), ldc, out_dtype,
                           _stream(stream)), "gemm_mx")


def gemm_mx_variant(variant, a_format, b_format, M, N, K, A, lda, A_scale, lda_scale, B, ldb,
                    B_scale, ldb_scale, C, ldc, out_dtype, stream=None):
    _check(_load().gemm_mx_variant(variant, a_format, b_format, M, N, K, _ptr(A), lda,
                                   _ptr(A_scale), lda_scale, _ptr(B), ldb, _ptr(B_scale),
                                   ldb_scale, _ptr(C), ldc, out_dtype, _stream(stream)),
           "gemm_mx_variant")


def gemm_mx_validate(a_format, b_format, M, N, K, A, lda, A_scale, lda_scale, B, ldb, B_scale,
                     ldb_scale, C, ldc, out_dtype) -> int:
    return _load().gemm_mx_validate(a_format, b_format, M, N, K, _ptr(A), lda, _ptr(A_scale),
                                    lda_scale, _ptr(B), ldb, _ptr(B_scale), ldb_scale, _ptr(C),
                                    ldc, out_dtype)


def gemm_mx_plan(variant, a_format, b_format, M, N, K, A, lda, A_scale, lda_scale, B, ldb,
                 B_scale, ldb_scale, C, ldc, out_dtype, num_cus=0):
    """(status, kernel_name, workgroups, threads_per_workgroup)."""
    k, g, b = _int(0), _i64(0), _int(0)
    rc = _load().gemm_mx_plan(variant, a_format, b_format, M, N, K, _ptr(A), lda, _ptr(A_scale),
                              lda_scale, _ptr(B), ldb, _ptr(B_scale), ldb_scale, _ptr(C), ldc,
                              out_dtype, num_cus, ctypes.byref(k), ctypes.byref(g),
                              ctypes.byref(b))
    return rc, gemm_bf16_kernel_name(k.value), g.value, b.value


def attention_fwd(B, Hq, Hkv, Lq, Lk, d, Q, K, V, O, LSE, scale, causal, out_dtype, stream=None):
    _check(_load().attention_fwd(B, Hq, Hkv, Lq, Lk, d, _ptr(Q), _ptr(K), _ptr(V), _ptr(O),
                                 _ptr(LSE), scale, int(causal), out_dtype, _stream(stream)),
           "attention_fwd")


def attention_fwd_variant(variant, B, Hq, Hkv, Lq, Lk, d, Q, K, V, O, LSE, scale, causal,
                          out_dtype, stream=None):
    _check(_load().attention_fwd_variant(variant, B, Hq, Hkv, Lq, Lk, d, _ptr(Q), _ptr(K),
                                         _ptr(V), _ptr(O), _ptr(LSE), scale, int(causal),
                                         out_dtype, _stream(stream)), "attention_fwd_variant")


def attention_fwd_validate(B, Hq, Hkv, Lq, Lk, d, Q, K, V, O, scale, causal, out_dtype) -> int:
    return _load().attention_fwd_validate(B, Hq, Hkv, Lq, Lk, d, _ptr(Q), _ptr(K), _ptr(V),
                                          _ptr(O), scale, int(causal), out_dtype)


def attention_fwd_plan(variant, B, Hq, Hkv, Lq, Lk, d, Q, K, V, O, scale, causal, out_dtype,
                       num_cus=0):
    """(status, kernel_name, workgroups, threads_per_workgroup)."""
    k, g, b = _int(0), _i64(0), _int(0)
    rc = _load().attention_fwd_plan(variant, B, Hq, Hkv, Lq, Lk, d, _ptr(Q), _ptr(K), _ptr(V),
                                    _ptr(O), scale, int(causal), out_dtype, num_cus,
                                    ctypes.byref(k), ctypes.byref(g), ctypes.byref(b))
    return rc, gemm_bf16_kernel_name(k.value), g.value, b.value


def gemm_bf16_kernel_name(kernel_id: int) -> str:
    return _load().gemm_bf16_kernel_name(kernel_id).decode()


def gemm_bf16_status_string(status: int) -> str:
    return _load().gemm_bf16_status_string(status).decode()


def gemm_bf16_version() -> int:
    return _load().gemm_bf16_version()


def matmul(A, B, out_dtype=None, variant: int = GEMM_VARIANT_AUTO, out=None, stream=None):
    """C = A @ B.T for bf16 device tensors A (M x K) and B (N x K) with unit column stride
    (a leading batch dimension is allowed on both).  Returns a new float32 (default) or
    bfloat16 tensor, or writes ``out``."""
    import torch
    if out_dtype is None:
        out_dtype = torch.float32
    od = {torch.float32: GEMM_OUT_FP32, torch.bfloat16: GEMM_OUT_BF16}[out_dtype]
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise TypeError("A and B must be bfloat16")
    if A.stride(-1) != 1 or B.stride(-1) != 1:
        raise ValueError("A and B must be K-contiguous (unit stride in the last dimension)")
    batched = A.dim() == 3
    if batched:
        batch, M, K = A.shape
        _, N, K2 = B.shape
    else:
        (M, K), (N, K2) = A.shape, B.shape
        batch = 1
    if K2 != K:
        raise ValueError("inner dimensions differ")
    if out is None:
        out = torch.empty((batch, M, N) if batched else (M, N), dtype=out_dtype, device=A.device)
    gemm_bf16_variant(variant, batch, M, N, K, A, A.stride(-2), A.stride(0) if batched else 0,
                      B, B.stride(-2), B.stride(0) if batched else 0,
                      out, out.stride(-2), out.stride(0) if batched else 0, od, stream)
    return out
