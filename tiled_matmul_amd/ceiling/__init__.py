"""Binding of libtmm_ceiling.so (include/ceiling.h): the measurement kernels bench.py runs
beside the decode GEMV (a cold streaming read and an empty kernel).  Argument marshalling
only; loading fails loudly when the library is not built."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtmm_ceiling.so")
SOURCE = os.path.join(_HERE, "ceiling.hip")
HEADER = os.path.join(os.path.dirname(os.path.dirname(_HERE)), "include", "ceiling.h")
_lib = None


def library():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        lib = ctypes.CDLL(LIB_PATH)
        i64, vp, i = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.ceiling_stream_read.argtypes = [vp, i64, vp, i, i, vp]
        lib.ceiling_stream_read.restype = i
        lib.ceiling_launch_floor.argtypes = [i, i, vp]
        lib.ceiling_launch_floor.restype = i
        _lib = lib
    return _lib


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def stream_read(src, nbytes: int, sink, grid: int, block: int) -> None:
    rc = library().ceiling_stream_read(src.data_ptr(), nbytes, sink.data_ptr(), grid, block, _stream())
    if rc != 0:
        raise RuntimeError(f"ceiling_stream_read: status {rc}")


def launch_floor(grid: int, block: int) -> None:
    rc = library().ceiling_launch_floor(grid, block, _stream())
    if rc != 0:
        raise RuntimeError(f"ceiling_launch_floor: status {rc}")
