"""The C-ABI library on the host: it loads, exports every function include/gemm_bf16.h
declares, validates arguments with the documented codes, and plans the documented kernels.
No GPU (validation and planning are host-only functions)."""
import ctypes

import pytest

import tiled_matmul_amd as tm

P = 1 << 12   # a fake, 16-byte aligned "device" address: validation never dereferences it


def test_library_exports_every_declared_symbol():
    lib = tm.library()
    names = tm.declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), f"missing export {n}"
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_version_and_strings():
    assert tm.gemm_bf16_version() == 10
    for s in range(8):
        assert tm.gemm_bf16_status_string(s).startswith("GEMM_")
    assert tm.gemm_bf16_status_string(99) == "unknown status"
    assert tm.gemm_bf16_kernel_name(4) == "pipe_256"


def v(batch=1, M=64, N=64, K=64, A=P, lda=None, sA=0, B=P, ldb=None, sB=0, C=P, ldc=None, sC=0,
      out=0):
    lda = K if lda is None else lda
    ldb = K if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return tm.gemm_bf16_validate(batch, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, out)


def test_validate_ok_cases():
    assert v() == tm.GEMM_OK
    assert v(K=0, lda=1, ldb=1) == tm.GEMM_OK
    assert v(M=0, C=None, A=None) == tm.GEMM_OK          # nothing to do: pointers unused
    assert v(batch=0, C=None) == tm.GEMM_OK
    assert v(K=0, lda=1, ldb=1, A=None, B=None) == tm.GEMM_OK   # empty sum needs only C
    assert v(batch=3, sA=0, sB=64 * 64, sC=64 * 64) == tm.GEMM_OK
    assert v(out=1, C=P + 2) == tm.GEMM_OK               # bf16 out needs 2-byte alignment


@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), tm.GEMM_ERR_ARG), (dict(N=-1), tm.GEMM_ERR_ARG), (dict(K=-1), tm.GEMM_ERR_ARG),
    (dict(lda=63), tm.GEMM_ERR_ARG), (dict(ldb=63), tm.GEMM_ERR_ARG),
    (dict(ldc=63), tm.GEMM_ERR_ARG), (dict(K=0, lda=0), tm.GEMM_ERR_ARG),
    (dict(batch=-1), tm.GEMM_ERR_ARG), (dict(batch=65536), tm.GEMM_ERR_ARG),
    (dict(batch=2, sC=64 * 64 - 1), tm.GEMM_ERR_ARG), (dict(sA=-8), tm.GEMM_ERR_ARG),
    (dict(A=None), tm.GEMM_ERR_NULL), (dict(B=None), tm.GEMM_ERR_NULL),
    (dict(C=None), tm.GEMM_ERR_NULL), (dict(out=2), tm.GEMM_ERR_DTYPE),
    (dict(out=-1), tm.GEMM_ERR_DTYPE), (dict(A=P + 1), tm.GEMM_ERR_ARG),
    (dict(C=P + 2), tm.GEMM_ERR_ARG), (dict(M=1 << 41), tm.GEMM_ERR_ARG),
])
def test_validate_error_codes(kw, code):
    assert v(**kw) == code


def plan(variant=0, batch=1, M=4096, N=4096, K=4096, A=P, lda=None, sA=0, B=P, ldb=None, sB=0,
         C=P, ldc=None, sC=0, out=0, cus=256):
    lda = K if lda is None else lda
    ldb = K if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return tm.gemm_bf16_plan(variant, batch, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, out, cus)


def test_plan_workloads():
    assert plan()[:2] == (0, "ring4_256")
    assert plan()[3] == 256
    assert plan(M=1)[:2] == (0, "gemv_lds")
    assert plan(M=4)[:2] == (0, "gemv_lds")
    assert plan(M=5)[:2] == (0, "gemv")
    assert plan(M=8)[:2] == (0, "gemv")
    assert plan(M=9)[:2] == (0, "gemv")
    assert plan(M=16)[:2] == (0, "gemv")
    assert plan(M=17)[1] != "gemv"
    assert plan(M=8192, N=14336, K=4096, out=1)[:2] == (0, "ring4_256")
    assert plan(variant=5)[:2] == (0, "spec_256")
    assert plan(variant=5)[3] == 512
    # K = 4100 with lda = 4100: rows 8-byte aligned, ragged K tail -> still the fast kernel
    assert plan(M=3000, N=5000, K=4100)[1] == "ring4_256"
    # odd pitch: rows only 2-byte aligned -> general MFMA kernel
    assert plan(M=3000, N=5000, K=4101)[1] == "mfma_128"
    assert plan(batch=64, M=256, N=256, K=1024, sA=256 * 1024, sB=256 * 1024,
                sC=256 * 256)[1] == "persist_128"
    assert plan(K=0, lda=1, ldb=1)[:2] == (0, "zero_fill")
    assert plan(M=0)[1] == "none"


def test_plan_persistent_grid_is_cu_count():
    rc, name, grid, block = plan(variant=4, M=8192, N=14336, K=4096)
    assert (rc, name, grid, block) == (0, "persist_256", 256, 256)
    rc, name, grid, _ = plan(variant=3, M=8192, N=14336, K=4096)
    assert (rc, name, grid) == (0, "pipe_256", 32 * 56)


def test_plan_variant_preconditions():
    assert plan(variant=6, M=17)[0] == tm.GEMM_ERR_UNSUPPORTED
    # pipelined / persistent / specialized: 4-byte aligned rows, any K
    assert plan(variant=3, K=4100)[:2] == (0, "pipe_256")
    assert plan(variant=3, K=4099, lda=4100, ldb=4100)[:2] == (0, "pipe_256")
    assert plan(variant=3, K=4099)[0] == tm.GEMM_ERR_UNSUPPORTED
    assert plan(variant=4, A=P + 4)[:2] == (0, "persist_256")
    assert plan(variant=4, A=P + 2)[0] == tm.GEMM_ERR_UNSUPPORTED
    assert plan(variant=5, K=4100)[:2] == (0, "spec_256")
    assert plan(variant=5, K=7, lda=8, ldb=10)[:2] == (0, "spec_256")
    assert plan(variant=5, batch=2, sA=4096 * 4096 + 1, sB=4096 * 4096,
                sC=4096 * 4096)[0] == tm.GEMM_ERR_UNSUPPORTED
    # ping-pong: 16-byte aligned rows and K % 8 == 0
    assert plan(variant=7)[:2] == (0, "pingpong_256")
    assert plan(variant=7, K=4100)[0] == tm.GEMM_ERR_UNSUPPORTED
    assert plan(variant=7, A=P + 8)[0] == tm.GEMM_ERR_UNSUPPORTED
    # five-slot ring, 8 and 4 waves: the pipelined kernels' preconditions
    assert plan(variant=8)[:2] == (0, "ring8_256")
    assert plan(variant=8)[3] == 512
    assert plan(variant=9)[:2] == (0, "ring4_256")
    assert plan(variant=9)[3] == 256
    assert plan(variant=9, K=4099, lda=4100, ldb=4100)[:2] == (0, "ring4_256")
    assert plan(variant=9, A=P + 2)[0] == tm.GEMM_ERR_UNSUPPORTED
    assert plan(variant=10)[:2] == (0, "dtv_256")
    assert plan(variant=10)[3] == 256
    assert plan(variant=10, K=4100)[0] == tm.GEMM_ERR_UNSUPPORTED      # 16-byte chunks need K % 8 == 0
    assert plan(variant=10, A=P + 8)[0] == tm.GEMM_ERR_UNSUPPORTED     # and 16-byte aligned rows
    # fixed producer / consumer waves: 256 x 128 tiles, 8 waves, K % 8 == 0, 4-byte aligned rows
    assert plan(variant=11) == (0, "roles_256x128", 256, 512)
    assert plan(variant=11, M=4096, N=2048)[:3] == (0, "roles_256x128", 256)
    assert plan(variant=11, M=512, N=512)[:3] == (0, "roles_256x128", 8)
    assert plan(variant=11, K=4100)[0] == tm.GEMM_ERR_UNSUPPORTED
    assert plan(variant=11, A=P + 2)[0] == tm.GEMM_ERR_UNSUPPORTED
    assert plan(variant=11, A=P + 4)[:2] == (0, "roles_256x128")
    assert plan(variant=12)[0] == tm.GEMM_ERR_ARG
    assert plan(variant=1)[1] == "simple_64"
    assert plan(variant=2)[1] == "mfma_128"


def test_calls_fail_cleanly_without_gfx950():
    """On a host without a gfx950 the launch path reports GEMM_ERR_ARCH, after validation."""
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present")
    except ImportError:
        pass
    lib = tm.library()
    assert lib.gemm_bf16(64, 64, 64, P, 64, P, 64, P, 64, 0, None) == tm.GEMM_ERR_ARCH
    assert lib.gemm_bf16(64, 64, 64, P, 63, P, 64, P, 64, 0, None) == tm.GEMM_ERR_ARG


def lplan(la, lb, variant=0, M=4096, N=4096, K=4096, A=P, lda=None, B=P, ldb=None, out=0, batch=1,
          sA=0, sB=0, sC=0):
    lda = (K if la == 0 else M) if lda is None else lda
    ldb = (K if lb == 0 else N) if ldb is None else ldb
    return tm.gemm_bf16_layout_plan(la, lb, variant, batch, M, N, K, A, lda, sA, B, ldb, sB, P, N,
                                    sC, out, 256)


def test_layout_validation():
    MN, KM = tm.GEMM_LAYOUT_MN_MAJOR, tm.GEMM_LAYOUT_K_MAJOR
    v = tm.gemm_bf16_layout_validate
    # MN-major A: pitch counts M (here K > M, so lda = M is fine and lda = K is not needed)
    assert v(MN, KM, 1, 100, 50, 300, P, 100, 0, P, 300, 0, P, 50, 0, 0) == tm.GEMM_OK
    assert v(MN, KM, 1, 100, 50, 300, P, 99, 0, P, 300, 0, P, 50, 0, 0) == tm.GEMM_ERR_ARG
    # K-major A needs lda >= K
    assert v(KM, KM, 1, 100, 50, 300, P, 100, 0, P, 300, 0, P, 50, 0, 0) == tm.GEMM_ERR_ARG
    # MN-major B: pitch counts N
    assert v(KM, MN, 1, 100, 50, 300, P, 300, 0, P, 50, 0, P, 50, 0, 0) == tm.GEMM_OK
    assert v(KM, MN, 1, 100, 50, 300, P, 300, 0, P, 49, 0, P, 50, 0, 0) == tm.GEMM_ERR_ARG
    assert v(2, KM, 1, 100, 50, 300, P, 300, 0, P, 300, 0, P, 50, 0, 0) == tm.GEMM_ERR_ARG
    assert v(KM, -1, 1, 100, 50, 300, P, 300, 0, P, 300, 0, P, 50, 0, 0) == tm.GEMM_ERR_ARG
    # both K-major: the same answers as gemm_bf16_validate
    assert v(KM, KM, 1, 64, 64, 64, P, 64, 0, P, 64, 0, P, 64, 0, 0) == tm.GEMM_OK


def test_layout_plan():
    MN, KM = tm.GEMM_LAYOUT_MN_MAJOR, tm.GEMM_LAYOUT_K_MAJOR
    assert lplan(KM, KM)[:2] == (0, "ring4_256")
    assert lplan(KM, MN)[:2] == (0, "ring4_256")
    assert lplan(MN, KM)[:2] == (0, "ring4_256")
    assert lplan(MN, MN)[:2] == (0, "ring4_256")
    assert lplan(KM, MN)[3] == 256
    # small shapes still take the ring kernel (tile count is not a precondition)
    assert lplan(KM, MN, M=64, N=64, K=64)[:2] == (0, "ring4_256")
    # MN-major extent not a multiple of 8, odd pitch, 2-byte aligned pointer: general kernel
    assert lplan(MN, KM, M=4095)[:2] == (0, "simple_64")
    assert lplan(KM, MN, N=4093)[:2] == (0, "simple_64")
    assert lplan(KM, MN, ldb=4097)[:2] == (0, "simple_64")
    assert lplan(KM, MN, B=P + 2)[:2] == (0, "simple_64")
    # forced variants
    assert lplan(KM, MN, variant=1)[:2] == (0, "simple_64")
    assert lplan(KM, MN, variant=9)[:2] == (0, "ring4_256")
    assert lplan(KM, MN, variant=9, N=4093)[0] == tm.GEMM_ERR_UNSUPPORTED
    for variant in (2, 3, 4, 5, 6, 7, 8, 10, 11):
        assert lplan(KM, MN, variant=variant)[0] == tm.GEMM_ERR_UNSUPPORTED, variant
    assert lplan(KM, MN, variant=12)[0] == tm.GEMM_ERR_ARG
    # K = 0: zero fill in any layout
    assert lplan(MN, MN, K=0, lda=4096, ldb=4096)[:2] == (0, "zero_fill")
    # both K-major: the K-major planner (the GEMV path included)
    assert lplan(KM, KM, M=1)[:2] == (0, "gemv_lds")


def splan(splits, M=1024, N=1024, K=16384, la=0, lb=0, ws=P, ws_bytes=(1 << 62), out=0,
          batch=1, lda=None, ldb=None, A=P, B=P):
    lda = (K if la == 0 else M) if lda is None else lda
    ldb = (K if lb == 0 else N) if ldb is None else ldb
    sA, sB, sC = (M * K, N * K, M * N) if batch > 1 else (0, 0, 0)
    return tm.gemm_bf16_splitk_plan(la, lb, splits, batch, M, N, K, A, lda, sA, B, ldb, sB, P, N,
                                    sC, out, ws, ws_bytes, 256)


def test_splitk_plan():
    MN, KM = tm.GEMM_LAYOUT_MN_MAJOR, tm.GEMM_LAYOUT_K_MAJOR
    # unsplit, the planner would run 64 tiles of 128 x 128 (a quarter of the CUs busy); split,
    # 16 tiles of 256 x 256 times 16 K ranges (of 16 blocks of 64) fill the 256 CUs
    assert splan(0) == (0, 16, "ring4_256", 256)
    # the workspace bounds the choice: room for 5 ranges
    assert splan(0, ws_bytes=5 * 1024 * 1024 * 4 + 100)[:2] == (0, 5)
    # no workspace: one range, the ordinary AUTO plan
    assert splan(0, ws=None, ws_bytes=0)[:3] == (0, 1, "persist_128")
    # at least 8 K blocks per range: K = 1024 (16 blocks) -> 2 ranges
    assert splan(0, K=1024)[:2] == (0, 2)
    assert splan(0, K=960)[:3] == (0, 1, "persist_128")
    # the threshold: split only while the unsplit kernel's tiles cover at most half the CUs
    # (128 tiles of 128 x 128 -> S = min(256 / 32 tiles of 256 x 256, 64 blocks / 8) = 8;
    # 144 tiles -> unsplit)
    assert splan(0, M=1024, N=2048, K=4096) == (0, 8, "ring4_256", 256)
    assert splan(0, M=1152, N=2048, K=4096)[:3] == (0, 1, "persist_128")
    # enough tiles already (4096^2: 256 tiles; 64 items of 256 x 256: 256 tiles of 128 x 128):
    # one range
    assert splan(0, M=4096, N=4096, K=4096) == (0, 1, "ring4_256", 256)
    assert splan(0, M=256, N=256, K=1024, batch=64)[:3] == (0, 1, "persist_128")
    # explicit counts, capped at the number of K blocks
    assert splan(3, M=4096, N=4096, K=4096) == (0, 3, "ring4_256", 256)
    assert splan(7, K=128) == (0, 2, "ring4_256", 32)
    assert splan(1)[:2] == (0, 1)
    assert splan(7, K=128, ws=None, ws_bytes=0)[0] == tm.GEMM_ERR_NULL
    # workspace checks: too small, misaligned, negative sizes and counts
    assert splan(2, ws_bytes=2 * 1024 * 1024 * 4)[0] == 0
    assert splan(2, ws_bytes=2 * 1024 * 1024 * 4 - 1)[0] == tm.GEMM_ERR_ARG
    assert splan(2, ws=P + 4)[0] == tm.GEMM_ERR_ARG
    assert splan(-1)[0] == tm.GEMM_ERR_ARG
    assert splan(0, ws_bytes=-1)[0] == tm.GEMM_ERR_ARG
    # layouts: MN-major operands split like K-major ones
    assert splan(0, la=MN, lb=MN)[:3] == (0, 16, "ring4_256")
    # the ring kernel cannot run (MN-major N not a multiple of 8): forced -> unsupported,
    # automatic -> one range on the general kernel
    assert splan(2, lb=MN, N=1020)[0] == tm.GEMM_ERR_UNSUPPORTED
    assert splan(0, lb=MN, N=1020)[:3] == (0, 1, "simple_64")
    # skinny M: the GEMV path, never split automatically
    assert splan(0, M=1)[:3] == (0, 1, "gemv_lds")
    assert splan(0, M=16)[:3] == (0, 1, "gemv")
    # K = 0: zero fill, whatever the count
    assert splan(0, K=0, lda=1, ldb=1)[:3] == (0, 1, "zero_fill")
    assert splan(5, K=0, lda=1, ldb=1)[:3] == (0, 1, "zero_fill")
    # bad arguments are reported as by the other entry points
    assert splan(2, lda=100)[0] == tm.GEMM_ERR_ARG


def mxplan(variant=0, fa=0, fb=0, M=4096, N=4096, K=4096, A=P, lda=None, SA=P, ldsa=None, B=P,
           ldb=None, SB=P, ldsb=None, out=0):
    lda = K if lda is None else lda
    ldb = K if ldb is None else ldb
    ldsa = max(K // 32, 1) if ldsa is None else ldsa
    ldsb = max(K // 32, 1) if ldsb is None else ldsb
    return tm.gemm_mx_plan(variant, fa, fb, M, N, K, A, lda, SA, ldsa, B, ldb, SB, ldsb, P, N, out,
                           256)


def test_mx_validation_and_plan():
    assert mxplan()[:2] == (0, "mx_ring_256") and mxplan()[2:] == (256, 256)
    assert mxplan(fa=1, fb=0, out=1)[:2] == (0, "mx_ring_256")
    # K not a multiple of 128, odd pitches, unaligned operands or scales: general kernel
    assert mxplan(K=4064)[:2] == (0, "mx_simple_64")
    assert mxplan(lda=4098)[:2] == (0, "mx_simple_64")
    assert mxplan(ldsa=130)[:2] == (0, "mx_simple_64")
    assert mxplan(A=P + 2)[:2] == (0, "mx_simple_64")
    assert mxplan(SB=P + 1)[:2] == (0, "mx_simple_64")
    assert mxplan(M=100, N=70, K=4064)[2] == 2 * 2
    # forced kernels
    assert mxplan(variant=1)[:2] == (0, "mx_simple_64")
    assert mxplan(variant=2, K=4064)[0] == tm.GEMM_ERR_UNSUPPORTED
    assert mxplan(variant=3)[0] == tm.GEMM_ERR_ARG
    # argument errors
    assert mxplan(K=4016)[0] == tm.GEMM_ERR_ARG          # K % 32
    assert mxplan(fa=2)[0] == tm.GEMM_ERR_ARG
    assert mxplan(lda=4095)[0] == tm.GEMM_ERR_ARG
    assert mxplan(ldsa=127)[0] == tm.GEMM_ERR_ARG
    assert mxplan(out=2)[0] == tm.GEMM_ERR_DTYPE
    assert mxplan(SA=None)[0] == tm.GEMM_ERR_NULL
    assert mxplan(M=-1)[0] == tm.GEMM_ERR_ARG
    # empty products
    assert mxplan(K=0, lda=1, ldb=1)[:2] == (0, "zero_fill")
    assert mxplan(M=0)[:2] == (0, "none")
    v = tm.gemm_mx_validate
    assert v(0, 0, 64, 64, 64, P, 64, P, 2, P, 64, P, 2, P, 64, 0) == tm.GEMM_OK
    assert v(0, 0, 64, 64, 64, P, 64, P, 1, P, 64, P, 2, P, 64, 0) == tm.GEMM_ERR_ARG


def test_attention_plan_variants():
    """Host-only planning of the attention forward: each variant's kernel, the MFMA kernels'
    preconditions (d = 64 or 128) and the workgroup grid (128 queries per workgroup)."""
    P = 1 << 12
    def aplan(variant, d=128, Lq=4096):
        return tm.attention_fwd_plan(variant, 1, 32, 8, Lq, 4096, d, P, P, P, P, 0.088, 1, 1, 256)
    assert aplan(tm.ATTN_VARIANT_MFMA)[:2] == (0, "attn_mfma")
    assert aplan(tm.ATTN_VARIANT_PIPE)[:2] == (0, "attn_pipe")
    assert aplan(tm.ATTN_VARIANT_SIMPLE)[:2] == (0, "attn_simple")
    assert aplan(tm.ATTN_VARIANT_AUTO)[1] in ("attn_mfma", "attn_pipe")
    assert aplan(tm.ATTN_VARIANT_PIPE)[2] == 32 * 32          # 32 query blocks x 32 heads
    assert aplan(tm.ATTN_VARIANT_PIPE, d=64)[:2] == (0, "attn_pipe")
    assert aplan(tm.ATTN_VARIANT_PIPE, d=32)[0] == tm.GEMM_ERR_UNSUPPORTED
    assert aplan(tm.ATTN_VARIANT_AUTO, d=32)[:2] == (0, "attn_simple")
    assert aplan(4)[0] == tm.GEMM_ERR_ARG


def test_splitk_noalloc_host_checks():
    """gemm_bf16_splitk_noalloc's argument checks run on the host before any device call."""
    f = tm.library().gemm_bf16_splitk_noalloc
    args = lambda splits, M=1024, N=4096, K=4096, batch=1: (0, 0, splits, batch, M, N, K, P, K, 0, P, K, 0, P, N,
                                                           0, 0, None)
    assert f(*args(-1)) == tm.GEMM_ERR_ARG
    # 8 ranges of 1024 x 4096 fp32 partials: 128 MiB, beyond the 64 MiB scratch
    assert f(*args(8)) == tm.GEMM_ERR_SCRATCH
    # the count is capped at ceil(K / 64) before the check: K = 320 gives at most 5 ranges of
    # 16 MiB, 80 MiB (the accepted side of the limit launches work, so no fake pointer takes it)
    assert f(*args(80, K=320)) == tm.GEMM_ERR_SCRATCH
    assert tm.gemm_bf16_status_string(tm.GEMM_ERR_SCRATCH).startswith("GEMM_ERR_SCRATCH")
    # a bad argument is reported before the size
    assert f(*(args(8)[:8] + (100,) + args(8)[9:])) == tm.GEMM_ERR_ARG


def test_ceiling_library_exports_and_checks():
    """libtmm_ceiling.so (the measurement kernels bench.py runs beside the GEMV) exports what
    include/ceiling.h declares and rejects bad arguments on the host."""
    import re
    from tiled_matmul_amd import ceiling as cl
    lib = cl.library()
    text = re.sub(r"/\*.*?\*/", "", open(cl.HEADER).read(), flags=re.S)
    names = re.findall(r"^\s*int\s+(ceiling_\w+)\s*\(", text, re.M)
    assert sorted(names) == ["ceiling_launch_floor", "ceiling_stream_read"]
    for n in names:
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value
    assert lib.ceiling_stream_read(P, 1000, P, 256, 256, None) == 1        # not a multiple of 16
    assert lib.ceiling_stream_read(P + 8, 1024, P, 256, 256, None) == 1    # misaligned
    assert lib.ceiling_stream_read(P, 1 << 31, P, 256, 256, None) == 1     # too large
    assert lib.ceiling_stream_read(P, 1024, P, 256, 96, None) == 1         # block not a multiple of 64
    assert lib.ceiling_stream_read(None, 1024, P, 256, 256, None) == 1
    assert lib.ceiling_launch_floor(0, 64, None) == 1


def kplan(mode, M=4096, N=4096, K=4096, batch=1, cus=256, A=P, lda=None):
    lda = K if lda is None else lda
    sA, sB, sC = (M * lda, N * lda, M * N) if batch > 1 else (0, 0, 0)
    return tm.gemm_bf16_streamk_plan(mode, batch, M, N, K, A, lda, sA, P, lda, sB, P, N, sC, 0, cus)


def test_streamk_plan():
    AUTO, DP, ALL = tm.GEMM_STREAMK_AUTO, tm.GEMM_STREAMK_DP, tm.GEMM_STREAMK_ALL
    # 256 tiles on 256 compute units: whole tiles only, the 16 KB of counters only
    rc, ws, dp, sk, slots, grid = kplan(AUTO)
    assert (rc, dp, sk, slots, grid) == (0, 256, 0, 0, 256) and ws == 16384
    # 289 tiles (one wave and 33): all 289 as stream-K slots of ceil(289 * 64 / 256) = 73 blocks
    rc, ws, dp, sk, slots, grid = kplan(AUTO, M=4352, N=4352)
    assert (rc, dp, sk) == (0, 0, 289)
    assert slots == -(-289 * 64 // 73) == 254 and grid == 254
    assert ws == 16384 + slots * 2 * 256 * 256 * 4
    # 600 tiles (two waves and 88): 256 whole, then 256 + 88 cut
    rc, ws, dp, sk, slots, grid = kplan(AUTO, M=6144, N=6400)
    assert (rc, dp, sk, grid) == (0, 256, 344, 256)
    # fewer tiles than compute units: whole tiles (AUTO, DP), all cut (ALL)
    assert kplan(AUTO, M=3000, N=5000, K=4096)[2:5] == (240, 0, 0)
    rc, ws, dp, sk, slots, grid = kplan(ALL, M=3000, N=5000, K=4096)
    assert (dp, sk, slots, grid) == (0, 240, 256, 256)
    assert kplan(DP, M=4352, N=4352)[2:5] == (289, 0, 0)
    # at least 4 K blocks per slot: 16 tiles x 16 blocks -> 64 slots of 4
    assert kplan(ALL, M=1000, N=1000, K=1000)[2:6] == (0, 16, 64, 64)
    # fewer than 4 blocks per tile: slots of 4 blocks spanning two tiles
    assert kplan(ALL, M=1000, N=1000, K=136)[2:6] == (0, 16, 12, 12)
    # errors: unknown mode, unaligned rows (ring kernel preconditions)
    assert kplan(3)[0] == tm.GEMM_ERR_ARG
    assert kplan(AUTO, A=P + 2)[0] == tm.GEMM_ERR_UNSUPPORTED
    assert kplan(AUTO, K=4095, lda=4095)[0] == tm.GEMM_ERR_UNSUPPORTED
    # a device beyond 800 compute units would need more than the 16 KB of counters
    assert kplan(AUTO, cus=900, M=8192, N=8192)[0] == tm.GEMM_ERR_UNSUPPORTED
