"""GPU parity of the attention forward (attention_fwd, attention_fwd_variant) against the CPU
oracle (oracle/attention.py), within the bound of oracle/check.py (check_attention), for O
and LSE.  Cases: grouped-query heads, causal and full masks, Lq < Lk, Lq > Lk (rows with no
key), a single query (decode), head dimensions 32/64/128, partial query and key blocks, both
output types, argument errors, and the prefill workload at full size on sampled heads/rows."""
import math

import numpy as np
import pytest

import oracle
from oracle import attention as att
from oracle import check as ck
import tiled_matmul_amd as tm
from tiled_matmul_amd import synth

from helpers import OUT_BF16, OUT_FP32, to_device

pytestmark = pytest.mark.gpu

AUTO, SIMPLE, MFMA, PIPE = tm.ATTN_VARIANT_AUTO, tm.ATTN_VARIANT_SIMPLE, tm.ATTN_VARIANT_MFMA, tm.ATTN_VARIANT_PIPE


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield


def run(Q, K, V, scale, causal, out_dtype, variant=AUTO):
    import torch
    B, Hq, Lq, d = Q.shape
    Hkv, Lk = K.shape[1], K.shape[2]
    dt = torch.float32 if out_dtype == OUT_FP32 else torch.int16
    O = torch.full((B, Hq, Lq, d), 7, dtype=dt, device="cuda")
    LSE = torch.full((B, Hq, Lq), 7.0, dtype=torch.float32, device="cuda")
    tm.attention_fwd_variant(variant, B, Hq, Hkv, Lq, Lk, d, to_device(Q), to_device(K),
                             to_device(V), O, LSE, scale, causal, out_dtype)
    torch.cuda.synchronize()
    o = O.cpu().numpy()
    if out_dtype == OUT_BF16:
        o = o.view(np.uint16)
    return o, LSE.cpu().numpy()


def qkv(B, Hq, Hkv, Lq, Lk, d, seed):
    Q = synth.normal(B * Hq * Lq, d, seed).reshape(B, Hq, Lq, d)
    K = synth.normal(B * Hkv * Lk, d, seed + 1).reshape(B, Hkv, Lk, d)
    V = synth.normal(B * Hkv * Lk, d, seed + 2).reshape(B, Hkv, Lk, d)
    return Q, K, V


def check(o, lse, Q, K, V, scale, causal, out_dtype, heads=None, rows=None, what=""):
    O, LSE, PV, SM = att.attention(Q, K, V, scale, causal, heads=heads, rows=rows)
    B, Hq = Q.shape[0], Q.shape[1]
    hs = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else heads
    rs = np.arange(Q.shape[2]) if rows is None else np.asarray(rows)
    og = np.stack([o[b, h][rs] for b, h in hs])
    lg = np.stack([lse[b, h][rs] for b, h in hs])
    r = ck.check_attention(og, O, PV, SM, K.shape[2], out_dtype, lg, LSE)
    assert r["ok"], f"{what}: {r}"


CASES = [  # B, Hq, Hkv, Lq, Lk, d, causal
    (1, 2, 2, 64, 64, 64, False), (2, 4, 2, 100, 100, 128, True), (1, 8, 2, 37, 129, 64, True),
    (1, 2, 1, 70, 40, 128, True), (1, 4, 4, 1, 300, 128, True), (1, 2, 2, 130, 130, 32, False),
    (2, 2, 1, 256, 256, 128, True), (1, 4, 1, 200, 333, 128, False), (1, 2, 2, 128, 128, 64, True),
]


@pytest.mark.parametrize("B,Hq,Hkv,Lq,Lk,d,causal", CASES)
def test_attention_parity(B, Hq, Hkv, Lq, Lk, d, causal):
    Q, K, V = qkv(B, Hq, Hkv, Lq, Lk, d, 1000 + Lq + Lk + d)
    scale = 1.0 / math.sqrt(d)
    P = 1 << 12
    kname = tm.attention_fwd_plan(AUTO, B, Hq, Hkv, Lq, Lk, d, P, P, P, P, scale, causal, 0)[1]
    variants = [AUTO, SIMPLE] + ([MFMA, PIPE] if kname in ("attn_mfma", "attn_pipe") else [])
    for variant in variants:
        for out_dtype in (OUT_FP32, OUT_BF16):
            o, lse = run(Q, K, V, scale, causal, out_dtype, variant)
            check(o, lse, Q, K, V, scale, causal, out_dtype,
                  what=f"variant {variant} out {out_dtype} ({kname})")


def test_attention_empty_and_errors():
    import torch
    Q, K, V = qkv(1, 2, 1, 8, 8, 64, 1100)
    # Lk = 0: every row empty
    O = torch.full((1, 2, 8, 64), 3.0, device="cuda")
    LSE = torch.zeros((1, 2, 8), device="cuda")
    tm.attention_fwd(1, 2, 1, 8, 0, 64, to_device(Q), to_device(K), to_device(V), O, LSE, 0.1,
                     1, OUT_FP32)
    torch.cuda.synchronize()
    assert torch.all(O == 0) and torch.all(torch.isneginf(LSE))
    for args, code in [((1, 3, 2, 8, 8, 64), tm.GEMM_ERR_ARG), ((1, 2, 1, 8, 8, 12), tm.GEMM_ERR_ARG),
                       ((1, 2, 1, 8, 8, 264), tm.GEMM_ERR_ARG)]:
        with pytest.raises(tm.GemmError) as e:
            tm.attention_fwd(*args, to_device(Q), to_device(K), to_device(V), O, LSE, 0.1, 1,
                             OUT_FP32)
        assert e.value.status == code
    for variant in (MFMA, PIPE):   # the MFMA kernels take d = 64 and 128 only
        with pytest.raises(tm.GemmError) as e:
            tm.attention_fwd_variant(variant, 1, 2, 1, 8, 8, 32, to_device(Q), to_device(K),
                                     to_device(V), O, LSE, 0.1, 1, OUT_FP32)
        assert e.value.status == tm.GEMM_ERR_UNSUPPORTED


def test_attention_lse_optional_and_deterministic():
    import torch
    Q, K, V = qkv(1, 4, 2, 96, 96, 128, 1110)
    Qd, Kd, Vd = to_device(Q), to_device(K), to_device(V)
    O1 = torch.empty((1, 4, 96, 128), device="cuda")
    O2 = torch.empty((1, 4, 96, 128), device="cuda")
    for variant in (AUTO, MFMA, PIPE):
        tm.attention_fwd_variant(variant, 1, 4, 2, 96, 96, 128, Qd, Kd, Vd, O1, None, 0.09, 1, OUT_FP32)
        tm.attention_fwd_variant(variant, 1, 4, 2, 96, 96, 128, Qd, Kd, Vd, O2, None, 0.09, 1, OUT_FP32)
        torch.cuda.synchronize()
        assert torch.equal(O1, O2), variant


@pytest.mark.parametrize("variant", [AUTO, MFMA, PIPE])
@pytest.mark.parametrize("name", sorted(synth.ATTN_WORKLOADS))
def test_attention_workloads_full_size_sampled(name, variant):
    w = synth.ATTN_WORKLOADS[name]
    Q, K, V = synth.make_attention_inputs(name)
    o, lse = run(Q, K, V, w["scale"], w["causal"], w["out"], variant)
    B, Hq = w["B"], w["Hq"]
    rng = np.random.default_rng(3)
    heads = sorted({(0, 0), (B - 1, Hq - 1)} | {(int(rng.integers(B)), int(rng.integers(Hq))) for _ in range(3)})
    rows = sorted({0, 1, 63, 64, w["Lq"] - 1} | set(rng.integers(0, w["Lq"], 6).tolist()))
    check(o, lse, Q, K, V, w["scale"], w["causal"], w["out"], heads=heads, rows=rows, what=name)
