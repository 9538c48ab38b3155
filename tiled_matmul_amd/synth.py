"""Seeded synthetic inputs for the bf16 GEMM, shared by the tests, the bench and the oracle's
callers.  This module holds none of the GEMM's arithmetic: it only draws numbers and rounds
them to bf16 bit patterns (uint16 arrays), which are then handed unchanged to both the GPU
path and the CPU oracle.

Generator.  SplitMix64 (G. L. Steele, D. Lea, C. H. Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014), used counter-based: the draw with counter c under seed s
is mix64(key(s) + (c + 1) * 0x9E3779B97F4A7C15) with key(s) = mix64(s), so any element can
be regenerated on its own.  Element (r, c) of a rows x cols operand uses counter r*cols + c
(independent of the row pitch).

Distributions:
  uniform [lo, hi):  u = (z >> 40) * 2^-24 in [0, 1);  lo + (hi - lo) * u
  normal (0, s^2):   Box-Muller from the draws 2e and 2e+1 of element e:
                     u1 = ((z1 >> 11) + 1) * 2^-53 in (0, 1], u2 = (z2 >> 11) * 2^-53,
                     s * sqrt(-2 ln u1) * cos(2 pi u2)
  integer [lo, hi]:  lo + (z >> 32) mod (hi - lo + 1)   (exactly representable in bf16)
Every value is rounded binary64 -> binary32 (nearest even) -> bf16 (nearest even).
Columns beyond ``cols`` in a padded row (pitch ``ld`` > cols) hold a quiet-NaN pattern, so
a kernel that reads past K poisons its output.
"""
from __future__ import annotations

import hashlib

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
PAD_BITS = 0x7FC0          # bf16 quiet NaN written into row padding
_CHUNK = 1 << 22           # elements per generation chunk (bounds temporaries)


def _mix64(z: np.ndarray, tmp: np.ndarray | None = None) -> np.ndarray:
    """SplitMix64's output function, in place on z (uint64); returns z."""
    if tmp is None:
        tmp = np.empty_like(z)
    with np.errstate(over="ignore"):
        np.right_shift(z, np.uint64(30), out=tmp)
        np.bitwise_xor(z, tmp, out=z)
        np.multiply(z, _M1, out=z)
        np.right_shift(z, np.uint64(27), out=tmp)
        np.bitwise_xor(z, tmp, out=z)
        np.multiply(z, _M2, out=z)
        np.right_shift(z, np.uint64(31), out=tmp)
        np.bitwise_xor(z, tmp, out=z)
    return z


def _key(seed: int) -> np.uint64:
    return _mix64(np.array([seed & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64))[0]


def draws(seed: int, start: int, count: int, out: np.ndarray | None = None,
          tmp: np.ndarray | None = None) -> np.ndarray:
    """Raw 64-bit draws with counters start .. start+count-1 (optionally into ``out``)."""
    z = np.empty(count, dtype=np.uint64) if out is None else out[:count]
    t = None if tmp is None else tmp[:count]
    z[:] = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        np.multiply(z, GAMMA, out=z)
        np.add(z, _key(seed), out=z)
    return _mix64(z, t)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """binary32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


class _Work:
    """Scratch buffers reused across chunks (fresh allocations are the slow part)."""

    def __init__(self, n: int):
        self.z = np.empty(2 * n, dtype=np.uint64)
        self.t = np.empty(2 * n, dtype=np.uint64)
        self.f = np.empty(n, dtype=np.float64)
        self.g = np.empty(n, dtype=np.float64)
        self.h = np.empty(n, dtype=np.float64)


def _values(kind: str, seed: int, start: int, count: int, p, w: _Work | None = None):
    """binary64 values of elements start .. start+count-1 (a view into ``w``)."""
    w = _Work(count) if w is None else w
    f, g, h = w.f[:count], w.g[:count], w.h[:count]
    if kind == "uniform":
        lo, hi = p
        z = draws(seed, start, count, w.z, w.t)
        np.right_shift(z, np.uint64(40), out=z)
        f[:] = z
        np.multiply(f, (hi - lo) * 2.0 ** -24, out=f)
        np.add(f, lo, out=f)
        return f
    if kind == "normal":
        (sigma,) = p
        z = draws(seed, 2 * start, 2 * count, w.z, w.t)
        np.right_shift(z, np.uint64(11), out=z)
        f[:] = z[0::2]                     # u1 = (z1 + 1) 2^-53 in (0, 1]
        np.add(f, 1.0, out=f)
        np.multiply(f, 2.0 ** -53, out=f)
        g[:] = z[1::2]                     # u2 = z2 2^-53 in [0, 1)
        np.multiply(g, 2.0 ** -53, out=g)
        np.log(f, out=f)                   # r = sigma sqrt(-2 ln u1)
        np.multiply(f, -2.0, out=f)
        np.sqrt(f, out=f)
        np.multiply(f, sigma, out=f)
        np.multiply(g, 2.0 * np.pi, out=h)  # cos(2 pi u2)
        np.cos(h, out=h)
        np.multiply(f, h, out=f)
        return f
    if kind == "integer":
        lo, hi = p
        z = draws(seed, start, count, w.z, w.t)
        np.right_shift(z, np.uint64(32), out=z)
        np.remainder(z, np.uint64(hi - lo + 1), out=z)
        f[:] = z
        np.add(f, lo, out=f)
        return f
    raise ValueError(f"unknown distribution {kind!r}")


def operand(kind: str, rows: int, cols: int, seed: int, params=(), ld: int | None = None,
            row_offset: int = 0) -> np.ndarray:
    """A rows x ld uint16 array of bf16 bit patterns; columns >= cols are NaN padding.

    ``row_offset`` regenerates rows row_offset .. row_offset+rows-1 of a larger operand.
    """
    ld = cols if ld is None else ld
    if ld < cols:
        raise ValueError("ld < cols")
    out = np.full((rows, ld), PAD_BITS, dtype=np.uint16)
    if rows == 0 or cols == 0:
        return out
    rows_per_chunk = max(1, _CHUNK // cols)
    w = _Work(min(rows, rows_per_chunk) * cols)
    f32 = np.empty(min(rows, rows_per_chunk) * cols, dtype=np.float32)
    for r0 in range(0, rows, rows_per_chunk):
        r1 = min(rows, r0 + rows_per_chunk)
        n = (r1 - r0) * cols
        v = _values(kind, seed, (row_offset + r0) * cols, n, params, w)
        f32[:n] = v
        out[r0:r1, :cols] = f32_to_bf16_bits(f32[:n]).reshape(r1 - r0, cols)
    return out


def uniform(rows, cols, seed, lo=-1.0, hi=1.0, ld=None):
    return operand("uniform", rows, cols, seed, (lo, hi), ld)


def normal(rows, cols, seed, sigma=1.0, ld=None):
    return operand("normal", rows, cols, seed, (sigma,), ld)


def integers(rows, cols, seed, lo=-4, hi=4, ld=None):
    return operand("integer", rows, cols, seed, (lo, hi), ld)


def sha256(x: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(x).tobytes()).hexdigest()


# ---------------------------------------------------------------------------------------
# The workloads.  Shapes, value distributions and output types of the five configurations
# the GEMM is measured and checked on; seeds are 1000*cfg for A and 1000*cfg+1 for B, and
# batch item b adds 2*b to both.
# ---------------------------------------------------------------------------------------
OUT_FP32, OUT_BF16 = 0, 1

WORKLOADS = {
    "single_tile_128": dict(cfg=1, M=128, N=128, K=128, batch=1,
                            a=("uniform", (-1.0, 1.0)), b=("uniform", (-1.0, 1.0)),
                            out=OUT_FP32),
    "square_4096": dict(cfg=2, M=4096, N=4096, K=4096, batch=1,
                        a=("normal", (1.0,)), b=("normal", (1.0,)), out=OUT_FP32),
    "gemv_m1": dict(cfg=3, M=1, N=4096, K=4096, batch=1,
                    a=("normal", (1.0,)), b=("normal", (0.02,)), out=OUT_FP32),
    "gemv_m16": dict(cfg=3, M=16, N=4096, K=4096, batch=1,
                     a=("normal", (1.0,)), b=("normal", (0.02,)), out=OUT_FP32),
    "ffn_up_8192x14336x4096": dict(cfg=4, M=8192, N=14336, K=4096, batch=1,
                                   a=("normal", (1.0,)), b=("normal", (0.02,)),
                                   out=OUT_BF16),
    "ffn_down_8192x4096x14336": dict(cfg=4, M=8192, N=4096, K=14336, batch=1,
                                     a=("normal", (1.0,)), b=("normal", (0.02,)),
                                     out=OUT_BF16),
    "irregular_3000x5000x4100": dict(cfg=5, M=3000, N=5000, K=4100, batch=1,
                                     a=("uniform", (-1.0, 1.0)), b=("uniform", (-1.0, 1.0)),
                                     out=OUT_FP32),
    "batched_64x256x256x1024": dict(cfg=5, M=256, N=256, K=1024, batch=64,
                                    a=("uniform", (-1.0, 1.0)), b=("uniform", (-1.0, 1.0)),
                                    out=OUT_FP32),
    # Not one of the five: the FFN down projection for a batch of 256 tokens (few output
    # tiles, long K), the shape split K is for.  The FFN configuration's distributions.
    "ffn_down_256x4096x14336": dict(cfg=4, M=256, N=4096, K=14336, batch=1,
                                    a=("normal", (1.0,)), b=("normal", (0.02,)),
                                    out=OUT_BF16),
    # Not one of the five: a square GEMM with 17 x 17 = 289 tiles of 256 x 256, one more than a
    # wave of 256 compute units (with some to spare), the shape stream-K is for.  The square
    # configuration's distributions.
    "square_4352x4352x4096": dict(cfg=2, M=4352, N=4352, K=4096, batch=1,
                                  a=("normal", (1.0,)), b=("normal", (1.0,)), out=OUT_FP32),
}


def seeds(cfg: int, item: int = 0):
    return 1000 * cfg + 2 * item, 1000 * cfg + 1 + 2 * item


def make_operands(name: str, item: int = 0, lda=None, ldb=None, rows=None, row_offset=0):
    """(A, B) bit-pattern arrays of workload ``name`` (batch item ``item``).

    ``rows``/``row_offset`` restrict A to a band of rows (for sampled checks at full size).
    """
    w = WORKLOADS[name]
    sa, sb = seeds(w["cfg"], item)
    M = w["M"] if rows is None else rows
    A = operand(w["a"][0], M, w["K"], sa, w["a"][1], lda, row_offset=row_offset)
    B = operand(w["b"][0], w["N"], w["K"], sb, w["b"][1], ldb)
    return A, B


# ---------------------------------------------------------------------------------------
# Block-scaled 8-bit operands (gemm_mx): element codes (uint8) and one E8M0 scale code per
# 32 consecutive columns.  Values are drawn as above and quantised per block of 32 the way
# the OCP microscaling format describes: shared exponent X = floor(log2(max |v|)) - emax of
# the element format (8 for E4M3, 15 for E5M2), scale code X + 127 (clamped to 0 .. 254),
# elements v / 2^X rounded to nearest even in the element format, saturating at its largest
# finite value.  Padding columns hold a NaN code (and padding scale columns 0xFF, NaN), so a
# kernel that reads them fails the check.
# ---------------------------------------------------------------------------------------
MX_E4M3, MX_E5M2 = 0, 1
_MX_EMAX = {MX_E4M3: 8, MX_E5M2: 15}
_MX_MAX = {MX_E4M3: 448.0, MX_E5M2: 57344.0}
MX_PAD_CODE = 0x7F        # NaN in both formats
MX_PAD_SCALE = 0xFF       # NaN scale


def fp8_codes(x: np.ndarray, fmt: int) -> np.ndarray:
    """float values -> 8-bit codes (round to nearest even, saturating)."""
    import torch
    dt = torch.float8_e4m3fn if fmt == MX_E4M3 else torch.float8_e5m2
    m = _MX_MAX[fmt]
    x32 = np.clip(np.asarray(x, dtype=np.float64), -m, m).astype(np.float32)
    return torch.from_numpy(np.ascontiguousarray(x32)).to(dt).view(torch.uint8).numpy()


def _mx_pad(rows, cols, ld, lds):
    ld = cols if ld is None else ld
    lds = cols // 32 if lds is None else lds
    if cols % 32:
        raise ValueError("columns must be a multiple of 32")
    if ld < cols or lds < cols // 32:
        raise ValueError("pitch below the extent")
    return (np.full((rows, ld), MX_PAD_CODE, dtype=np.uint8),
            np.full((rows, lds), MX_PAD_SCALE, dtype=np.uint8))


def mx_operand(kind: str, rows: int, cols: int, seed: int, fmt: int, params=(), ld=None,
               lds=None, row_offset: int = 0):
    """(codes rows x ld, scales rows x lds) of ``kind`` values quantised to the MX format."""
    codes, scales = _mx_pad(rows, cols, ld, lds)
    if rows == 0 or cols == 0:
        return codes, scales
    rows_per_chunk = max(1, _CHUNK // cols)
    w = _Work(min(rows, rows_per_chunk) * cols)
    for r0 in range(0, rows, rows_per_chunk):
        r1 = min(rows, r0 + rows_per_chunk)
        v = _values(kind, seed, (row_offset + r0) * cols, (r1 - r0) * cols, params, w)
        blk = v.reshape(r1 - r0, cols // 32, 32)
        amax = np.abs(blk).max(axis=2)
        with np.errstate(divide="ignore"):
            X = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - _MX_EMAX[fmt]
        X = np.where(amax > 0, X, -127.0)
        sc = np.clip(X + 127, 0, 254)
        q = blk / np.exp2(sc - 127)[:, :, None]
        codes[r0:r1, :cols] = fp8_codes(q.reshape(r1 - r0, cols), fmt)
        scales[r0:r1, :cols // 32] = sc.astype(np.uint8)
    return codes, scales


def mx_integers(rows: int, cols: int, seed: int, fmt: int, lo=-4, hi=4, scale_lo=126,
                scale_hi=128, ld=None, lds=None):
    """Integer elements in [lo, hi] (exact in both formats for |v| <= 4) and scale codes in
    [scale_lo, scale_hi], each from its own counter stream."""
    codes, scales = _mx_pad(rows, cols, ld, lds)
    if rows == 0 or cols == 0:
        return codes, scales
    v = _values("integer", seed, 0, rows * cols, (lo, hi)).reshape(rows, cols)
    codes[:, :cols] = fp8_codes(v, fmt)
    s = _values("integer", seed + 7919, 0, rows * (cols // 32), (scale_lo, scale_hi))
    scales[:, :cols // 32] = s.reshape(rows, cols // 32).astype(np.uint8)
    return codes, scales


# Workloads of the block-scaled GEMM: the square and FFN shapes above with the same value
# distributions, quantised to MXFP8.
MX_WORKLOADS = {
    "mx_e4m3_square_4096": dict(cfg=2, M=4096, N=4096, K=4096, fa=MX_E4M3, fb=MX_E4M3,
                                a=("normal", (1.0,)), b=("normal", (1.0,)), out=OUT_FP32),
    "mx_e5m2_e4m3_square_4096": dict(cfg=2, M=4096, N=4096, K=4096, fa=MX_E5M2, fb=MX_E4M3,
                                     a=("normal", (1.0,)), b=("normal", (1.0,)), out=OUT_FP32),
    "mx_e4m3_ffn_up_8192x14336x4096": dict(cfg=4, M=8192, N=14336, K=4096, fa=MX_E4M3,
                                           fb=MX_E4M3, a=("normal", (1.0,)),
                                           b=("normal", (0.02,)), out=OUT_BF16),
}


def make_mx_operands(name: str, rows=None, row_offset=0):
    """(A, SA, B, SB) of MX workload ``name``; ``rows``/``row_offset`` select a band of A."""
    w = MX_WORKLOADS[name]
    sa, sb = seeds(w["cfg"])
    M = w["M"] if rows is None else rows
    A, SA = mx_operand(w["a"][0], M, w["K"], sa, w["fa"], w["a"][1], row_offset=row_offset)
    B, SB = mx_operand(w["b"][0], w["N"], w["K"], sb, w["fb"], w["b"][1])
    return A, SA, B, SB


# Attention forward workloads: [B][H][L][d] bf16 tensors of N(0,1) values (Q, K, V from their
# own seeds), scale 1/sqrt(d).  A 4096-token causal prefill with grouped-query heads (32 query
# heads over 8 key/value heads, d = 128) and a full (unmasked) attention with d = 64.
ATTN_WORKLOADS = {
    "attn_prefill_b1_h32_kv8_l4096_d128": dict(B=1, Hq=32, Hkv=8, Lq=4096, Lk=4096, d=128,
                                               causal=True, scale=128 ** -0.5, out=OUT_BF16,
                                               seed=6000),
    "attn_full_b2_h16_l2048_d64": dict(B=2, Hq=16, Hkv=16, Lq=2048, Lk=2048, d=64,
                                       causal=False, scale=64 ** -0.5, out=OUT_FP32, seed=6100),
}


def make_attention_inputs(name: str):
    """(Q, K, V) bf16 bit arrays of attention workload ``name``."""
    w = ATTN_WORKLOADS[name]
    B, Hq, Hkv, Lq, Lk, d, s = w["B"], w["Hq"], w["Hkv"], w["Lq"], w["Lk"], w["d"], w["seed"]
    Q = normal(B * Hq * Lq, d, s).reshape(B, Hq, Lq, d)
    K = normal(B * Hkv * Lk, d, s + 1).reshape(B, Hkv, Lk, d)
    V = normal(B * Hkv * Lk, d, s + 2).reshape(B, Hkv, Lk, d)
    return Q, K, V
