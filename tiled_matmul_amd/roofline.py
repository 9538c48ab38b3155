"""Roofline arithmetic for the GEMM C = A * B^T (host logic, no GPU).

The roofline of the page "读书笔记-《面向机器学习系统的现代 GPU 编程》" (section "Roofline"):
attainable FLOP/s is the smaller of the compute peak and bandwidth x arithmetic intensity,
where arithmetic intensity (AI) is FLOPs per byte moved to or from HBM, and the ridge point
peak / bandwidth separates bandwidth-bound from compute-bound kernels.

Algorithmic bytes count each operand read once and C written once:
    bytes = (M*K + N*K) * in_bytes + M*N * out_bytes       (times the batch)
    flops = 2 * M * N * K                                  (times the batch)
This is the minimum traffic of any schedule, not what a given tiling re-reads.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Machine:
    name: str
    peak_tflops: float      # dense matrix peak for the contraction's input type
    hbm_tb_s: float         # peak HBM bandwidth

    @property
    def ridge(self) -> float:
        """FLOP per byte at which the two roofs meet."""
        return self.peak_tflops * 1e12 / (self.hbm_tb_s * 1e12)


# AMD's published MI355X figures: dense bf16 MFMA 2.5 PFLOP/s, HBM3E 8 TB/s.
MI355X_BF16 = Machine("MI355X bf16 dense", 2500.0, 8.0)
# 256 CUs x 4096 bf16 FLOP/clk/CU x 2.4 GHz, the clock-derived figure behind the headline.
MI355X_BF16_CLOCK_DERIVED_TFLOPS = 256 * 4096 * 2.4e9 / 1e12


def flops(M: int, N: int, K: int, batch: int = 1) -> int:
    return 2 * M * N * K * batch


def algorithmic_bytes(M: int, N: int, K: int, out_bytes: int, in_bytes: int = 2,
                      batch: int = 1) -> int:
    return ((M * K + N * K) * in_bytes + M * N * out_bytes) * batch


def intensity(M: int, N: int, K: int, out_bytes: int, in_bytes: int = 2,
              batch: int = 1) -> float:
    return flops(M, N, K, batch) / algorithmic_bytes(M, N, K, out_bytes, in_bytes, batch)


def attainable_tflops(machine: Machine, ai: float) -> float:
    """min(peak, bandwidth * AI), in TFLOP/s."""
    return min(machine.peak_tflops, machine.hbm_tb_s * ai)


def bound(machine: Machine, ai: float) -> str:
    """'mfma' above the ridge (compute-bound), 'hbm' below it (bandwidth-bound)."""
    return "mfma" if ai >= machine.ridge else "hbm"


def roofline_time_s(machine: Machine, M: int, N: int, K: int, out_bytes: int,
                    in_bytes: int = 2, batch: int = 1) -> float:
    f = flops(M, N, K, batch)
    b = algorithmic_bytes(M, N, K, out_bytes, in_bytes, batch)
    return max(f / (machine.peak_tflops * 1e12), b / (machine.hbm_tb_s * 1e12))
