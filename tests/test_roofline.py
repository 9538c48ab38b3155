"""Roofline arithmetic pinned to the figures the page "读书笔记-《面向机器学习系统的现代 GPU
编程》" prints in its section "Roofline" (tests/golden/roofline_pages.json).  No GPU."""
import json
import os

import pytest

from tiled_matmul_amd import roofline as rl

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "roofline_pages.json")))


def close(a, b):
    return abs(a - b) <= G["rel_tol"] * abs(b)


def test_b200_ridge():
    b200 = rl.Machine("B200", G["b200_fp16_peak_tflops"], G["b200_hbm_tb_s"])
    assert close(b200.ridge, G["b200_ridge_flop_per_byte"])


@pytest.mark.parametrize("case", ["gemm_4096x4096_fp16", "decode_1x4096x4096_fp16"])
def test_worked_intensities(case):
    c = G[case]
    ai = rl.intensity(c["M"], c["N"], c["K"], c["out_bytes"], c["in_bytes"])
    assert close(ai, c["ai"])
    b200 = rl.Machine("B200", G["b200_fp16_peak_tflops"], G["b200_hbm_tb_s"])
    assert rl.bound(b200, ai) == {"compute": "mfma", "bandwidth": "hbm"}[c["bound"]]


def test_exact_counts():
    assert rl.flops(4096, 4096, 4096) == 137438953472
    assert rl.algorithmic_bytes(4096, 4096, 4096, 4) == 134217728
    assert rl.algorithmic_bytes(1, 4096, 4096, 4) == 33579008
    assert rl.algorithmic_bytes(256, 256, 1024, 4, batch=64) == 83886080
    assert rl.intensity(4096, 4096, 4096, 4) == 1024.0


def test_mi355x_roofs():
    m = rl.MI355X_BF16
    assert abs(m.ridge - 312.5) < 1e-9
    assert rl.bound(m, rl.intensity(4096, 4096, 4096, 4)) == "mfma"
    assert rl.bound(m, rl.intensity(1, 4096, 4096, 4)) == "hbm"
    t = rl.roofline_time_s(m, 4096, 4096, 4096, 4)
    assert abs(t - 137438953472 / 2.5e15) < 1e-15
    assert abs(rl.MI355X_BF16_CLOCK_DERIVED_TFLOPS - 2516.5824) < 1e-6
