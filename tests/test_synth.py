"""The seeded input generator: published SplitMix64 outputs, determinism, distributions,
bf16 rounding (against torch's conversion), padding.  No GPU."""
import os

import numpy as np
import pytest

from tiled_matmul_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_published_sequence():
    want = [int(l, 16) for l in open(os.path.join(GOLDEN, "splitmix64_seed0.txt"))
            if l.strip() and not l.startswith("#")]
    state = np.array([(i + 1) * 0x9E3779B97F4A7C15 % 2 ** 64 for i in range(3)],
                     dtype=np.uint64)
    got = [int(v) for v in synth._mix64(state.copy())]
    assert got == want


def test_counter_based_and_deterministic():
    a = synth.draws(42, 0, 1000)
    b = synth.draws(42, 0, 1000)
    assert np.array_equal(a, b)
    assert np.array_equal(synth.draws(42, 300, 50), a[300:350])
    assert not np.array_equal(synth.draws(43, 0, 1000), a)


def test_row_offset_regenerates_band():
    full = synth.normal(40, 33, 9)
    band = synth.operand("normal", 7, 33, 9, (1.0,), row_offset=20)
    assert np.array_equal(band, full[20:27])


def test_padding_is_nan():
    x = synth.uniform(5, 10, 1, ld=16)
    assert np.all(x[:, 10:] == synth.PAD_BITS)
    assert np.array_equal(x[:, :10], synth.uniform(5, 10, 1))


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    v = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.f32_to_bf16_bits(v), ref)


def _decode(h):
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_distribution_moments():
    u = _decode(synth.uniform(256, 1024, 3))
    assert u.min() >= -1.0 and u.max() <= 1.0
    assert abs(u.mean()) < 0.01 and abs(u.var() - 1 / 3) < 0.01
    n = _decode(synth.normal(256, 1024, 4, sigma=0.02))
    assert abs(n.mean()) < 2e-4 and abs(n.std() - 0.02) < 2e-4
    i = _decode(synth.integers(256, 1024, 5))
    assert set(np.unique(i)) == set(range(-4, 5))


def test_workload_table_shapes():
    w = synth.WORKLOADS
    assert (w["square_4096"]["M"], w["square_4096"]["N"], w["square_4096"]["K"]) == (4096,) * 3
    assert w["gemv_m1"]["M"] == 1 and w["gemv_m16"]["M"] == 16
    assert w["batched_64x256x256x1024"]["batch"] == 64
    assert w["ffn_up_8192x14336x4096"]["out"] == synth.OUT_BF16
    A, B = synth.make_operands("single_tile_128")
    assert A.shape == (128, 128) and B.shape == (128, 128)
