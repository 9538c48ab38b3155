"""Host tools of the profiles: the per-kernel source hash that ties a committed counter
summary to the code it was measured on (no GPU)."""
import os

import tiled_matmul_amd as tm
from tiled_matmul_amd import proftools as pt


def test_every_planner_kernel_has_its_source():
    lib = tm.library()
    names = [lib.gemm_bf16_kernel_name(k).decode() for k in range(1, 20)] + ["splitk_reduce"]
    assert "?" not in names
    for n in names:
        assert n in pt.KERNEL_SOURCE, n
        assert os.path.exists(os.path.join(pt.CSRC, pt.KERNEL_SOURCE[n])), n
    for f in pt.SHARED_SOURCES:
        assert os.path.exists(os.path.join(pt.CSRC, f)), f


def test_hash_covers_exactly_the_kernel_sources(tmp_path, monkeypatch):
    src = tmp_path / "csrc"
    src.mkdir()
    for f in os.listdir(pt.CSRC):
        (src / f).write_bytes(open(os.path.join(pt.CSRC, f), "rb").read())
    monkeypatch.setattr(pt, "CSRC", str(src))
    ring, attn, gemv = (pt.kernel_source_sha(k) for k in ("ring4_256", "attn_mfma", "gemv_lds"))
    assert len({ring, attn, gemv}) == 3
    with open(src / "attention.hip", "a") as f:          # another kernel's file changes
        f.write("\n// edit\n")
    assert pt.kernel_source_sha("ring4_256") == ring
    assert pt.kernel_source_sha("attn_mfma") != attn
    with open(src / "gemm_bf16.hip", "a") as f:          # the host planner is not hashed
        f.write("\n// edit\n")
    assert pt.kernel_source_sha("ring4_256") == ring
    with open(src / "common.hpp", "a") as f:             # a shared header changes
        f.write("\n// edit\n")
    assert pt.kernel_source_sha("ring4_256") != ring
    assert pt.kernel_source_sha("gemv_lds") != gemv


def test_duration_quantiles():
    q = pt.duration_quantiles([1000 * i for i in range(1, 11)])   # 1 .. 10 us
    assert q == {"avg": 5.5, "median": 5.5, "min": 1.0, "p90": 9.0, "max": 10.0}
    assert pt.duration_quantiles([7000])["p90"] == 7.0
