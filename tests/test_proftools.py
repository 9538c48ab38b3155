"""Host tools of the profiles: the per-kernel source hash that ties a committed counter
summary to the code it was measured on (no GPU)."""
import os
import sys

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


def _csv(path, header, rows):
    with open(path, "w") as f:
        f.write(",".join(header) + "\n")
        for r in rows:
            f.write(",".join(str(x) for x in r) + "\n")


def test_mfma_summary_arithmetic(tmp_path):
    """Two dispatches of a kernel, 100 us each: GRBM_GUI_ACTIVE summed over the 8 XCDs gives
    the clock, the MFMA-busy cycles over all 1024 SIMDs the utilisation, 512 flops per
    counted op the rate."""
    ns = 100_000
    cyc = 200_000   # per XCD -> 2.0 GHz
    ops = 2 * 4096 ** 3 // 512
    cnt = [("GRBM_GUI_ACTIVE", 8 * cyc), ("SQ_VALU_MFMA_BUSY_CYCLES", cyc * 1024 // 2),
           ("SQ_INSTS_VALU_MFMA_MOPS_BF16", ops), ("SQ_LDS_IDX_ACTIVE", cyc * 256 // 4),
           ("SQ_LDS_BANK_CONFLICT", 0)]
    _csv(tmp_path / "c.csv", ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"],
         [(d, "gemm_ring_kernel<x>", n, v) for d in (1, 2) for n, v in cnt] + [(3, "other", "GRBM_GUI_ACTIVE", 1)])
    _csv(tmp_path / "t.csv", ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"],
         [(1, "gemm_ring_kernel<x>", 0, ns), (2, "gemm_ring_kernel<x>", 10 * ns, 11 * ns), (3, "other", 0, 5)])
    r = pt.mfma_summary(str(tmp_path / "c.csv"), str(tmp_path / "t.csv"), "gemm_ring")
    assert r["dispatches"] == 2
    assert abs(r["ghz"] - 2.0) < 1e-12 and abs(r["mfma_util"] - 0.5) < 1e-12 and abs(r["lds_util"] - 0.25) < 1e-12
    assert r["flops"] == 2 * 4096 ** 3
    assert abs(r["tflops"] - 2 * 4096 ** 3 / ns / 1e3) < 1e-9
    assert abs(r["frac_peak_at_clock"] - r["tflops"] / (2500.0 * 2.0 / 2.4)) < 1e-12


def test_traffic_scaling_by_copy_calibration(tmp_path, monkeypatch):
    """The counters of a kernel scaled by what the same counters read for a copy of known size."""
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    _csv(tmp_path / "f.csv", hdr, [(1, "k_a", "FETCH_SIZE", 100.0), (2, "k_a", "FETCH_SIZE", 300.0)])
    _csv(tmp_path / "w.csv", hdr, [(1, "k_a", "WRITE_SIZE", 50.0)])
    _csv(tmp_path / "cf.csv", hdr, [(1, "copyBuffer", "FETCH_SIZE", 512.0)])   # half of 1 MiB
    _csv(tmp_path / "cw.csv", hdr, [(1, "copyBuffer", "WRITE_SIZE", 1024.0)])
    out = tmp_path / "o.json"
    monkeypatch.setattr(sys, "argv", ["x", "traffic", "--fetch", str(tmp_path / "f.csv"), "--write", str(tmp_path / "w.csv"),
                                      "--copy-fetch", str(tmp_path / "cf.csv"), "--copy-write", str(tmp_path / "cw.csv"),
                                      "--copy-kernel", "copyBuffer", "--copy-bytes", str(2 ** 20), "--kernel", "k_a",
                                      "--plan-kernel", "ring4_256", "--workload", "w", "--grid", "256", "--block", "256",
                                      "--out", str(out)])
    pt.main()
    import json
    d = json.load(open(out))
    assert d["hbm_read_bytes_per_launch"] == 200.0 * 1024 * 2     # mean 200 KiB, scaled x2
    assert d["hbm_write_bytes_per_launch"] == 50.0 * 1024
    assert (d["grid"], d["block"]) == (256, 256)
    assert d["kernel_source_sha"] == pt.kernel_source_sha("ring4_256")


def test_durations_grouped_by_launch_shape(tmp_path):
    f = tmp_path / "k.csv"
    hdr = "Kernel_Name,Start_Timestamp,End_Timestamp,Workgroup_Size_X,Grid_Size_X\n"
    rows = ["k,300,1300,256,65536", "k,0,2000,256,65536", "k,100,600,1024,262144", "j,5,10,64,64"]
    f.write_text(hdr + "\n".join(rows) + "\n")
    d = pt.kernel_durations_by_launch(str(f))
    # grid sizes count threads: 65536 / 256 = 256 workgroups; launch order by start time
    assert d == {("k", 256, 256): [2000, 1000], ("k", 256, 1024): [500], ("j", 1, 64): [5]}
