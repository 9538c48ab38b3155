"""Host-side pieces of bench.py (no GPU): the engine-clock sampler reads the level the amdgpu driver
marks current in pp_dpm_sclk."""
import os
import sys
import time

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def test_sclk_sampler_reads_the_current_level(tmp_path):
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("0: 500Mhz \n1: 1897Mhz *\n2: 2400Mhz \n")
    s = bench.SclkSampler()
    s.path = str(f)
    with s:
        time.sleep(0.05)
    r = s.summary()
    assert r["median"] == 1897 and r["min"] == 1897 and r["max"] == 1897 and r["samples"] >= 2
    assert r["start"] == 1897 and r["end"] == 1897
    # a timed region of a few milliseconds still reports (its start and end readings)
    s2 = bench.SclkSampler()
    s2.path = str(f)
    with s2:
        pass
    r2 = s2.summary(wall_s=0.002)
    assert r2["median"] == 1897 and r2["samples"] >= 2 and r2["timed_region_s"] == 0.002


def test_trace_taken_only_on_the_same_sources_and_launch(tmp_path, monkeypatch):
    import json
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    sha = bench.kernel_source_sha("ring4_256")
    d = {"kernel_source_sha": sha, "grid": 256, "block": 256, "avg_us": 100.0, "median_us": 99.0,
         "dispatches": 20, "command": "x"}
    json.dump(d, open(tmp_path / "profiles" / "trace_ring4_256_w1.json", "w"))
    t = bench.trace_for("ring4_256", "w1", 256, 256)
    r = bench.traced_rate(t, 2.0e14 * 1e-4, 2500.0, 1e12)       # 2e14 FLOP/s over 100 us
    assert abs(r["achieved_avg"] - 200.0) < 1e-9 and abs(r["frac_avg"] - 0.08) < 1e-12
    assert abs(r["achieved_median"] - 200.0 * 100 / 99) < 1e-9
    assert bench.trace_for("ring4_256", "w1", 240, 256) is None          # another launch
    assert bench.trace_for("ring4_256", "w2", 256, 256) is None          # no summary
    d["kernel_source_sha"] = "0" * 16
    json.dump(d, open(tmp_path / "profiles" / "trace_ring4_256_w3.json", "w"))
    assert bench.trace_for("ring4_256", "w3", 256, 256) is None          # other sources
    assert bench.traced_rate(None, 1.0, 1.0, 1.0) is None


def test_sclk_sampler_without_sysfs():
    s = bench.SclkSampler()
    s.path = None
    with s:
        pass
    assert s.summary() is None


def test_traffic_taken_only_on_the_same_sources_and_launch(tmp_path, monkeypatch):
    import json
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    sha = bench.kernel_source_sha("ring4_256")
    def put(kernel, wl, **kw):
        d = {"kernel_source_sha": sha if kernel != "splitk_reduce" else bench.kernel_source_sha(kernel),
             "hbm_bytes_per_launch": 100.0}
        d.update(kw)
        json.dump(d, open(tmp_path / "profiles" / f"traffic_{kernel}_{wl}.json", "w"))
    put("ring4_256", "w1", grid=256, block=256)
    assert bench.traffic_for("ring4_256", "w1", 256, 256) == 100.0
    assert bench.traffic_for("ring4_256", "w1", 240, 256) is None          # another launch
    assert bench.traffic_for("ring4_256", "w2", 256, 256) is None          # no summary
    put("ring4_256", "w3", grid=256, block=256, kernel_source_sha="0" * 16)
    assert bench.traffic_for("ring4_256", "w3", 256, 256) is None          # other sources
    put("ring4_256", "w4", grid=256, block=256)
    put("splitk_reduce", "w4")
    assert bench.traffic_for("ring4_256+splitk_reduce", "w4", 256, 256) == 200.0   # a two-kernel call


def test_rate_at_the_reported_clock_only_over_long_regions():
    res = {"flops": 2.0 * 4096 ** 3, "bytes": 134217728, "tflops": 1250.0, "ms": 0.11,
           "kernel": "ring4_256", "name": "no_such_workload", "grid": 256, "block": 256}
    sclk = {"median": 1875, "timed_region_s": 0.5}
    r = bench.gemm_roofline(dict(res, sclk=sclk))
    assert abs(r["frac_at_sclk"] - 1250.0 / (2500.0 * 1875 / 2400.0)) < 1e-12
    # a region of a few milliseconds: the reading is the idle level, no scaled rate
    r = bench.gemm_roofline(dict(res, sclk=dict(sclk, median=462, timed_region_s=0.0022)))
    assert r["frac_at_sclk"] is None
    assert "frac_at_sclk" not in bench.gemm_roofline(dict(res, sclk=None))
