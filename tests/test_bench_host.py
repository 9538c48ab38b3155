"""Host-side pieces of bench.py (no GPU): the engine-clock sampler reads the level the driver
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
    assert r["median"] == 1897 and r["min"] == 1897 and r["max"] == 1897 and r["samples"] >= 1
    assert s.summary(wall_s=0.45)["median"] == 1897
    assert s.summary(wall_s=0.1) is None          # too short for the driver's reading


def test_sclk_sampler_without_sysfs():
    s = bench.SclkSampler()
    s.path = None
    with s:
        pass
    assert s.summary() is None
