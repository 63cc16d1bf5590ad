"""Host-side logic of bench.py: the one-GPU guard and the HBM-counter bookkeeping."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"] and msg["n_gpus"] == 2


def test_counter_entries_cover_known_kernels():
    for name, c in bench.HBM_COUNTERS.items():
        assert name in bench.KERNEL_SOURCES
        assert set(c) == {"digest", "fetch_kib", "write_kib", "fetch_factor", "write_factor"}
        assert c["fetch_factor"] > 0 and c["write_factor"] > 0


def test_traffic_scales_by_calibration_and_goes_stale(monkeypatch):
    name = "mfma_split_kv"
    fresh = {"digest": bench.source_digest(name), "fetch_kib": 1000.0, "write_kib": 10.0,
             "fetch_factor": 0.5, "write_factor": 1.0}
    monkeypatch.setitem(bench.HBM_COUNTERS, name, fresh)
    assert bench.hbm_traffic(name) == pytest.approx(1000.0 * 1024 / 0.5 + 10.0 * 1024)
    stale = dict(fresh, digest="0" * 16)
    monkeypatch.setitem(bench.HBM_COUNTERS, name, stale)
    assert bench.hbm_traffic(name) is None
    assert bench.hbm_traffic("not_a_kernel") is None


def test_source_digest_depends_on_every_listed_file(tmp_path, monkeypatch):
    for f in ("a.hip", "common.h"):
        (tmp_path / f).write_text(f)
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    monkeypatch.setitem(bench.KERNEL_SOURCES, "k", ["a.hip", "common.h"])
    d0 = bench.source_digest("k")
    (tmp_path / "common.h").write_text("changed")
    assert bench.source_digest("k") != d0


def test_host_info_and_pool_size(monkeypatch):
    info = bench.host_info()
    assert info["cpus_visible"] == len(os.sched_getaffinity(0)) >= 1
    monkeypatch.setenv("OMP_NUM_THREADS", "3")
    assert bench.pool_size() == min(3, info["cpus_visible"])
    monkeypatch.delenv("OMP_NUM_THREADS")
    assert 1 <= bench.pool_size() <= 16


def test_clock_summary_uses_the_settled_half():
    """The clock probe keeps the second half of its samples (the first half is
    the ramp and the power sensor's trailing average) and reads the power cap
    in watts whether amdsmi reports watts or microwatts."""
    b = bench
    clk = [2400.0] * 50 + [1800.0] * 49 + [1900.0]
    r = b.summarise_clock(clk, [300.0] * 50 + [1390.0] * 50, [1.4e9] * 100)
    assert r["sclk_mhz_median"] == 1800.0 and r["sclk_mhz_max"] == 1900.0 and r["samples"] == 50
    assert r["socket_power_w_median"] == 1390.0 and r["power_limit_w"] == 1400.0
    assert b.summarise_clock([2000.0, 2000.0], [], [1400.0])["power_limit_w"] == 1400.0
    assert "error" in b.summarise_clock([], [], [])
