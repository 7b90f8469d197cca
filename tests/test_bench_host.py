"""bench.py's host side (no GPU): the one-GPU rule, the algorithmic
accounting the roofline credits, and when measured traffic may be reported
(only for the kernel sources and configuration the counters were taken on)."""
import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_without_running():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 4096), (256, 8192, 28672), (1, 8192, 8192)])
def test_algorithmic_work(M, N, K):
    assert bench.gemm_flops(M, N, K) == 2 * M * N * K
    assert bench.gemm_bytes(M, N, K) == 2 * (M * K + N * K + M * N)
    assert bench.gemm_bytes(M, N, K, out_bytes=4) == 2 * (M * K + N * K) + 4 * M * N
    assert bench.RIDGE == pytest.approx(312.5)


def _write_traffic(root, rec):
    os.makedirs(os.path.join(root, "profiles"), exist_ok=True)
    with open(os.path.join(root, "profiles", "traffic.json"), "w") as f:
        json.dump(rec, f)


def test_measured_traffic_only_for_matching_sources_and_config(tmp_path, monkeypatch):
    src = tmp_path / "dense_gemm_bf16_amd" / "csrc"
    src.mkdir(parents=True)
    (src / "k.hip").write_text("kernel v1\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h = bench.kernel_source_hash()
    expect = hashlib.sha256(b"k.hip" + b"kernel v1\n").hexdigest()[:16]
    assert h == expect
    rec = {"w": {"kernel_src_hash": h, "config": "cfg_a", "l2_fabric_bytes_per_launch": 1234}}
    _write_traffic(str(tmp_path), rec)
    assert bench.measured_traffic("w", "cfg_a") == 1234
    assert bench.measured_traffic("w", "cfg_b") is None        # another plan
    assert bench.measured_traffic("other", "cfg_a") is None    # another workload
    (src / "k.hip").write_text("kernel v2\n")                  # the kernel changed
    assert bench.measured_traffic("w", "cfg_a") is None
    (src / "k.hip").write_text("kernel v1\n")
    (src / "sub").mkdir()                                      # files in subfolders count
    (src / "sub" / "a.hpp").write_text("x\n")
    assert bench.kernel_source_hash() != h


def test_cpu_model_reads_the_host():
    info = bench.cpu_model()
    assert info["logical_cpus"] == os.cpu_count()
    assert info["model"] is None or isinstance(info["model"], str)


def test_clock_summary():
    s = [{"gfx": [1800, 1900], "mem": 1300}, None, {"gfx": [2000], "mem": 1300}]
    c = bench.summarize_clocks(s)
    assert c["sclk_mhz_median"] == 1900 and c["sclk_mhz_min"] == 1800
    assert c["sclk_mhz_max"] == 2000 and c["mclk_mhz_median"] == 1300
    assert bench.summarize_clocks([None]) is None


def test_committed_traffic_record_adds_up():
    """The committed record's bytes are its counters times the copy
    calibration factors, as the counters summary states."""
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        table = json.load(f)
    for name, rec in table.items():
        want = (rec["fetch_kib_per_launch"] * 1024 * rec["copy_fetch_factor"]
                + rec["write_kib_per_launch"] * 1024 * rec["copy_write_factor"])
        assert rec["l2_fabric_bytes_per_launch"] == pytest.approx(want, rel=2e-4), name
        assert os.path.exists(os.path.join(ROOT, rec["source"])), name
