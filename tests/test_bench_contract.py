"""bench.py's host-side contract, on the CPU: one GPU only, and stored HBM
traffic is reported only while the kernel sources still match the hash it was
taken with."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_flop_counting():
    import attn_inputs as ai
    w = ai.WORKLOADS["c5"]
    f_fwd, f_bwd = bench.flops(w, True)
    assert f_fwd == 0.5 * 4 * 4 * 64 * 4096 * 4096 * 128
    assert f_bwd == 2.5 * f_fwd


def test_stored_traffic_follows_source_hash(tmp_path, monkeypatch):
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.stored_traffic("fa_fwd") is None  # no file
    path.write_text(json.dumps({"source_sha256": bench.kernel_source_hash(),
                                "bytes_per_launch": {"fa_fwd": 123}}))
    assert bench.stored_traffic("fa_fwd") == 123
    path.write_text(json.dumps({"source_sha256": "0" * 64, "bytes_per_launch": {"fa_fwd": 123}}))
    assert bench.stored_traffic("fa_fwd") is None  # kernels changed since


def test_time_stats():
    st = bench.time_stats([4.0, 1.0, 3.0, 2.0, 10.0])
    assert st == {"median": 3.0, "min": 1.0, "p90": 7.6}


def test_dpm_levels_and_peak_formula():
    assert bench.parse_dpm_levels("0: 500Mhz \n1: 1600Mhz *\n2: 2400Mhz\n") == [500, 1600, 2400]
    assert bench.parse_dpm_levels("no clocks here") == []
    # 256 CUs x 4096 FLOP per clock at 2.4 GHz: the 2.517 PFLOP/s behind the published 2.5
    assert abs(256 * 4096 * 2400e6 / 1e12 - 2516.6) < 0.1
