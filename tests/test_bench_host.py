"""The benchmark's host-side arithmetic and contract, on the CPU: the refusal of more
than one GPU, the roofline row of one direction, the HBM traffic read back from the
committed counter summary, the kernel-source hash the summary is tied to, and the CPU
baseline's rate."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_device_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_direction_roofline_counts_each_payload_byte_read_once_and_written_once():
    payload = 4 << 30
    each_ms = [1.0, 2.0, 3.0, 4.0]          # mean 2.5 ms, median 2.5 ms
    row = bench.direction_roofline(payload, each_ms)
    assert row["launches"] == 4
    assert row["kernel_ms"] == 2.5 and row["kernel_ms_min"] == 1.0 and row["kernel_ms_max"] == 4.0
    achieved = 2 * payload / 2.5e-3 / 1e9
    assert row["achieved"] == round(achieved, 1)
    assert row["gbs"] == round(payload / 2.5e-3 / 1e9, 1)
    assert row["hbm_frac"] == round(achieved / bench.HBM_PEAK_GBS, 4)
    assert row["hbm_frac_of_median"] == row["hbm_frac"]


def test_traffic_is_the_scaled_counters_of_the_committed_summary_or_nothing():
    t = json.load(open(bench.TRAFFIC_FILE))
    size = t["algorithmic_bytes_per_launch"]
    if t["kernel_source_sha256"] != bench.kernel_source_hash():
        # counters taken on another kernel are never attached
        assert bench.traffic_for("scatter", size) is None
        return
    cal = t["calibration"]
    for d in ("gather", "scatter"):
        want = (t[d]["fetch_kib"] * cal["fetch_scale"] + t[d]["write_kib"] * cal["write_scale"]) * 1024
        got = bench.traffic_for(d, size)
        assert abs(got - want) <= 1
        # every byte once each way: within 0.1 % of the algorithmic bytes
        assert abs(got / size - 1) < 1e-3
    assert bench.traffic_for("scatter", size + 16) is None
    assert bench.traffic_for("sideways", size) is None


def test_kernel_source_hash_ignores_comments_and_layout_but_not_code(tmp_path, monkeypatch):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.h"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", ["a.hip", "b.h"])
    a.write_text("int f(int x) { return x + 1; } // one\n")
    b.write_text("#define N 4\n")
    h0 = bench.kernel_source_hash()
    a.write_text("/* new comment */\nint f(int x)\n{\n    return x + 1;   // two\n}\n")
    assert bench.kernel_source_hash() == h0
    a.write_text("int f(int x) { return x + 2; }\n")
    assert bench.kernel_source_hash() != h0


def test_cpu_baseline_rate_is_bytes_moved_over_oracle_time():
    res = dict(name="llama8b", pool=dict(num_layers=32),
               cpu=dict(gather_s=0.5, scatter_s=1.5, moved=8 << 30, threads=16,
                        single=dict(bytes=1 << 30, s=2.0, sample="gather of 4/32 layers")))
    out = bench.cpu_baseline(res)
    assert out["value"] == round((8 << 30) / 2.0 / 1e9, 4)
    assert out["cores"] == 16 and out["kind"] == "oracle" and out["unit"] == "GB/s"
    assert out["single_core"]["cores"] == 1
    assert out["single_core"]["value"] == round((1 << 30) / 2.0 / 1e9, 4)
    assert "nproc" in out and "cpu_model" in out
    assert bench.cpu_baseline(dict(cpu=None)) is None


@pytest.mark.parametrize("flag", ["--no-small-calls", "--no-placement", "--no-host-path", "--no-duplex"])
def test_bench_flags_parse(flag):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "3", flag],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
