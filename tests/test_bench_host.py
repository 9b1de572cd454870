"""Host logic of bench.py that needs no GPU: the one-GPU guard, the default
run, and the rule that the HBM traffic figure is reported only while the
decode sources match the ones the counters were taken on."""
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
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout.strip()


def test_defaults_are_one_gpu_and_a_short_run(monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    a = bench.parse()
    assert a.gpus == 1 and a.steps > 0 and a.warmup > 0
    assert not (a.no_gemm or a.no_extras or a.no_cpu_baseline or a.traffic or a.mfma_counters)


def test_traffic_reported_only_for_matching_sources(tmp_path, monkeypatch):
    rec = json.load(open(bench.TRAFFIC_FILE))
    got = bench.measured_traffic()
    assert got == rec["traffic_bytes_per_launch"], "committed sources and counters disagree"
    # a decode source that differs from the one the counters were taken on
    src = tmp_path / "gemv_i2s.hip"
    src.write_bytes(open(os.path.join(ROOT, bench.DECODE_SOURCES[0]), "rb").read() + b"\n// edit\n")
    monkeypatch.setattr(bench, "DECODE_SOURCES", (str(src),) + tuple(bench.DECODE_SOURCES[1:]))
    assert bench.measured_traffic() is None
    # a missing or unreadable record
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic() is None
