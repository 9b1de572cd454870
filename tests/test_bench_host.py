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
    import hashlib
    h = hashlib.sha256()
    for rel in bench.DECODE_SOURCES:
        h.update(open(os.path.join(ROOT, rel), "rb").read())
    rec = tmp_path / "traffic.json"
    rec.write_text(json.dumps({"source_sha256": h.hexdigest(), "traffic_bytes_per_launch": 12345}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    assert bench.measured_traffic() == 12345
    # a decode source that differs from the one the counters were taken on
    src = tmp_path / "gemv_i2s.hip"
    src.write_bytes(open(os.path.join(ROOT, bench.DECODE_SOURCES[0]), "rb").read() + b"\n// edit\n")
    monkeypatch.setattr(bench, "DECODE_SOURCES", (str(src),) + tuple(bench.DECODE_SOURCES[1:]))
    assert bench.measured_traffic() is None
    # a missing or unreadable record
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic() is None


def test_step_count_is_exact():
    """The timed graph holds exactly --steps steps, continuing the copy
    rotation after the warmup steps (checked with a stand-in for torch that
    records the captured launches)."""
    calls = []

    class FakeEvent:
        def __init__(self, **kw):
            pass

        def record(self, stream=None):
            pass

        def elapsed_time(self, other):
            return 1.0

    class FakeGraph:
        def __init__(self):
            self.fns = []

        def replay(self):
            calls.append(tuple(self.fns))

    class Ctx:
        def __init__(self, g=None):
            self.g = g

        def __enter__(self):
            FakeTorch._capturing = self.g

        def __exit__(self, *a):
            FakeTorch._capturing = None

    class FakeCuda:
        Event = FakeEvent
        CUDAGraph = FakeGraph

        @staticmethod
        def graph(g, stream=None):
            return Ctx(g)

        @staticmethod
        def stream(s):
            return Ctx()

        @staticmethod
        def synchronize():
            pass

    class FakeTorch:
        cuda = FakeCuda
        _capturing = None

    R = 32
    layers = [[(lambda r=r, j=j: FakeTorch._capturing.fns.append((r, j))) for j in range(4)]
              for r in range(R)]
    ms, spread, piped = bench.time_steps(FakeTorch, None, layers, steps=20, warmup=5,
                                         spread_reps=2)
    warm = tuple((i % R, j) for i in range(5) for j in range(4))
    timed = tuple((i % R, j) for i in range(5, 25) for j in range(4))
    # one untimed launch of the timed graph, then (warmup graph, timed graph)
    # for the timed step and each spread repetition, then back-to-back replays
    assert calls[0] == timed and len(calls) == 1 + 2 * (1 + 2) + 2
    assert calls[1:7] == [warm, timed] * 3 and calls[7:] == [timed, timed]
    assert ms == 1.0 / 20 and len(spread) == 3 and piped == round(1e3 / 20, 3)
