"""bench.py's command line on the CPU: it measures one GPU only and says so for more, its
help text lists the workloads, and its warm-up loop keeps going until the clock has had time to
settle (no GPU needed for any of these)."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_help_lists_the_workloads_and_options():
    r = _run("--help")
    assert r.returncode == 0
    for word in ("c3", "c4", "c5", "c5d1", "c1", "c2", "c2s2", "--region", "--flush",
                 "--channels-last", "--stride3d", "--copy-calibration"):
        assert word in r.stdout, word


def test_warm_up_runs_at_least_the_steps_and_the_settle_time(monkeypatch):
    # the warm-up loop with the device synchronisation stubbed out (no GPU here): at least
    # --warmup steps, in doubling batches until --settle-ms of wall time has passed
    import time
    import types

    import torch
    sys.path.insert(0, ROOT)
    import bench
    monkeypatch.setattr(torch.cuda, "synchronize", lambda *a, **k: None)
    calls = []

    def step():
        calls.append(time.perf_counter())

    assert bench.warm_up(step, types.SimpleNamespace(warmup=0, settle_ms=0.0)) == 0
    assert bench.warm_up(step, types.SimpleNamespace(warmup=5, settle_ms=0.0)) == 5
    assert len(calls) == 5
    calls.clear()

    def slow_step():
        time.sleep(0.001)
        step()

    n = bench.warm_up(slow_step, types.SimpleNamespace(warmup=3, settle_ms=20.0))
    assert n == len(calls) and n in (3, 9, 21, 45)     # 3, then batches of 6, 12, 24
    assert calls[-1] - calls[0] >= 0.018
    assert "--settle-ms" in _run("--help").stdout
