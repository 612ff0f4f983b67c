"""bench.py's command line on the CPU: it measures one GPU only and says so for more, and its
help text lists the workloads (no GPU needed for either)."""
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
