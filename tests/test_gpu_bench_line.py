"""bench.py's JSON line on the GPU: one short run of the default workload (the head pass, with
its oracle pass on the host) and one of a small 2D workload, checked for the fields the line
promises -- metric, value and unit, the step counts, the dominant kernel's roofline, the oracle
baseline and the parity of every output against it."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _line(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


def _common(d, steps, warmup):
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == steps and d["warmup"] == warmup
    assert d["value"] > 0 and d["ms_per_step"] == d["value"] and d["higher_is_better"] is False
    r = d["roofline"]
    assert r["bound"] in ("hbm", "mfma", "alu") and r["unit"] in ("GB/s", "TFLOP/s")
    assert r["peak"] > 0 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert "workload" in d["config"]


def test_default_line_head_pass():
    d = _line("--no-workloads", "--steps", "3", "--warmup", "1", "--settle-ms", "0")
    _common(d, 3, 1)
    assert d["config"]["algo"] == "fused" and d["dtype"] == "bf16"
    assert d["roofline"]["bound"] == "hbm" and d["roofline"]["unit"] == "GB/s"
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    p = d["parity"]
    assert p["ok"] is True and p["positions"] == 16 * 352 * 624


def test_small_2d_workload_line():
    d = _line("--workload", "c1", "--no-cpu-baseline", "--steps", "3", "--warmup", "1",
              "--settle-ms", "0")
    _common(d, 3, 1)
    assert d["config"]["workload"] == "c1" and d["roofline"]["kernel"] == "mfma2d"
