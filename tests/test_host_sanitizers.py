"""Host-code sanitizers (CPU only): the oracle's C loops and the C ABI's host code built with
AddressSanitizer and UndefinedBehaviorSanitizer and driven through every entry point.

* The oracle (gcc): every function on tiny inputs in both dtypes, layouts, strides and
  epilogues, and its argument checks (tests/sanitize/oracle_driver.c).
* The C ABI (hipcc, sanitizers on the host pass; the device code is built but never run):
  argument validation, size queries, algorithm choice and the region helpers, with requests
  that never reach a device (tests/sanitize/abi_driver.cpp).

A sanitizer finding aborts the driver (no recovery), so the test fails on any of them.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "x3x3_convolution_amd", "csrc")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")


def _run(cmd, env=None):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=600)
    return r.returncode, r.stdout + r.stderr


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    rc, out = _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-o", exe,
                    os.path.join(ROOT, "oracle", "conv_oracle.c"),
                    os.path.join(HERE, "oracle_driver.c"), "-lm"])
    assert rc == 0, out
    rc, out = _run([exe], env=SAN_ENV)
    assert rc == 0 and "oracle driver ok" in out, out
    assert "AddressSanitizer" not in out and "runtime error" not in out, out


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    sources = ["api.hip", "simt2d.hip", "mfma2d.hip", "igemm3d.hip", "head.hip", "stencil.hip",
               "video.hip", "calib.hip"]
    # sanitizers on the host side only (the validation, planning and launch code); the device
    # code is built as usual, never run
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address",
             "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all",
             "-I" + os.path.join(ROOT, "include")]
    objs = [str(tmp_path / (src + ".o")) for src in sources]

    def compile_one(i):
        return _run(["hipcc"] + flags + ["-c", os.path.join(CSRC, sources[i]), "-o", objs[i]])
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        for rc, out in ex.map(compile_one, range(len(sources))):
            assert rc == 0, out[-4000:]
    drv = str(tmp_path / "abi_driver.o")
    rc, out = _run(["hipcc"] + flags + ["-c", os.path.join(HERE, "abi_driver.cpp"), "-o", drv])
    assert rc == 0, out
    exe = str(tmp_path / "abi_san")
    rc, out = _run(["hipcc", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                    "-fsanitize=undefined", drv] + objs + ["-o", exe])
    assert rc == 0, out[-4000:]
    env = dict(SAN_ENV, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")   # the HIP runtime's own
    rc, out = _run([exe], env=env)
    assert rc == 0 and "abi driver ok" in out, out
    assert "AddressSanitizer" not in out and "runtime error" not in out, out
