"""Builds the gfx950 HIP library libconv3x3.so in-tree with hipcc.

Every source under csrc/ is compiled for gfx950 only, with packed-fp32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops), then linked into one shared library next to
this file.  Object files go to _build/ at the repository root.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libconv3x3.so")
SOURCES = ["api.hip", "simt2d.hip", "mfma2d.hip", "igemm3d.hip", "head.hip", "stencil.hip",
           "video.hip", "calib.hip"]
ARCH = "gfx950"
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]


def _compile(src: str, obj: str, extra) -> None:
    cmd = ["hipcc"] + FLAGS + list(extra) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; anything else is shown
    noise = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, msg))
    if msg.strip():
        sys.stderr.write(msg + "\n")


def build(extra_flags=(), jobs: int = 4) -> str:
    """Compile every HIP source for gfx950 and link libconv3x3.so.  Always recompiles."""
    bdir = os.path.join(ROOT, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = [os.path.join(bdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda so: _compile(so[0], so[1], extra_flags), zip(SOURCES, objs)))
    tmp = LIB + ".tmp%d" % os.getpid()
    # (--no-undefined: a kernel whose host stub was not emitted fails here, not at load time)
    cmd = ["hipcc", "--offload-arch=" + ARCH, "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
