"""Every output of every workload at full size, against the oracle.

The tolerance tests elsewhere check the full-size workloads at sampled positions; here the oracle
evaluates every output element on the host cores, from the exact bits the GPU read, and the
comparison runs over all of them: d = y_gpu - y_oracle over the whole tensor, saturated and zero
outputs included.  The bounds (the workload text's): max|d| <= 1.6e-2 and rms(d) <= 2e-3 for
clamped or activated outputs, rel-rms = rms(d) / rms(y_oracle) <= 4e-3 for unclamped ones.  All
three numbers are computed for every case; when CONV_PARITY_OUT names a file, each case appends
its record to it as one JSON line.

Each GPU output is written into a NaN-filled buffer with guard bands, so an output the kernel
never wrote, or a write outside the tensor, fails the test.
"""
import json
import os
import sys
import time

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from gpu_support import (DEV, EPI, TOL_ACT, TOL_LINEAR, alloc_guarded, assert_within, bits,
                         check_guards, metrics, odt)
from x3x3_convolution_amd import conv as C
from x3x3_convolution_amd.plan import Conv3x3, Conv3x3x3

pytestmark = pytest.mark.gpu

ALGO_NAME = {C.ALGO_SIMT: "simt", C.ALGO_MFMA: "mfma", C.ALGO_SPLIT_HEAD: "split",
             C.ALGO_FUSED_HEAD: "fused"}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _record(name, algo, layout, m, n_out, oracle_s):
    activated = si.WORKLOADS[name].epilogue != "none"
    rec = dict(workload=name, algo=ALGO_NAME[algo], layout=layout, outputs=int(n_out),
               max_abs=m["max_abs"], rms=m["rms"], rel_rms=m["rel_rms"],
               bound=dict(TOL_ACT) if activated else dict(TOL_LINEAR),
               oracle_s=round(oracle_s, 2))
    _say("full %s" % json.dumps(rec))
    path = os.environ.get("CONV_PARITY_OUT")
    if path:
        with open(path, "a") as fh:
            fh.write(json.dumps(rec) + "\n")
    assert_within(m, activated=activated)


class _Ref:
    """The inputs of one workload on the GPU and the oracle's output over all of it."""

    def __init__(self, name, layout=oracle.CHANNELS_FIRST):
        wl = si.WORKLOADS[name]
        self.wl = wl
        self.x, self.w, self.b = si.make_inputs(wl, device=DEV)
        stride = wl.stride
        t0 = time.perf_counter()
        if wl.kind == "2d":
            self.y = oracle.conv2d(bits(self.x), bits(self.w), bits(self.b), stride,
                                   odt(self.x.dtype), EPI[wl.epilogue], oracle.CHANNELS_FIRST)
        else:
            self.y = oracle.conv3d(bits(self.x), bits(self.w), bits(self.b), 1, odt(self.x.dtype),
                                   EPI[wl.epilogue], oracle.CHANNELS_LAST)
        self.oracle_s = time.perf_counter() - t0
        _say("oracle over all of %s: %d outputs in %.1f s" % (name, self.y.size, self.oracle_s))


_cache = {}


def _ref(name):
    """One oracle pass per workload per session (the head's is shared by its three algorithms);
    the previous workload's tensors are dropped first."""
    if name not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        _cache[name] = _Ref(name)
    return _cache[name]


@pytest.mark.parametrize("name,algo", [(n, a) for n in ("c1", "c2", "c2s2")
                                       for a in (C.ALGO_SIMT, C.ALGO_MFMA)])
def test_2d_every_output(name, algo):
    r = _ref(name)
    wl = r.wl
    _say("2d every output: %s algo %s" % (name, ALGO_NAME[algo]))
    op = Conv3x3(r.w, r.b, wl.N, wl.H, wl.W, stride=wl.stride, epilogue=wl.epilogue, algo=algo)
    buf, y = alloc_guarded(op.out_shape(), r.x.dtype)
    op(r.x, y)
    torch.cuda.synchronize()
    check_guards(buf, y.numel())
    m = metrics(bits(y), r.y, r.x.dtype)
    _record(name, algo, "NCHW", m, y.numel(), r.oracle_s)


@pytest.mark.parametrize("name", ["c2", "c2s2"])
def test_2d_nhwc_every_output(name):
    """The same workloads through the channels-last (NHWC) matrix-core kernel."""
    r = _ref(name)
    wl = r.wl
    _say("2d NHWC every output: %s" % name)
    xl = r.x.permute(0, 2, 3, 1).contiguous()
    op = Conv3x3(r.w, r.b, wl.N, wl.H, wl.W, stride=wl.stride, epilogue=wl.epilogue,
                 channels_last=True)
    buf, y = alloc_guarded(op.out_shape(), r.x.dtype)
    op(xl, y)
    torch.cuda.synchronize()
    check_guards(buf, y.numel())
    m = metrics(bits(y), np.ascontiguousarray(r.y.transpose(0, 2, 3, 1)), r.x.dtype)
    _record(name, C.ALGO_MFMA, "NHWC", m, y.numel(), r.oracle_s)


CASES_3D = [("c3", C.ALGO_MFMA), ("c3", C.ALGO_SPLIT_HEAD), ("c3", C.ALGO_FUSED_HEAD),
            ("c4", C.ALGO_MFMA), ("c5", C.ALGO_MFMA), ("c5d1", C.ALGO_MFMA)]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,algo", CASES_3D, ids=["%s-%s" % (n, ALGO_NAME[a]) for n, a in CASES_3D])
def test_3d_every_output(name, algo):
    r = _ref(name)
    wl = r.wl
    _say("3d every output: %s algo %s" % (name, ALGO_NAME[algo]))
    op = Conv3x3x3(r.w, r.b, wl.N, wl.D, wl.H, wl.W, epilogue=wl.epilogue, algo=algo)
    assert op.algo == algo
    buf, y = alloc_guarded(op.out_shape(), r.x.dtype)
    op(r.x, y)
    torch.cuda.synchronize()
    check_guards(buf, y.numel())
    del op
    m = metrics(bits(y), r.y, r.x.dtype)
    _record(name, algo, "NDHWC", m, y.numel(), r.oracle_s)
