"""2D convolution over channels-last (NHWC) tensors on the matrix cores, through the C ABI,
against the oracle's channels-last definition: bit-exact on integer inputs, within tolerance on
random ones, and bit-identical to the NCHW path (the two layouts run the same contraction in the
same order)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from gpu_support import (DEV, alloc_guarded, assert_bit_exact, assert_within, bits, check_guards,
                         metrics, odt, sample_points_2d, EPI)
from x3x3_convolution_amd import conv as C
from x3x3_convolution_amd.plan import Conv3x3

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def nhwc(t):
    return t.permute(0, 2, 3, 1).contiguous()


def run_nhwc(x, w, b, H, W, stride, epilogue, algo=C.ALGO_AUTO):
    """x is NHWC; returns y NHWC, written inside NaN-filled guard bands."""
    N = x.shape[0]
    op = Conv3x3(w, b, N, H, W, stride=stride, epilogue=epilogue, algo=algo, channels_last=True)
    buf, y = alloc_guarded(op.out_shape(), x.dtype)
    op(x, y)
    torch.cuda.synchronize()
    check_guards(buf, y.numel())
    return y


def oracle_nhwc(x, w, b, stride, epilogue):
    return oracle.conv2d(bits(x), bits(w), bits(b), stride, odt(x.dtype), EPI[epilogue],
                         oracle.CHANNELS_LAST)


CASES = [
    # N, Ci, Co, H, W, stride, dtype, epilogue
    (1, 16, 16, 64, 64, 1, "f16", "relu"),
    (2, 8, 7, 13, 37, 1, "f16", "none"),        # ragged rows and columns, C_out % 4 != 0
    (2, 8, 7, 13, 37, 2, "f16", "clamp1"),
    (1, 64, 64, 19, 50, 1, "bf16", "relu"),
    (1, 40, 40, 20, 71, 2, "f16", "relu"),
    (3, 24, 64, 9, 16, 1, "bf16", "none"),
    (1, 64, 33, 33, 1, 2, "f16", "none"),       # W = 1
    (1, 8, 1, 1, 1, 1, "f16", "relu"),
    (2, 64, 64, 32, 64, 2, "f16", "relu"),
    (1, 64, 64, 70, 262, 1, "f16", "relu"),
    (5, 16, 16, 128, 256, 1, "f16", "relu"),    # 320 tiles: workgroups run two
    (9, 16, 24, 64, 250, 2, "bf16", "clamp1"),  # 288 tiles at stride 2
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_nhwc_integer_exact(case):
    N, Ci, Co, H, W, s, dt, epi = case
    _say("nhwc int %s" % (case,))
    x, w, b = si.integer_case("2d", N, Ci, Co, H, W, dtype=dt, seed=500 + CASES.index(case),
                              device=DEV)
    xl = nhwc(x)
    y = run_nhwc(xl, w, b, H, W, s, epi)
    assert_bit_exact(y, oracle_nhwc(xl, w, b, s, epi), x.dtype)


def test_nhwc_random_tolerance_and_same_bits_as_nchw():
    for s in (1, 2):
        x, w, b = si.random_case("2d", 2, 64, 64, 40, 72, dtype="f16", seed=10 + s, device=DEV)
        x = torch.relu(x)
        y = run_nhwc(nhwc(x), w, b, 40, 72, s, "relu")
        m = metrics(bits(y), oracle_nhwc(nhwc(x), w, b, s, "relu"), x.dtype)
        _say("nhwc random s=%d %s" % (s, m))
        assert_within(m, activated=True)
        op = Conv3x3(w, b, 2, 40, 72, stride=s, epilogue="relu", algo=C.ALGO_MFMA)
        y_nchw = op(x)
        torch.cuda.synchronize()
        assert torch.equal(nhwc(y_nchw).view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("name", ["c2", "c2s2"])
def test_nhwc_full_size_sampled(name):
    """The TAESD-style workloads with channels-last activations, sampled outputs."""
    wl = si.WORKLOADS[name]
    x, w, b = si.make_inputs(wl, device=DEV)
    xl = nhwc(x)
    del x
    y = run_nhwc(xl, w, b, wl.H, wl.W, wl.stride, wl.epilogue)
    pts = sample_points_2d(wl.N, wl.H_out, wl.W_out, 400, seed=2)
    ref = oracle.conv2d_points(bits(xl), bits(w), bits(b), pts, wl.stride, oracle.F16,
                               EPI[wl.epilogue], oracle.CHANNELS_LAST)
    idx = torch.from_numpy(pts.astype(np.int64)).to(y.device)
    got = bits(y[idx[:, 0], idx[:, 1], idx[:, 2], :])
    m = metrics(got, ref, wl.torch_dtype)
    _say("%s nhwc sampled %d %s" % (name, len(pts), m))
    assert_within(m, activated=True)
