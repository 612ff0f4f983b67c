"""The library's calls inside a captured HIP graph: they enqueue kernels only (no allocation, no
synchronisation, no memset), so a decoder can capture a sequence of convolutions once and replay
it.  A graph of a 2D conv, a 3D conv that splits K (workspace partials + reduce), one that splits
K over the waves of a workgroup, one on the stream-K schedule (its arrival counters cleared by a
kernel of the call, so every replay starts from zero), the fused head and the video step is
replayed several times, with new inputs copied in and eager work in between, and every replay
must equal the eager calls on the same inputs bit for bit."""
from __future__ import annotations

import sys

import pytest
import torch

import synthetic_inputs as si
from gpu_support import DEV
from x3x3_convolution_amd import conv as C
from x3x3_convolution_amd.plan import Conv3x3, Conv3x3x3

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bits(t):
    return t.view(torch.int16) if t.dtype != torch.uint8 else t


def test_graph_replays_equal_eager_calls():
    torch.manual_seed(0)
    x2, w2, b2 = si.random_case("2d", 2, 64, 64, 40, 72, dtype="f16", seed=21, device=DEV)
    x3, w3, b3 = si.random_case("3d", 1, 512, 64, 6, 10, D=2, dtype="bf16", seed=22, device=DEV)
    xh, wh, bh = si.random_case("3d", 1, 64, 12, 12, 40, D=3, dtype="bf16", seed=23, device=DEV)
    op2 = Conv3x3(w2, b2, 2, 40, 72, stride=1, epilogue="relu", algo=C.ALGO_MFMA)
    op3 = Conv3x3x3(w3, b3, 1, 2, 6, 10, epilogue="none", algo=C.ALGO_MFMA)
    assert op3.ws_bytes > 0, "expected a split-K plan (workspace partials)"
    xk, wk, bk = si.random_case("3d", 1, 512, 512, 44, 78, D=1, dtype="bf16", seed=24, device=DEV)
    xs, ws, bs = si.random_case("3d", 1, 416, 300, 44, 78, D=4, dtype="bf16", seed=25, device=DEV)
    assert C.conv3x3x3_describe(1, 512, 512, 1, 44, 78).startswith("igemm32_kq ")
    assert C.conv3x3x3_describe(1, 416, 300, 4, 44, 78).startswith("igemm32_sk ")
    opk = Conv3x3x3(wk, bk, 1, 1, 44, 78, epilogue="none", algo=C.ALGO_AUTO)
    ops = Conv3x3x3(ws, bs, 1, 4, 44, 78, epilogue="relu", algo=C.ALGO_AUTO)
    ops.workspace.fill_(0xA5)   # counters start as garbage: the call clears them
    oph = Conv3x3x3(wh, bh, 1, 3, 12, 40, epilogue="clamp1", algo=C.ALGO_FUSED_HEAD)
    y2 = torch.empty(op2.out_shape(), dtype=torch.float16, device=DEV)
    y3 = torch.empty(op3.out_shape(), dtype=torch.bfloat16, device=DEV)
    yh = torch.empty(oph.out_shape(), dtype=torch.bfloat16, device=DEV)
    yk = torch.empty(opk.out_shape(), dtype=torch.bfloat16, device=DEV)
    ys = torch.empty(ops.out_shape(), dtype=torch.bfloat16, device=DEV)
    rgb = torch.empty((1, 3, 24, 80, 3), dtype=torch.uint8, device=DEV)

    def run(stream=None):
        op2(x2, y2, stream=stream)
        op3(x3, y3, stream=stream)
        opk(xk, yk, stream=stream)
        ops(xs, ys, stream=stream)
        oph(xh, yh, stream=stream)
        C.conv_video_rgb8(yh, rgb, 1, 3, 12, 40, 12, C.DTYPE_BF16, stream)

    # warm-up on a side stream, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()

    gen = torch.Generator(device="cpu").manual_seed(5)
    for rep in range(4):
        # new inputs in the captured buffers
        x2.copy_(torch.relu(torch.randn(x2.shape, generator=gen)).to(x2.dtype))
        x3.copy_(torch.randn(x3.shape, generator=gen).to(x3.dtype))
        xh.copy_(torch.randn(xh.shape, generator=gen).to(xh.dtype))
        xk.copy_(torch.randn(xk.shape, generator=gen).to(xk.dtype))
        xs.copy_(torch.randn(xs.shape, generator=gen).to(xs.dtype))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        outs = (y2, y3, yk, ys, yh, rgb)
        got = [t.clone() for t in outs]
        # eager work between replays, on the same inputs: the reference
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        run()
        torch.cuda.synchronize()
        names = ("2d", "3d split-K", "3d K over waves", "3d stream-K", "fused head", "video")
        for name, a, b in zip(names, got, outs):
            assert torch.equal(_bits(a), _bits(b)), "replay %d: %s differs from the eager call" % (rep, name)
        _say("graph replay %d equals the eager calls" % rep)
