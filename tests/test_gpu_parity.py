"""Parity of the HIP path (through the C ABI) with the CPU oracle on an MI355X.

* integer-valued inputs: every partial sum is exact in fp32 and in the storage dtype, so every
  kernel must reproduce the oracle bit for bit (index, halo, padding, tail and race bugs show);
* random inputs at small sizes spanning several tiles and ragged tails: full tensors within the
  fp16/bf16 tolerances;
* the workloads at full size, in the launch configuration the benchmark times: sampled outputs
  within the tolerances, plus guard-band / NaN-poison and run-twice determinism checks.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from gpu_support import (DEV, EPI, alloc_guarded, assert_bit_exact, assert_within, bits,
                         check_guards, gather_2d, gather_3d, metrics, odt, oracle_2d, oracle_3d,
                         run_2d, run_3d, sample_points_2d, sample_points_3d)
from x3x3_convolution_amd import conv as C
from x3x3_convolution_amd.plan import Conv3x3x3

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# ------------------------------------------------------------------------------------------
# integer-exact parity
# ------------------------------------------------------------------------------------------
CASES_2D_INT = [
    # N, Ci, Co, H, W, stride, dtype, epilogue
    (1, 16, 16, 64, 64, 1, "f16", "relu"),
    (2, 5, 7, 13, 37, 1, "f16", "none"),
    (2, 5, 7, 13, 37, 2, "f16", "clamp1"),
    (1, 64, 64, 19, 45, 1, "bf16", "relu"),
    (1, 33, 40, 20, 70, 2, "f16", "relu"),
    (3, 3, 130, 9, 10, 1, "bf16", "none"),
    (1, 17, 24, 33, 1, 2, "f16", "none"),
    (1, 1, 1, 1, 1, 1, "f16", "relu"),
    (2, 64, 64, 32, 64, 2, "f16", "relu"),
]


@pytest.mark.parametrize("case", CASES_2D_INT, ids=[str(c) for c in CASES_2D_INT])
def test_simt2d_integer_exact(case):
    N, Ci, Co, H, W, s, dt, epi = case
    _say("simt2d int %s" % (case,))
    x, w, b = si.integer_case("2d", N, Ci, Co, H, W, dtype=dt, seed=CASES_2D_INT.index(case),
                              device=DEV)
    y = run_2d(x, w, b, s, epi, guarded=True)
    assert_bit_exact(y, oracle_2d(x, w, b, s, epi), x.dtype)


CASES_2D_MFMA_INT = [
    # N, Ci, Co, H, W, stride, dtype, epilogue  (C_in % 8 == 0, C_in, C_out <= 64, W % 8 == 0)
    (1, 16, 16, 64, 64, 1, "f16", "relu"),
    (2, 8, 7, 13, 40, 1, "f16", "none"),        # ragged rows, a partial column tile
    (2, 8, 7, 13, 40, 2, "f16", "clamp1"),
    (1, 64, 64, 19, 48, 1, "bf16", "relu"),
    (1, 40, 40, 20, 72, 2, "f16", "relu"),
    (3, 24, 64, 9, 16, 1, "bf16", "none"),
    (1, 64, 33, 33, 8, 2, "f16", "none"),       # W = 8: one column group
    (1, 8, 1, 1, 8, 1, "f16", "relu"),
    (2, 64, 64, 32, 64, 2, "f16", "relu"),
    (1, 64, 64, 70, 264, 1, "f16", "relu"),
    (5, 16, 16, 128, 256, 1, "f16", "relu"),    # 320 tiles: workgroups run two
    (9, 16, 24, 64, 256, 2, "bf16", "clamp1"),  # 288 tiles at stride 2
]


@pytest.mark.parametrize("case", CASES_2D_MFMA_INT, ids=[str(c) for c in CASES_2D_MFMA_INT])
def test_mfma2d_integer_exact(case):
    N, Ci, Co, H, W, s, dt, epi = case
    _say("mfma2d int %s" % (case,))
    x, w, b = si.integer_case("2d", N, Ci, Co, H, W, dtype=dt,
                              seed=100 + CASES_2D_MFMA_INT.index(case), device=DEV)
    y = run_2d(x, w, b, s, epi, guarded=True, algo=C.ALGO_MFMA)
    assert_bit_exact(y, oracle_2d(x, w, b, s, epi), x.dtype)


CASES_3D_INT = [
    # N, Ci, Co, D, H, W, dtype, epilogue, algo
    (1, 32, 12, 3, 9, 35, "bf16", "clamp1", C.ALGO_MFMA),
    (2, 40, 20, 2, 11, 19, "bf16", "none", C.ALGO_MFMA),
    (1, 8, 1, 1, 5, 5, "bf16", "relu", C.ALGO_MFMA),
    (1, 64, 130, 4, 9, 17, "f16", "none", C.ALGO_MFMA),
    (1, 8, 12, 16, 128, 128, "bf16", "clamp1", C.ALGO_MFMA),     # no split-K, narrow tiles
    (1, 8, 129, 16, 64, 64, "bf16", "relu", C.ALGO_MFMA),        # no split-K, wide tiles
    # the direct head's 64-channel stages: K split to one chunk per workgroup (the stage's second
    # chunk empty), five chunks of which the last holds 8 channels, 24 channels (three pieces of
    # one chunk), and 136 channels split 3 + 2 chunks (a full pair, a half pair, a full pair)
    (1, 256, 12, 3, 20, 70, "bf16", "relu", C.ALGO_MFMA),
    (1, 136, 7, 4, 9, 33, "f16", "none", C.ALGO_MFMA),
    (2, 24, 16, 2, 17, 40, "bf16", "clamp1", C.ALGO_MFMA),
    (1, 136, 12, 16, 64, 128, "bf16", "relu", C.ALGO_MFMA),
    # frame groups: 13 frames as 8 + 5 (eight per workgroup, a part-empty last group), 9 frames as
    # 4 + 4 + 1 (four per workgroup)
    (1, 40, 12, 13, 9, 40, "bf16", "relu", C.ALGO_MFMA),
    (1, 72, 5, 9, 11, 36, "f16", "clamp1", C.ALGO_MFMA),
    (1, 32, 12, 3, 9, 50, "bf16", "clamp1", C.ALGO_SPLIT_HEAD),
    (2, 64, 5, 1, 7, 130, "bf16", "none", C.ALGO_SPLIT_HEAD),
    (1, 8, 12, 4, 70, 64, "f16", "clamp1", C.ALGO_SPLIT_HEAD),
    (1, 16, 12, 16, 40, 100, "bf16", "relu", C.ALGO_SPLIT_HEAD),
    (1, 32, 12, 3, 9, 50, "bf16", "clamp1", C.ALGO_FUSED_HEAD),
    (2, 64, 5, 1, 7, 130, "bf16", "none", C.ALGO_FUSED_HEAD),
    (1, 8, 12, 4, 70, 64, "f16", "clamp1", C.ALGO_FUSED_HEAD),
    (1, 16, 12, 16, 40, 100, "bf16", "relu", C.ALGO_FUSED_HEAD),
    (1, 40, 7, 2, 33, 157, "bf16", "clamp1", C.ALGO_FUSED_HEAD),
    (1, 8, 12, 1, 1, 1, "bf16", "clamp1", C.ALGO_FUSED_HEAD),
    # the head's production channel count (8 chunks: several chunk pairs per Z row, prefetches
    # that stay in the row) and an odd chunk count (136 channels: 5 chunks padded to 6)
    (1, 256, 12, 3, 9, 130, "bf16", "clamp1", C.ALGO_SPLIT_HEAD),
    (1, 256, 12, 3, 9, 130, "bf16", "clamp1", C.ALGO_FUSED_HEAD),
    (1, 136, 12, 3, 9, 130, "bf16", "none", C.ALGO_SPLIT_HEAD),
    (1, 136, 12, 3, 9, 130, "bf16", "none", C.ALGO_FUSED_HEAD),
    (1, 136, 5, 6, 11, 70, "f16", "relu", C.ALGO_FUSED_HEAD),
    # more frame groups than one (the per-group input and output windows), a partial last group
    (1, 16, 12, 22, 6, 40, "bf16", "clamp1", C.ALGO_FUSED_HEAD),
    (1, 16, 12, 22, 6, 40, "bf16", "clamp1", C.ALGO_SPLIT_HEAD),
    # row ranges that run from the end of one strip into the next (several strips, a frame-group
    # count that leaves ranges of a few rows), one and two samples
    (1, 32, 12, 40, 37, 300, "bf16", "clamp1", C.ALGO_FUSED_HEAD),
    (1, 32, 12, 40, 37, 300, "bf16", "clamp1", C.ALGO_SPLIT_HEAD),
    (2, 16, 12, 32, 17, 380, "f16", "relu", C.ALGO_FUSED_HEAD),
    (2, 16, 12, 32, 17, 380, "f16", "relu", C.ALGO_SPLIT_HEAD),
    # the production channel count (C_in 256) in more shapes: fp16, two frame groups (the second
    # part-empty) over two strips; C_out 7 on two samples; ranges that cross strips; a single
    # position
    # long K: the head's stages over 16 chunks per Z row; K split 32 and 64 ways (one chunk per
    # split, the reduce over that many partials)
    (1, 512, 12, 3, 9, 130, "bf16", "clamp1", C.ALGO_FUSED_HEAD),
    (1, 512, 12, 3, 9, 130, "bf16", "clamp1", C.ALGO_SPLIT_HEAD),
    (1, 1024, 40, 2, 5, 9, "bf16", "relu", C.ALGO_MFMA),
    (1, 2048, 64, 1, 8, 16, "f16", "none", C.ALGO_MFMA),
    (1, 256, 12, 5, 13, 140, "f16", "relu", C.ALGO_FUSED_HEAD),
    (1, 256, 12, 5, 13, 140, "f16", "relu", C.ALGO_SPLIT_HEAD),
    (2, 256, 7, 4, 10, 60, "bf16", "none", C.ALGO_FUSED_HEAD),
    (2, 256, 7, 4, 10, 60, "bf16", "none", C.ALGO_SPLIT_HEAD),
    (1, 256, 12, 40, 37, 300, "bf16", "clamp1", C.ALGO_FUSED_HEAD),
    (1, 256, 12, 40, 37, 300, "bf16", "clamp1", C.ALGO_SPLIT_HEAD),
    (1, 256, 12, 1, 1, 1, "bf16", "clamp1", C.ALGO_FUSED_HEAD),
]


@pytest.mark.parametrize("case", CASES_3D_INT, ids=[str(c) for c in CASES_3D_INT])
def test_conv3d_integer_exact(case):
    N, Ci, Co, D, H, W, dt, epi, algo = case
    _say("conv3d int %s" % (case,))
    x, w, b = si.integer_case("3d", N, Ci, Co, H, W, D=D, dtype=dt, seed=CASES_3D_INT.index(case),
                              device=DEV)
    y = run_3d(x, w, b, epi, algo, guarded=True)
    assert_bit_exact(y, oracle_3d(x, w, b, epi), x.dtype)


# One spatial tap at a time through the head kernels.  The GEMM rows of the taps sit in different
# places -- taps 0..7 in the 32-row accumulator blocks, tap 8 in the 16-row tile whose operands and
# results are moved between lanes -- so with a weight tensor that is zero except at one (ky, kx),
# a wrong row, lane or k order shows up as that whole tap wrong.  No clamp, so nothing saturates.
# C_in 32 (one chunk pair per Z row) and the production 256 (four pairs).
@pytest.mark.parametrize("ci", [32, 256])
@pytest.mark.parametrize("algo", [C.ALGO_SPLIT_HEAD, C.ALGO_FUSED_HEAD])
@pytest.mark.parametrize("tap", range(9))
def test_head_single_spatial_tap_exact(tap, algo, ci):
    ky, kx = divmod(tap, 3)
    _say("head single tap (%d, %d) algo %d C_in %d" % (ky, kx, algo, ci))
    x, w, b = si.integer_case("3d", 1, ci, 12, 9, 50, D=3, dtype="bf16", seed=700 + tap, device=DEV)
    only = torch.zeros_like(w)
    only[:, :, :, ky, kx] = w[:, :, :, ky, kx]
    assert torch.count_nonzero(only) > 0
    y = run_3d(x, only, b, "none", algo, guarded=True)
    assert_bit_exact(y, oracle_3d(x, only, b, "none"), x.dtype)


# The 32x32 MFMA family (C_out > 16) picks its tile -- 8x32, 16x16 (256 positions), 4x32 or 8x16
# (128 positions) -- and split-K count from a cost model; these shapes reach each of the eight
# (tile, split) combinations.  The workspace size says whether K is split.
CASES_W32_TILES = [
    # N, Ci, Co, D, H, W, epilogue, tile, split-K
    (1, 32, 20, 1, 5, 13, "relu", "4x32", False),
    (1, 64, 20, 1, 5, 13, "none", "4x32", True),
    (2, 32, 20, 16, 33, 13, "clamp1", "8x16", False),
    (2, 96, 20, 16, 9, 13, "none", "8x16", True),
    (2, 32, 20, 16, 33, 17, "relu", "8x32", False),
    (1, 96, 20, 16, 9, 33, "none", "8x32", True),
    (2, 32, 260, 16, 33, 13, "none", "16x16", False),
    (2, 96, 20, 16, 20, 13, "clamp1", "16x16", True),
]


@pytest.mark.parametrize("case", CASES_W32_TILES, ids=["%s-%s" % (c[7], "splitk" if c[8] else "nosplit")
                                                       for c in CASES_W32_TILES])
def test_conv3d_w32_tiles_integer_exact(case):
    N, Ci, Co, D, H, W, epi, tile, splitk = case
    _say("conv3d w32 tile %s" % (case,))
    ws = C.conv3x3x3_workspace_bytes(N, Ci, Co, D, H, W, dtype=C.DTYPE_BF16, algo=C.ALGO_MFMA)
    assert (ws > 0) == splitk
    assert C.conv3x3x3_describe(N, Ci, Co, D, H, W, algo=C.ALGO_MFMA).startswith(
        "igemm32 tile=%s rows=256 " % tile)
    x, w, b = si.integer_case("3d", N, Ci, Co, H, W, D=D, dtype="bf16",
                              seed=300 + CASES_W32_TILES.index(case), device=DEV)
    y = run_3d(x, w, b, epi, C.ALGO_MFMA, guarded=True)
    assert_bit_exact(y, oracle_3d(x, w, b, epi), x.dtype)


# The 32x32 family with K split over the four waves of a workgroup (64-row tiles, the partial
# tiles summed through LDS, no workspace), where the cost model sends it: few positions, many
# input channels.  Ragged chunk counts (264 channels: waves of 2, 2, 2, 3 chunks, the last chunk
# a quarter full; 296: 2, 3, 2, 3), part-empty 64-row tiles (72, 130 channels), ragged
# frame edges, first and last frames with two temporal taps, both 128-position tiles and fp16.
CASES_KQ = [
    # N, Ci, Co, D, H, W, dtype, epilogue, tile
    (1, 264, 72, 3, 36, 60, "bf16", "relu", "4x32"),
    (1, 296, 130, 1, 50, 90, "bf16", "none", "4x32"),
    (1, 256, 256, 2, 44, 78, "bf16", "clamp1", "8x16"),
    (1, 488, 72, 3, 36, 60, "f16", "none", "4x32"),
]


@pytest.mark.parametrize("case", CASES_KQ, ids=[str(c) for c in CASES_KQ])
def test_conv3d_kq_integer_exact(case):
    N, Ci, Co, D, H, W, dt, epi, tile = case
    _say("conv3d kq %s" % (case,))
    dtype = C.DTYPE_F16 if dt == "f16" else C.DTYPE_BF16
    assert C.conv3x3x3_workspace_bytes(N, Ci, Co, D, H, W, dtype=dtype, algo=C.ALGO_AUTO) == 0
    assert C.conv3x3x3_describe(N, Ci, Co, D, H, W, dtype=dtype).startswith(
        "igemm32_kq tile=%s rows=64 splits=1 " % tile)
    x, w, b = si.integer_case("3d", N, Ci, Co, H, W, D=D, dtype=dt,
                              seed=500 + CASES_KQ.index(case), device=DEV)
    y = run_3d(x, w, b, epi, C.ALGO_AUTO, guarded=True)
    assert_bit_exact(y, oracle_3d(x, w, b, epi), x.dtype)


# The 32x32 family's stream-K schedule, where the cost model sends it: one round of whole
# 256-row tiles would wait for the interior frames' tiles (three temporal taps), and K is long.
# About one workgroup per tile, each taking an equal share of all tiles' stages; a tile split
# between workgroups is summed from fp32 partials by the piece that ends last, in K order.  Both
# 128-position tiles, part-empty second 256-row tiles (300 and 384 channels: padding waves compute
# zeros and store nothing), 184 to 256 workgroups, three to five frames, fp16, and the low-res
# 512 -> 512 convolution itself.  Tiles split in two (the one-burst sum) in every case, and in
# three (the general K-order sum) in the first, third and fourth (16 to 24 such tiles each).
CASES_SK = [
    # N, Ci, Co, D, H, W, dtype, epilogue, tile
    (1, 416, 384, 5, 44, 33, "bf16", "relu", "4x32"),
    (1, 416, 300, 4, 44, 78, "f16", "none", "8x16"),
    (1, 416, 300, 5, 36, 78, "bf16", "clamp1", "8x16"),
    (1, 448, 384, 3, 44, 78, "f16", "relu", "8x16"),
    (1, 512, 512, 4, 44, 78, "bf16", "none", "8x16"),
]


@pytest.mark.parametrize("case", CASES_SK, ids=[str(c) for c in CASES_SK])
def test_conv3d_stream_k_integer_exact(case):
    N, Ci, Co, D, H, W, dt, epi, tile = case
    _say("conv3d stream-K %s" % (case,))
    dtype = C.DTYPE_F16 if dt == "f16" else C.DTYPE_BF16
    assert C.conv3x3x3_workspace_bytes(N, Ci, Co, D, H, W, dtype=dtype, algo=C.ALGO_AUTO) > 0
    assert C.conv3x3x3_describe(N, Ci, Co, D, H, W, dtype=dtype).startswith(
        "igemm32_sk tile=%s rows=256 splits=1 " % tile)
    x, w, b = si.integer_case("3d", N, Ci, Co, H, W, D=D, dtype=dt,
                              seed=700 + CASES_SK.index(case), device=DEV)
    op = Conv3x3x3(w, b, N, D, H, W, epilogue=epi, algo=C.ALGO_AUTO)
    op.workspace.fill_(0xA5)   # counters and slots start as garbage: the call clears what it needs
    ys = []
    for _ in range(2):         # the second call finds the first one's partials and counters
        buf, y = alloc_guarded(op.out_shape(), x.dtype)
        op(x, y)
        torch.cuda.synchronize()
        check_guards(buf, y.numel())
        ys.append(y)
    assert_bit_exact(ys[0], oracle_3d(x, w, b, epi), x.dtype)
    assert torch.equal(ys[0].view(torch.int16), ys[1].view(torch.int16))


# Spatial stride 2 (H, W halve, frames keep stride 1): the 32x32 family's 128-position tiles
# (4x32, 8x16) with the even/odd window columns; the first four shapes reach each (tile,
# split-K) combination, the others vary C_in, C_out, dtype and ragged edges.
CASES_S2 = [
    # N, Ci, Co, D, H, W, dtype, epilogue, split-K (None: not asserted)
    (1, 16, 5, 1, 9, 9, "bf16", "relu", False),
    (1, 64, 5, 1, 9, 9, "bf16", "none", True),
    (2, 16, 5, 16, 65, 9, "bf16", "clamp1", False),
    (2, 96, 5, 16, 17, 9, "bf16", "none", True),
    (1, 64, 130, 3, 33, 50, "f16", "relu", None),
    (1, 32, 20, 5, 40, 65, "bf16", "none", None),
    (2, 8, 64, 2, 17, 17, "bf16", "clamp1", None),
    (1, 40, 300, 1, 2, 1, "bf16", "none", None),
]


def run_3d_s2(x, w, b, epilogue):
    N, D, H, W, _ = x.shape
    op = Conv3x3x3(w, b, N, D, H, W, epilogue=epilogue, algo=C.ALGO_AUTO, stride=2)
    assert op.algo == C.ALGO_MFMA
    buf, y = alloc_guarded(op.out_shape(), x.dtype)
    op(x, y)
    torch.cuda.synchronize()
    check_guards(buf, y.numel())
    return y, op


def oracle_3d_s2(x, w, b, epilogue):
    return oracle.conv3d(bits(x), bits(w), bits(b), 2, odt(x.dtype), EPI[epilogue],
                         oracle.CHANNELS_LAST)


@pytest.mark.parametrize("case", CASES_S2, ids=[str(c) for c in CASES_S2])
def test_conv3d_stride2_integer_exact(case):
    N, Ci, Co, D, H, W, dt, epi, splitk = case
    _say("conv3d stride 2 int %s" % (case,))
    x, w, b = si.integer_case("3d", N, Ci, Co, H, W, D=D, dtype=dt, seed=400 + CASES_S2.index(case),
                              device=DEV)
    y, op = run_3d_s2(x, w, b, epi)
    assert y.shape == (N, D, (H - 1) // 2 + 1, (W - 1) // 2 + 1, Co)
    if splitk is not None:
        assert (op.ws_bytes > 0) == splitk
    assert_bit_exact(y, oracle_3d_s2(x, w, b, epi), x.dtype)


def test_conv3d_stride2_random_tolerance():
    x, w, b = si.random_case("3d", 1, 256, 256, 24, 40, D=3, dtype="bf16", seed=8, device=DEV)
    y, _ = run_3d_s2(x, w, b, "none")
    y2, _ = run_3d_s2(x, w, b, "none")
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "not deterministic"
    m = metrics(bits(y), oracle_3d_s2(x, w, b, "none"), x.dtype)
    _say("stride 2 random %s" % (m,))
    assert_within(m, activated=False)


def test_conv3d_no_bias_integer_exact():
    x, w, _ = si.integer_case("3d", 1, 32, 12, 5, 9, D=2, dtype="bf16", seed=3, device=DEV,
                              with_bias=False)
    for algo in (C.ALGO_MFMA, C.ALGO_SPLIT_HEAD, C.ALGO_FUSED_HEAD):
        y = run_3d(x, w, None, "clamp1", algo)
        assert_bit_exact(y, oracle_3d(x, w, None, "clamp1"), x.dtype)
    x, w, _ = si.integer_case("2d", 2, 6, 9, 11, 13, dtype="f16", seed=4, device=DEV,
                              with_bias=False)
    y = run_2d(x, w, None, 1, "relu")
    assert_bit_exact(y, oracle_2d(x, w, None, 1, "relu"), x.dtype)
    x, w, _ = si.integer_case("2d", 2, 16, 9, 11, 16, dtype="f16", seed=4, device=DEV,
                              with_bias=False)
    y = run_2d(x, w, None, 1, "relu", algo=C.ALGO_MFMA)
    assert_bit_exact(y, oracle_2d(x, w, None, 1, "relu"), x.dtype)


# ------------------------------------------------------------------------------------------
# random inputs at small sizes, whole tensors within tolerance
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("algo", [C.ALGO_SIMT, C.ALGO_MFMA])
def test_2d_random_tolerance(algo):
    for s in (1, 2):
        x, w, b = si.random_case("2d", 2, 64, 64, 40, 72, dtype="f16", seed=s, device=DEV)
        x = torch.relu(x)
        y = run_2d(x, w, b, s, "relu", algo=algo)
        m = metrics(bits(y), oracle_2d(x, w, b, s, "relu"), x.dtype)
        _say("2d random algo=%d s=%d %s" % (algo, s, m))
        assert_within(m, activated=True)


@pytest.mark.parametrize("algo", [C.ALGO_MFMA, C.ALGO_SPLIT_HEAD, C.ALGO_FUSED_HEAD])
def test_head_random_tolerance(algo):
    x, w, b = si.random_case("3d", 1, 256, 12, 12, 40, D=3, dtype="bf16", seed=5, device=DEV)
    y = run_3d(x, w, b, "clamp1", algo)
    m = metrics(bits(y), oracle_3d(x, w, b, "clamp1"), x.dtype)
    _say("head random algo=%d %s" % (algo, m))
    assert_within(m, activated=True)


@pytest.mark.parametrize("Ci,Co,D,H,W", [(256, 64, 3, 10, 20), (512, 512, 2, 6, 10)])
def test_mfma_random_tolerance(Ci, Co, D, H, W):
    x, w, b = si.random_case("3d", 1, Ci, Co, H, W, D=D, dtype="bf16", seed=6, device=DEV)
    y = run_3d(x, w, b, "none", C.ALGO_MFMA)
    m = metrics(bits(y), oracle_3d(x, w, b, "none"), x.dtype)
    _say("mfma random %s %s" % ((Ci, Co, D, H, W), m))
    assert_within(m, activated=False)


# ------------------------------------------------------------------------------------------
# the workloads at full size
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("algo", [C.ALGO_SIMT, C.ALGO_MFMA])
def test_c1_full_tensor(algo):
    wl = si.WORKLOADS["c1"]
    x, w, b = si.make_inputs(wl, device=DEV)
    y = run_2d(x, w, b, wl.stride, wl.epilogue, guarded=True, algo=algo)
    m = metrics(bits(y), oracle_2d(x, w, b, wl.stride, wl.epilogue), x.dtype)
    _say("c1 algo=%d %s" % (algo, m))
    assert_within(m, activated=True)


@pytest.mark.parametrize("name,algo", [(n, a) for n in ("c2", "c2s2")
                                       for a in (C.ALGO_SIMT, C.ALGO_MFMA)])
def test_c2_full_size_sampled(name, algo):
    wl = si.WORKLOADS[name]
    x, w, b = si.make_inputs(wl, device=DEV)
    y = run_2d(x, w, b, wl.stride, wl.epilogue, guarded=True, algo=algo)
    y2 = run_2d(x, w, b, wl.stride, wl.epilogue, algo=algo)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "not deterministic"
    pts = sample_points_2d(wl.N, wl.H_out, wl.W_out, 400, seed=1)
    ref = oracle.conv2d_points(bits(x), bits(w), bits(b), pts, wl.stride, oracle.F16,
                               oracle.EPI_RELU, oracle.CHANNELS_FIRST)
    m = metrics(gather_2d(y, pts), ref, x.dtype)
    _say("%s algo=%d sampled %d %s" % (name, algo, len(pts), m))
    assert_within(m, activated=True)


@pytest.mark.parametrize("algo", [C.ALGO_SIMT, C.ALGO_MFMA])
def test_2d_largest_image_sampled(algo):
    """The largest 2D image the matrix-core kernel takes: 64 channels of 4096 x 4088 fp16, just
    below 2 GiB per image of x and of y (one 32-bit buffer range each), three images so that the
    last one's addresses cross 4 GiB.  Sampled outputs of every image against the oracle; the
    SIMT kernel on the same input."""
    wl = dataclasses.replace(si.WORKLOADS["c2"], N=3, H=4096, W=4088)
    assert wl.C_in * wl.H * wl.W * 2 < 1 << 31 < 2 * wl.C_in * wl.H * wl.W * 2
    _say("largest 2D image: %s algo %d" % ((wl.N, wl.C_in, wl.C_out, wl.H, wl.W), algo))
    x, w, b = si.make_inputs(wl, device=DEV)
    y = run_2d(x, w, b, wl.stride, wl.epilogue, guarded=True, algo=algo)
    pts = sample_points_2d(wl.N, wl.H_out, wl.W_out, 150, seed=5)
    pts = np.concatenate([pts, np.array([[1, 0, 0], [1, wl.H - 1, wl.W - 1]], np.int32)])
    ref = oracle.conv2d_points(bits(x), bits(w), bits(b), pts, wl.stride, oracle.F16,
                               oracle.EPI_RELU, oracle.CHANNELS_FIRST)
    m = metrics(gather_2d(y, pts), ref, x.dtype)
    _say("largest 2D image algo=%d sampled %d %s" % (algo, len(pts), m))
    assert_within(m, activated=True)


@pytest.mark.parametrize("name,algo", [("c3", C.ALGO_MFMA), ("c3", C.ALGO_SPLIT_HEAD),
                                       ("c3", C.ALGO_FUSED_HEAD),
                                       ("c4", C.ALGO_MFMA), ("c5", C.ALGO_MFMA),
                                       ("c5d1", C.ALGO_MFMA)])
def test_3d_full_size_sampled(name, algo):
    wl = si.WORKLOADS[name]
    _say("full size %s algo %d" % (name, algo))
    x, w, b = si.make_inputs(wl, device=DEV)
    y = run_3d(x, w, b, wl.epilogue, algo, guarded=True)
    y2 = run_3d(x, w, b, wl.epilogue, algo)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "not deterministic"
    del y2
    n_rand = 300 if wl.C_out * wl.C_in <= 256 * 256 else 120
    pts = sample_points_3d(wl.N, wl.D, wl.H, wl.W, n_rand, seed=2)
    epi = {"none": oracle.EPI_NONE, "relu": oracle.EPI_RELU, "clamp1": oracle.EPI_CLAMP1}
    ref = oracle.conv3d_points(bits(x), bits(w), bits(b), pts, 1, oracle.BF16,
                               epi[wl.epilogue], oracle.CHANNELS_LAST)
    m = metrics(gather_3d(y, pts), ref, x.dtype)
    _say("%s algo %d sampled %d %s" % (name, algo, len(pts), m))
    assert_within(m, activated=wl.epilogue != "none")


@pytest.mark.parametrize("name,D,algo", [("c3", 32, C.ALGO_FUSED_HEAD), ("c3", 32, C.ALGO_SPLIT_HEAD),
                                         ("c3", 32, C.ALGO_MFMA), ("c4", 160, C.ALGO_MFMA)])
def test_3d_beyond_32bit_offsets(name, D, algo):
    """Inputs past 32-bit byte offsets: the output head over 32 frames (3.6 GB of input, on the
    head kernels, which address each workgroup's six input and four output frames through their
    own 32-bit ranges, and on the direct 27-tap kernel, which addresses ten input rows at a time)
    and the mid-decoder conv over 160 frames (4.5 GB in and out).  Sampled outputs in the first,
    middle and last frames against the oracle."""
    wl = dataclasses.replace(si.WORKLOADS[name], D=D)
    _say("beyond 32-bit offsets: %s D=%d algo %d" % (name, D, algo))
    auto = C.conv3x3x3_select_algo(wl.N, wl.C_in, wl.C_out, wl.D, wl.H, wl.W, 1,
                                   C.LAYOUT_CHANNELS_LAST, C.DTYPE_BF16, C.ALGO_AUTO)
    assert auto == (C.ALGO_FUSED_HEAD if wl.C_out <= 12 else C.ALGO_MFMA)
    x, w, b = si.make_inputs(wl, device=DEV)
    y = run_3d(x, w, b, wl.epilogue, algo, guarded=True)
    pts = sample_points_3d(wl.N, wl.D, wl.H, wl.W, 100, seed=3)
    ref = oracle.conv3d_points(bits(x), bits(w), bits(b), pts, 1, oracle.BF16, EPI[wl.epilogue],
                               oracle.CHANNELS_LAST)
    m = metrics(gather_3d(y, pts), ref, x.dtype)
    _say("%s D=%d algo %d sampled %d %s" % (name, D, algo, len(pts), m))
    assert_within(m, activated=wl.epilogue != "none")


def test_3d_wide_frame_past_2gib():
    """One input frame of 2 GiB (2048 x 2048 positions x 256 channels): past the 32x32 family's
    per-frame range, so C_out > 16 runs on the 16x16x32 wide tiles, which address x with 64-bit
    offsets.  Sampled outputs against the oracle."""
    wl = si.Workload("wide", "3d", N=1, C_in=256, C_out=32, D=1, H=2048, W=2048, dtype="bf16",
                     epilogue="none", x_dist="normal", w_var=1.0 / (27 * 256), x_id=61, w_id=61)
    assert wl.H * wl.W * wl.C_in * 2 >= 1 << 31
    _say("wide frame past 2 GiB: %s" % ((wl.N, wl.C_in, wl.C_out, wl.D, wl.H, wl.W),))
    x, w, b = si.make_inputs(wl, device=DEV)
    y = run_3d(x, w, b, wl.epilogue, C.ALGO_MFMA, guarded=True)
    pts = sample_points_3d(wl.N, wl.D, wl.H, wl.W, 150, seed=4)
    ref = oracle.conv3d_points(bits(x), bits(w), bits(b), pts, 1, oracle.BF16, EPI[wl.epilogue],
                               oracle.CHANNELS_LAST)
    m = metrics(gather_3d(y, pts), ref, x.dtype)
    _say("wide frame sampled %d %s" % (len(pts), m))
    assert_within(m, activated=False)


def test_fused_head_at_least_as_accurate_as_split_head():
    """The fused head keeps the temporal GEMM's fp32 sums through the nine-tap stencil, the split
    head rounds them to bf16 in its plane.  On the full-size head the fused outputs must be
    within tolerance of the oracle and no less accurate than the split head's, at the same
    sampled points (errors against the unrounded fp64 oracle value)."""
    wl = si.WORKLOADS["c3"]
    x, w, b = si.make_inputs(wl, device=DEV)
    pts = sample_points_3d(wl.N, wl.D, wl.H, wl.W, 2000, seed=5)
    ref = oracle.conv3d_points(bits(x), bits(w), bits(b), pts, 1, oracle.BF16,
                               oracle.EPI_CLAMP1, oracle.CHANNELS_LAST)
    errs = {}
    for algo in (C.ALGO_SPLIT_HEAD, C.ALGO_FUSED_HEAD):
        y = run_3d(x, w, b, wl.epilogue, algo, guarded=algo == C.ALGO_FUSED_HEAD)
        got = oracle.decode(gather_3d(y, pts), oracle.BF16).reshape(ref.shape)
        errs[algo] = float(np.sqrt(np.mean((got - ref) ** 2)))
        del y
    _say("rms error vs fp64: split %.3e fused %.3e" % (errs[C.ALGO_SPLIT_HEAD], errs[C.ALGO_FUSED_HEAD]))
    assert errs[C.ALGO_FUSED_HEAD] <= errs[C.ALGO_SPLIT_HEAD] * 1.02


@pytest.mark.parametrize("Co", [12, 5, 7])
def test_split_head_plane_stage_matches_oracle_plane(Co):
    """The split head's first stage on its own (conv_head_temporal): the 112-channel plane must
    equal the oracle's split-mode plane rounded to bf16, and the channels past the 9*C_out tap
    channels must be written as zero (g starts as a NaN sentinel; integer inputs, so every sum
    is exact)."""
    N, Ci, D, H, W = 1, 32, 3, 9, 50
    x, w, b = si.integer_case("3d", N, Ci, Co, H, W, D=D, dtype="bf16", seed=77 + Co, device=DEV)
    from x3x3_convolution_amd.plan import Conv3x3x3
    op = Conv3x3x3(w, b, N, D, H, W, epilogue="clamp1", algo=C.ALGO_SPLIT_HEAD)
    g = torch.full((N, D, H, W, 112), 0x7FFF, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    C.conv_head_temporal(x, op.w_packed, g, N, Ci, Co, D, H, W, C.DTYPE_BF16)
    torch.cuda.synchronize()
    _, gref = oracle.head_split(bits(x), bits(w), bits(b), oracle.BF16, oracle.EPI_CLAMP1,
                                oracle.CHANNELS_LAST, round_g=True, return_g=True)
    got = bits(g)
    assert np.array_equal(got[..., :9 * Co], oracle.encode(gref, oracle.BF16))
    assert np.all(got[..., 9 * Co:] == 0)
