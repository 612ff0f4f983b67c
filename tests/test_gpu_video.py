"""Parity of the video step (conv_video_rgb8) with the oracle: the bytes must be identical.

Inputs are seeded synthetic head outputs (values spread over and beyond [-1, 1], with zeros of
both signs, tiny values, infinities and NaNs mixed in), so every rounding case and the clamp are
exercised; shapes cover the byte-store path (W not a multiple of 8), a ragged last chunk of 256
positions, and the full 704x1248 frame size.  A second test runs the fused head into the video
step on integer inputs, where the head's output is exact, against the oracle's convolution
followed by its video step.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from gpu_support import DEV, bits, odt, oracle_3d
from x3x3_convolution_amd import conv as C
from x3x3_convolution_amd.plan import Conv3x3x3

pytestmark = pytest.mark.gpu

GUARD = 512
FILL = 0xA5


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _synthetic_y(shape, dtype, seed):
    """Head-like outputs: mostly N(0, 0.6^2), some far outside [-1, 1], special values sprinkled."""
    g = torch.Generator("cpu").manual_seed(si.SEED_BASE + 900 + seed)
    v = torch.randn(shape, generator=g) * 0.6
    u = torch.rand(shape, generator=g)
    v = torch.where(u < 0.05, v * 8.0, v)
    specials = torch.tensor([0.0, -0.0, 1.0, -1.0, 0.5, -0.5, 1e-30, -1e-30, float("inf"),
                             float("-inf"), float("nan"), 127.0 / 127.5 - 1.0])
    idx = torch.randint(0, specials.numel(), shape, generator=g)
    v = torch.where(u > 0.97, specials[idx], v)
    return v.to(torch.float16 if dtype == "f16" else torch.bfloat16)


def _run(y, N, D, H, W):
    n = N * D * 2 * H * 2 * W * 3
    buf = torch.full((n + 2 * GUARD,), FILL, dtype=torch.uint8, device=DEV)
    rgb = buf[GUARD:GUARD + n].view(N, D, 2 * H, 2 * W, 3)
    C.conv_video_rgb8(y, rgb, N, D, H, W, 12, C.DTYPE_BF16 if y.dtype == torch.bfloat16 else
                      C.DTYPE_F16)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert np.all(host[:GUARD] == FILL) and np.all(host[GUARD + n:] == FILL), "write outside rgb"
    return host[GUARD:GUARD + n].reshape(N, D, 2 * H, 2 * W, 3)


CASES = [
    # N, D, H, W, dtype
    (1, 2, 3, 17, "bf16"),     # byte stores (W % 8 != 0)
    (2, 3, 5, 264, "bf16"),    # 16-byte stores, ragged last chunk of 8 positions
    (1, 1, 1, 1, "bf16"),
    (1, 4, 7, 520, "f16"),
    (1, 2, 4, 256, "f16"),     # exactly one chunk per row
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_video_bytes_match_oracle(case):
    N, D, H, W, dt = case
    _say("video %s" % (case,))
    y = _synthetic_y((N, D, H, W, 12), dt, CASES.index(case)).to(DEV)
    got = _run(y, N, D, H, W)
    want = oracle.video_rgb8(oracle.decode(bits(y), odt(y.dtype)))
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, "%d bytes differ, first at %d: got %d want %d" % (
        bad.size, bad[0], got.flat[bad[0]], want.flat[bad[0]])


def test_video_full_frame_size():
    """The 704x1248 RGB frames of the output head (16 frames of 352x624 positions)."""
    N, D, H, W = 1, 16, 352, 624
    _say("video full size")
    y = _synthetic_y((N, D, H, W, 12), "bf16", 99).to(DEV)
    got = _run(y, N, D, H, W)
    want = oracle.video_rgb8(oracle.decode(bits(y), oracle.BF16))
    assert np.array_equal(got, want)


def test_head_then_video_integer_exact():
    """Fused head (integer inputs: its output equals the oracle's, rounded once) followed by the
    video step, against the oracle's convolution and video step."""
    N, Ci, Co, D, H, W = 1, 32, 12, 3, 9, 140
    x, w, b = si.integer_case("3d", N, Ci, Co, H, W, D=D, dtype="bf16", seed=21, device=DEV)
    # scale the integer outputs into the codes' range: halve w and b twice (exact in bf16)
    w, b = w * 0.25, b * 0.25
    op = Conv3x3x3(w, b, N, D, H, W, epilogue="clamp1", algo=C.ALGO_FUSED_HEAD)
    y = op(x)
    torch.cuda.synchronize()
    got = _run(y, N, D, H, W)
    yref = oracle.decode(oracle.encode(oracle_3d(x, w, b, "clamp1"), oracle.BF16), oracle.BF16)
    want = oracle.video_rgb8(yref.reshape(N, D, H, W, Co))
    assert np.array_equal(got, want)


def test_fused_rgb_head_integer_exact():
    """conv3x3x3_head_rgb8 on integer inputs (exact head output) against the oracle's
    convolution and video step; guard bands around the frames."""
    N, Ci, D, H, W = 2, 40, 3, 11, 150
    x, w, b = si.integer_case("3d", N, Ci, 12, H, W, D=D, dtype="bf16", seed=23, device=DEV)
    w, b = w * 0.25, b * 0.25
    op = Conv3x3x3(w, b, N, D, H, W, epilogue="clamp1", algo=C.ALGO_FUSED_HEAD)
    n = N * D * 2 * H * 2 * W * 3
    buf = torch.full((n + 2 * GUARD,), FILL, dtype=torch.uint8, device=DEV)
    rgb = buf[GUARD:GUARD + n].view(N, D, 2 * H, 2 * W, 3)
    op.rgb8(x, rgb)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert np.all(host[:GUARD] == FILL) and np.all(host[GUARD + n:] == FILL), "write outside rgb"
    yref = oracle.decode(oracle.encode(oracle_3d(x, w, b, "clamp1"), oracle.BF16), oracle.BF16)
    want = oracle.video_rgb8(yref.reshape(N, D, H, W, 12))
    assert np.array_equal(host[GUARD:GUARD + n].reshape(want.shape), want)


@pytest.mark.parametrize("shape", [(1, 5, 33, 140, 64), (1, 16, 352, 624, 256)],
                         ids=["small", "c3_full"])
def test_fused_rgb_head_random(shape):
    """Random inputs: the fused RGB head's bytes equal the fused head followed by the video step
    (the same arithmetic), and stay within the head's tolerance of the oracle's bytes (at most 3
    codes: max|d| 1.6e-2 of the head's output times 127.5); sampled at full size."""
    N, D, H, W, Ci = shape
    _say("fused rgb head %s" % (shape,))
    if shape[1] == 16:
        x, w, b = si.make_inputs(si.WORKLOADS["c3"], device=DEV)
    else:
        x, w, b = si.random_case("3d", N, Ci, 12, H, W, D=D, dtype="bf16", seed=7, device=DEV)
    op = Conv3x3x3(w, b, N, D, H, W, epilogue="clamp1", algo=C.ALGO_FUSED_HEAD)
    rgb = op.rgb8(x)
    y = op(x)
    rgb2 = torch.empty_like(rgb)
    C.conv_video_rgb8(y, rgb2, N, D, H, W, 12, C.DTYPE_BF16)
    torch.cuda.synchronize()
    assert torch.equal(rgb, rgb2)
    if shape[1] == 16:
        from gpu_support import sample_points_3d
        pts = sample_points_3d(N, D, H, W, 400, seed=5)
        yref = oracle.conv3d_points(bits(x), bits(w), bits(b), pts, 1, oracle.BF16,
                                    oracle.EPI_CLAMP1, oracle.CHANNELS_LAST)
        qref = oracle.quantize_u8(oracle.decode(oracle.encode(yref, oracle.BF16), oracle.BF16))
        got = rgb.cpu().numpy()
        for i, (n_, d_, h_, w_) in enumerate(pts):
            for k in range(12):
                c, dy, dx = k // 4, (k // 2) % 2, k % 2
                assert abs(int(got[n_, d_, 2 * h_ + dy, 2 * w_ + dx, c]) - int(qref[i, k])) <= 3
    else:
        yref = oracle_3d(x, w, b, "clamp1")
        want = oracle.video_rgb8(oracle.decode(oracle.encode(yref, oracle.BF16), oracle.BF16))
        d = np.abs(rgb.cpu().numpy().astype(np.int32) - want.astype(np.int32))
        assert d.max() <= 3 and d.mean() < 0.05, (d.max(), d.mean())
