"""Pins of the oracle's video step (oracle/video.py): the quantisation against exact rational
arithmetic over every fp16 and bf16 bit pattern, the pixel shuffle against PyTorch's
pixel_shuffle, and the composition on a hand-checked example.  No GPU."""
from fractions import Fraction

import numpy as np
import torch

import oracle


def _exact_code(x: float) -> int:
    """clamp(round-half-even(127.5 * (x + 1)), 0, 255) in exact arithmetic; NaN -> 0."""
    if x != x:
        return 0
    if x == float("inf"):
        return 255
    if x == float("-inf"):
        return 0
    t = Fraction(255, 2) * (Fraction(x) + 1)
    return min(255, max(0, round(t)))          # Fraction.__round__ rounds half to even


def _all_values(dtype):
    bits = np.arange(65536, dtype=np.uint16)
    return oracle.decode(bits, dtype)           # exact fp64 values of every pattern


def test_quantize_matches_exact_arithmetic_bf16():
    v = _all_values(oracle.BF16)
    got = oracle.quantize_u8(v)
    want = np.array([_exact_code(float(x)) for x in v], np.uint8)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, (bad[:5], v[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_quantize_matches_exact_arithmetic_f16():
    v = _all_values(oracle.F16)
    got = oracle.quantize_u8(v)
    want = np.array([_exact_code(float(x)) for x in v], np.uint8)
    assert np.array_equal(got, want)


def test_quantize_landmarks():
    q = oracle.quantize_u8(np.array([-1.0, 1.0, 0.0, -0.5, 0.5, 2.0, -3.0, np.nan, 1e-30, -1e-30,
                                     -0.0, np.inf, -np.inf]))
    # 0 -> 127.5 ties to even 128; -0.5 -> 63.75 -> 64; 0.5 -> 191.25 -> 191
    assert q.tolist() == [0, 255, 128, 64, 191, 255, 0, 0, 128, 127, 128, 255, 0]


def test_pixel_shuffle_matches_torch():
    rng = np.random.default_rng(1)
    q = rng.integers(0, 256, size=(2, 3, 5, 7, 12), dtype=np.uint8)   # (N, D, H, W, 12)
    got = oracle.pixel_shuffle2_nhwc(q)
    t = torch.from_numpy(q.astype(np.int64)).reshape(6, 5, 7, 12).permute(0, 3, 1, 2)  # NCHW
    ref = torch.nn.functional.pixel_shuffle(t, 2).permute(0, 2, 3, 1).reshape(2, 3, 10, 14, 3)
    assert got.shape == (2, 3, 10, 14, 3)
    assert np.array_equal(got, ref.numpy().astype(np.uint8))


def test_video_rgb8_hand_example():
    """One position: channels 0..3 are the red sub-pixels (row-major over the 2x2 block),
    4..7 green, 8..11 blue."""
    y = np.array([-1, 1, 0, -0.5, 1, 1, 1, 1, -1, -1, -1, 0.5], np.float64).reshape(1, 1, 1, 1, 12)
    rgb = oracle.video_rgb8(y)
    assert rgb.shape == (1, 1, 2, 2, 3)
    assert rgb[0, 0].tolist() == [[[0, 255, 0], [255, 255, 0]],
                                  [[128, 255, 0], [64, 255, 191]]]


def test_single_fp32_rounding_is_exact_for_fp16_and_bf16():
    """The kernels code a value with one fp32 fused multiply-add (127.5*v + 127.5, rounded once),
    a round-half-even, the sign rule for a result of exactly 127.5, and a clamp.  Emulated here
    (the fp64 sum is exact or already at 127.5, so its fp32 rounding is the fma's): equal to the
    exact oracle for every fp16 and bf16 pattern."""
    for dt in (oracle.F16, oracle.BF16):
        v = _all_values(dt)
        with np.errstate(all="ignore"):
            t = (v * 127.5 + 127.5).astype(np.float32)
            q = np.rint(t).astype(np.float64)
            q = np.where((v < 0) & (t == np.float32(127.5)), 127.0, q)
            q = np.clip(np.where(np.isnan(q), 0.0, q), 0, 255).astype(np.uint8)
        assert np.array_equal(q, oracle.quantize_u8(v))
