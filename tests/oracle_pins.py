"""The checks that pin the CPU oracle to facts fixed outside it: exact number-format conversions
by numpy/torch, closed forms, invariants of the convolution, special cases that reduce to a
library routine, and hand-worked examples under tests/golden/.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError on a mismatch.  They are run
against the real oracle by test_oracle_pins.py and against deliberately broken copies of it by
test_oracle_mutants.py (which shows that a plausible mistake fails at least one of them).
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch
import torch.nn.functional as F

F16, BF16 = 0, 1
CF, CL = 0, 1
NONE, RELU, CLAMP1 = 0, 1, 2

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def f16bits(a) -> np.ndarray:
    with np.errstate(over="ignore"):  # overflow to infinity is part of what is checked
        return np.ascontiguousarray(np.asarray(a, np.float64).astype(np.float16)).view(np.uint16)


def bf16bits(a) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.float32))).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bits_of(a, dtype):
    return f16bits(a) if dtype == F16 else bf16bits(a)


def small_values(rng, shape, scale=64):
    """Values k/scale with small integer k: exact in fp16 and bf16 (|k| <= 127)."""
    return rng.integers(-127, 128, size=shape).astype(np.float64) / scale


def epi_np(v, epi):
    if epi == RELU:
        return np.where(v < 0, 0.0, v)
    if epi == CLAMP1:
        return np.minimum(1.0, np.maximum(-1.0, v))
    return v


# ---------------------------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------------------------
def pin_decode_all_patterns(orc):
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref16 = allb.view(np.float16).astype(np.float64)
    got16 = orc.decode(allb, F16)
    nan16 = np.isnan(ref16)
    assert np.array_equal(np.isnan(got16), nan16)
    assert np.array_equal(got16[~nan16], ref16[~nan16])
    refbf = torch.from_numpy(allb.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    gotbf = orc.decode(allb, BF16)
    nanbf = np.isnan(refbf)
    assert np.array_equal(np.isnan(gotbf), nanbf)
    assert np.array_equal(gotbf[~nanbf], refbf[~nanbf])


def pin_encode_matches_libraries(orc):
    rng = np.random.default_rng(1)
    # fp16: numpy rounds fp64 -> binary16 directly, ties to even; magnitudes from deep subnormal
    # to past overflow.
    mag = np.exp2(rng.uniform(-27, 17, 20000))
    v = mag * rng.choice([-1.0, 1.0], mag.size)
    v = np.concatenate([v, [0.0, -0.0, 65504.0, 65519.0, 65520.0, 1e6, -1e6, 2.0 ** -25,
                            3 * 2.0 ** -26, 2.0 ** -24, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11]])
    assert np.array_equal(orc.encode(v, F16), f16bits(v))
    # bf16: torch rounds fp32 -> bf16 with ties to even; use fp32-exact inputs so that no
    # double rounding is involved on the library side.
    with np.errstate(over="ignore"):
        v32 = (np.exp2(rng.uniform(-140, 129, 20000)) * rng.choice([-1.0, 1.0], 20000)).astype(np.float32)
    v32 = v32[np.isfinite(v32)]
    extra = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 3.3895314e38, -0.0], np.float32)
    v32 = np.concatenate([v32, extra])
    assert np.array_equal(orc.encode(v32.astype(np.float64), BF16), bf16bits(v32))


def pin_encode_ties_by_hand(orc):
    # binary16 around 1.0: spacing 2^-10.  1 + 2^-11 is a tie -> even (1.0); 1 + 3*2^-11 -> up.
    assert orc.encode(np.array([1 + 2.0 ** -11]), F16)[0] == 0x3C00
    assert orc.encode(np.array([1 + 3 * 2.0 ** -11]), F16)[0] == 0x3C02
    # largest finite binary16 is 65504; 65520 is the tie with 65536 (= overflow) -> infinity
    assert orc.encode(np.array([65519.0]), F16)[0] == 0x7BFF
    assert orc.encode(np.array([65520.0]), F16)[0] == 0x7C00
    # bfloat16 around 1.0: spacing 2^-7
    assert orc.encode(np.array([1 + 2.0 ** -8]), BF16)[0] == 0x3F80
    assert orc.encode(np.array([1 + 3 * 2.0 ** -8]), BF16)[0] == 0x3F82
    assert orc.encode(np.array([-2.5]), BF16)[0] == 0xC020


# ---------------------------------------------------------------------------------------------
# convolution definition
# ---------------------------------------------------------------------------------------------
def pin_delta_2d(orc):
    """One-hot weight at (co=ci, ky, kx): y is x shifted by (ky-1, kx-1) with zero fill."""
    rng = np.random.default_rng(2)
    N, C, H, W = 2, 3, 5, 7
    x = small_values(rng, (N, C, H, W))
    xb = f16bits(x)
    for ky in range(3):
        for kx in range(3):
            w = np.zeros((C, C, 3, 3))
            for c in range(C):
                w[c, c, ky, kx] = 1.0
            y = orc.conv2d(xb, f16bits(w), None, 1, F16, NONE, CF)
            ref = np.zeros_like(x)
            for h in range(H):
                for ww in range(W):
                    ih, iw = h + ky - 1, ww + kx - 1
                    if 0 <= ih < H and 0 <= iw < W:
                        ref[:, :, h, ww] = x[:, :, ih, iw]
            assert np.array_equal(y, ref), (ky, kx)
            # the same through the channels-last layout
            yl = orc.conv2d(np.ascontiguousarray(xb.transpose(0, 2, 3, 1)), f16bits(w), None, 1,
                            F16, NONE, CL)
            assert np.array_equal(yl.transpose(0, 3, 1, 2), ref), (ky, kx, "NHWC")


def pin_delta_3d(orc):
    """One-hot weight at (co=ci, kd, ky, kx): a shift by (kd-1, ky-1, kx-1) with zero fill."""
    rng = np.random.default_rng(3)
    N, C, D, H, W = 1, 2, 4, 4, 5
    x = small_values(rng, (N, D, H, W, C))
    xb = bf16bits(x)
    for kd in range(3):
        for ky in range(3):
            for kx in range(3):
                w = np.zeros((C, C, 3, 3, 3))
                for c in range(C):
                    w[c, c, kd, ky, kx] = 1.0
                y = orc.conv3d(xb, bf16bits(w), None, 1, BF16, NONE, CL)
                ref = np.zeros_like(x)
                for d in range(D):
                    for h in range(H):
                        for ww in range(W):
                            i, j, k = d + kd - 1, h + ky - 1, ww + kx - 1
                            if 0 <= i < D and 0 <= j < H and 0 <= k < W:
                                ref[:, d, h, ww, :] = x[:, i, j, k, :]
                assert np.array_equal(y, ref), (kd, ky, kx)


def _count_valid(n, size, stride=1):
    """Number of taps t in {0,1,2} with 0 <= stride*n - 1 + t < size."""
    return sum(1 for t in range(3) if 0 <= stride * n - 1 + t < size)


def pin_ones_borders(orc):
    """x = 1, w = 1, no bias: the closed-form count of in-image taps times C_in --
    9/6/4 (2D interior/edge/corner), 27/18/12/8 (3D)."""
    C = 5
    for (H, W) in [(6, 7), (2, 3), (1, 4)]:
        x = f16bits(np.ones((1, C, H, W)))
        w = f16bits(np.ones((3, C, 3, 3)))
        y = orc.conv2d(x, w, None, 1, F16, NONE, CF)
        for h in range(H):
            for ww in range(W):
                assert np.all(y[0, :, h, ww] == C * _count_valid(h, H) * _count_valid(ww, W))
    y = orc.conv2d(f16bits(np.ones((1, C, 6, 7))), f16bits(np.ones((2, C, 3, 3))), None, 1, F16,
                   NONE, CF)
    assert y[0, 0, 2, 3] == 9 * C and y[0, 0, 0, 3] == 6 * C and y[0, 0, 0, 0] == 4 * C
    D, H, W = 4, 5, 6
    x = bf16bits(np.ones((1, D, H, W, C)))
    w = bf16bits(np.ones((2, C, 3, 3, 3)))
    y = orc.conv3d(x, w, None, 1, BF16, NONE, CL)
    for d in range(D):
        for h in range(H):
            for ww in range(W):
                exp = C * _count_valid(d, D) * _count_valid(h, H) * _count_valid(ww, W)
                assert np.all(y[0, d, h, ww, :] == exp)
    assert y[0, 1, 1, 1, 0] == 27 * C and y[0, 0, 1, 1, 0] == 18 * C
    assert y[0, 0, 0, 1, 0] == 12 * C and y[0, 0, 0, 0, 0] == 8 * C
    # stride 2 at odd and even sizes: output (oh, ow) covers input rows 2*oh-1 .. 2*oh+1
    for (H, W) in [(7, 8), (8, 7)]:
        y = orc.conv2d(f16bits(np.ones((1, C, H, W))), f16bits(np.ones((1, C, 3, 3))), None, 2,
                       F16, NONE, CF)
        assert y.shape == (1, 1, (H - 1) // 2 + 1, (W - 1) // 2 + 1)
        for oh in range(y.shape[2]):
            for ow in range(y.shape[3]):
                assert y[0, 0, oh, ow] == C * _count_valid(oh, H, 2) * _count_valid(ow, W, 2)


def pin_linearity(orc):
    """conv(a*x1 + b*x2) = a*conv(x1) + b*conv(x2); likewise in w (no bias, identity)."""
    rng = np.random.default_rng(4)
    x1 = rng.integers(-8, 9, (2, 3, 6, 5)).astype(np.float64)
    x2 = rng.integers(-8, 9, (2, 3, 6, 5)).astype(np.float64)
    w1 = small_values(rng, (4, 3, 3, 3), 16)
    w2 = small_values(rng, (4, 3, 3, 3), 16)
    for s in (1, 2):
        lhs = orc.conv2d(f16bits(2 * x1 - 3 * x2), f16bits(w1), None, s, F16, NONE, CF)
        rhs = (2 * orc.conv2d(f16bits(x1), f16bits(w1), None, s, F16, NONE, CF)
               - 3 * orc.conv2d(f16bits(x2), f16bits(w1), None, s, F16, NONE, CF))
        assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
        lhs = orc.conv2d(f16bits(x1), f16bits(w1 + w2), None, s, F16, NONE, CF)
        rhs = (orc.conv2d(f16bits(x1), f16bits(w1), None, s, F16, NONE, CF)
               + orc.conv2d(f16bits(x1), f16bits(w2), None, s, F16, NONE, CF))
        assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
    x1 = rng.integers(-4, 5, (1, 3, 4, 5, 2)).astype(np.float64)
    x2 = rng.integers(-4, 5, (1, 3, 4, 5, 2)).astype(np.float64)
    w = small_values(rng, (3, 2, 3, 3, 3), 16)
    lhs = orc.conv3d(bf16bits(x1 + 2 * x2), bf16bits(w), None, 1, BF16, NONE, CL)
    rhs = (orc.conv3d(bf16bits(x1), bf16bits(w), None, 1, BF16, NONE, CL)
           + 2 * orc.conv3d(bf16bits(x2), bf16bits(w), None, 1, BF16, NONE, CL))
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def pin_stride2_is_subsampled_stride1(orc):
    rng = np.random.default_rng(5)
    for (H, W) in [(8, 8), (7, 9), (1, 2), (2, 1)]:
        x = f16bits(small_values(rng, (2, 3, H, W)))
        w = f16bits(small_values(rng, (4, 3, 3, 3)))
        b = f16bits(small_values(rng, (4,)))
        y1 = orc.conv2d(x, w, b, 1, F16, RELU, CF)
        y2 = orc.conv2d(x, w, b, 2, F16, RELU, CF)
        assert y2.shape[2:] == ((H - 1) // 2 + 1, (W - 1) // 2 + 1)
        assert np.array_equal(y2, y1[:, :, ::2, ::2])
    x = bf16bits(small_values(rng, (1, 3, 7, 6, 2)))
    w = bf16bits(small_values(rng, (3, 2, 3, 3, 3)))
    y1 = orc.conv3d(x, w, None, 1, BF16, NONE, CL)
    y2 = orc.conv3d(x, w, None, 2, BF16, NONE, CL)
    assert np.array_equal(y2, y1[:, :, ::2, ::2, :])
    for n in range(1, 20):
        assert orc.out_size(n, 2) == (n - 1) // 2 + 1 and orc.out_size(n, 1) == n


def pin_split_equals_direct(orc):
    """The head split (temporal 3x1x1 conv into nine tap channels, then the nine-tap shifted
    sum) is algebraically the 27-tap convolution: equal in fp64 without the intermediate
    rounding.  With it, G is exactly the rounded unrounded plane."""
    rng = np.random.default_rng(6)
    for (Ci, Co, D, H, W) in [(4, 3, 3, 4, 5), (2, 12, 2, 3, 3), (3, 2, 1, 5, 4)]:
        x = bf16bits(rng.standard_normal((1, D, H, W, Ci)))
        w = bf16bits(rng.standard_normal((Co, Ci, 3, 3, 3)) * 0.2)
        b = bf16bits(rng.standard_normal((Co,)) * 0.3)
        for epi in (NONE, CLAMP1):
            yd = orc.conv3d(x, w, b, 1, BF16, epi, CL)
            ys, g = orc.head_split(x, w, b, BF16, epi, CL, round_g=False, return_g=True)
            assert np.allclose(ys, yd, rtol=1e-12, atol=1e-12)
        yr, gr = orc.head_split(x, w, b, BF16, CLAMP1, CL, round_g=True, return_g=True)
        assert np.array_equal(gr, orc.decode(orc.encode(g, BF16), BF16))
        # G's channel (ky*3+kx)*C_out+co at (d,h,w) is the temporal sum of tap (ky,kx):
        # a one-hot weight at (co, ci, kd, ky, kx) puts x[d-1+kd, h, w, ci] there.
        wd = np.zeros((Co, Ci, 3, 3, 3))
        wd[Co - 1, 0, 2, 0, 1] = 1.0
        _, g1 = orc.head_split(x, bf16bits(wd), None, BF16, NONE, CL, return_g=True)
        xv = orc.decode(x, BF16)
        exp = np.zeros((1, D, H, W))
        exp[:, :D - 1] = xv[:, 1:, :, :, 0]
        assert np.array_equal(g1[..., (0 * 3 + 1) * Co + Co - 1], exp)
        assert np.count_nonzero(g1) == np.count_nonzero(exp)


def pin_depth1_is_2d_centre_slice(orc):
    rng = np.random.default_rng(7)
    x2 = small_values(rng, (2, 5, 6, 3))              # NHWC
    w3 = small_values(rng, (4, 3, 3, 3, 3))
    b = small_values(rng, (4,))
    y3 = orc.conv3d(bf16bits(x2[:, None]), bf16bits(w3), bf16bits(b), 1, BF16, CLAMP1, CL)
    y2 = orc.conv2d(bf16bits(x2), bf16bits(w3[:, :, 1]), bf16bits(b), 1, BF16, CLAMP1, CL)
    assert np.array_equal(y3[:, 0], y2)


def pin_kd_only_is_per_frame_2d(orc):
    rng = np.random.default_rng(8)
    x = small_values(rng, (1, 4, 5, 6, 3))
    w3 = np.zeros((2, 3, 3, 3, 3))
    w3[:, :, 1] = small_values(rng, (2, 3, 3, 3))
    y3 = orc.conv3d(bf16bits(x), bf16bits(w3), None, 1, BF16, NONE, CL)
    for d in range(4):
        y2 = orc.conv2d(bf16bits(x[:, d]), bf16bits(w3[:, :, 1]), None, 1, BF16, NONE, CL)
        assert np.array_equal(y3[:, d], y2)


def pin_bias_and_epilogues(orc):
    """w = 0: y = E(bias) everywhere; E = identity / ReLU (negative -> 0) / clamp to [-1,1]."""
    b = np.array([-2.5, -0.75, 0.0, 0.5, 1.25, 3.0])
    x = f16bits(np.ones((1, 2, 3, 4)))
    w = f16bits(np.zeros((6, 2, 3, 3)))
    for epi, exp in [(NONE, b), (RELU, np.maximum(b, 0)), (CLAMP1, np.clip(b, -1, 1))]:
        y = orc.conv2d(x, w, f16bits(b), 1, F16, epi, CF)
        assert np.array_equal(y, np.broadcast_to(exp[None, :, None, None], y.shape))
        y3 = orc.conv3d(bf16bits(np.ones((1, 2, 3, 3, 2))), bf16bits(np.zeros((6, 2, 3, 3, 3))),
                        bf16bits(b), 1, BF16, epi, CL)
        assert np.array_equal(y3, np.broadcast_to(exp, y3.shape))
    y = orc.conv2d(x, w, None, 1, F16, NONE, CF)
    assert np.all(y == 0)


def pin_torch_float64(orc):
    """Tiny random shapes against torch's float64 CPU convolution (padding 1, no flip)."""
    rng = np.random.default_rng(9)
    for (N, Ci, Co, H, W, s, epi, dt) in [(2, 3, 4, 7, 9, 1, RELU, F16), (1, 5, 2, 6, 5, 2, NONE, F16),
                                          (1, 2, 3, 5, 5, 2, CLAMP1, BF16), (3, 1, 1, 1, 3, 1, NONE, BF16)]:
        xb = bits_of(rng.standard_normal((N, Ci, H, W)), dt)
        wb = bits_of(rng.standard_normal((Co, Ci, 3, 3)) * 0.3, dt)
        bb = bits_of(rng.standard_normal((Co,)) * 0.3, dt)
        y = orc.conv2d(xb, wb, bb, s, dt, epi, CF)
        ref = F.conv2d(torch.from_numpy(orc.decode(xb, dt)), torch.from_numpy(orc.decode(wb, dt)),
                       torch.from_numpy(orc.decode(bb, dt)), stride=s, padding=1).numpy()
        assert np.allclose(y, epi_np(ref, epi), rtol=1e-12, atol=1e-12)
    for (N, Ci, Co, D, H, W, s, epi) in [(1, 3, 5, 4, 5, 6, 1, NONE), (2, 2, 3, 3, 4, 3, 1, CLAMP1),
                                         (1, 2, 2, 2, 7, 6, 2, RELU)]:
        x = rng.standard_normal((N, D, H, W, Ci))
        xb = bf16bits(x)
        wb = bf16bits(rng.standard_normal((Co, Ci, 3, 3, 3)) * 0.2)
        bb = bf16bits(rng.standard_normal((Co,)) * 0.3)
        y = orc.conv3d(xb, wb, bb, s, BF16, epi, CL)
        xt = torch.from_numpy(orc.decode(xb, BF16)).permute(0, 4, 1, 2, 3)
        ref = F.conv3d(xt, torch.from_numpy(orc.decode(wb, BF16)),
                       torch.from_numpy(orc.decode(bb, BF16)), stride=(1, s, s),
                       padding=1).permute(0, 2, 3, 4, 1).numpy()
        assert np.allclose(y, epi_np(ref, epi), rtol=1e-12, atol=1e-12)
        # NCDHW layout gives the same numbers
        yc = orc.conv3d(np.ascontiguousarray(xb.transpose(0, 4, 1, 2, 3)), wb, bb, s, BF16, epi, CF)
        assert np.array_equal(yc.transpose(0, 2, 3, 4, 1), y)


def pin_numpy_im2col(orc):
    """2D as an explicit patch matrix times the flattened weight (numpy, float64)."""
    rng = np.random.default_rng(10)
    N, Ci, Co, H, W = 2, 4, 3, 6, 7
    for s in (1, 2):
        xb = f16bits(rng.standard_normal((N, Ci, H, W)))
        wb = f16bits(rng.standard_normal((Co, Ci, 3, 3)) * 0.3)
        x = orc.decode(xb, F16)
        w = orc.decode(wb, F16)
        xp = np.pad(x, ((0, 0), (0, 0), (1, 1), (1, 1)))
        Ho, Wo = (H - 1) // s + 1, (W - 1) // s + 1
        cols = np.empty((N, Ho, Wo, Ci, 3, 3))
        for oh in range(Ho):
            for ow in range(Wo):
                cols[:, oh, ow] = xp[:, :, s * oh:s * oh + 3, s * ow:s * ow + 3]
        ref = (cols.reshape(N * Ho * Wo, -1) @ w.reshape(Co, -1).T).reshape(N, Ho, Wo, Co)
        y = orc.conv2d(xb, wb, None, s, F16, NONE, CF)
        assert np.allclose(y, ref.transpose(0, 3, 1, 2), rtol=1e-12, atol=1e-12)


def pin_points_match_full(orc):
    rng = np.random.default_rng(11)
    xb = bf16bits(rng.standard_normal((2, 3, 5, 6, 4)))
    wb = bf16bits(rng.standard_normal((3, 4, 3, 3, 3)) * 0.2)
    bb = bf16bits(rng.standard_normal((3,)))
    for s in (1, 2):
        y = orc.conv3d(xb, wb, bb, s, BF16, CLAMP1, CL)
        pts = np.array([[n, d, h, w] for n in range(2) for d in range(3)
                        for h in range(y.shape[2]) for w in range(y.shape[3])], np.int32)
        yp = orc.conv3d_points(xb, wb, bb, pts, s, BF16, CLAMP1, CL)
        assert np.array_equal(yp, y.reshape(-1, 3))
    xb = f16bits(rng.standard_normal((2, 3, 5, 6)))
    wb = f16bits(rng.standard_normal((4, 3, 3, 3)) * 0.2)
    for s in (1, 2):
        y = orc.conv2d(xb, wb, None, s, F16, RELU, CF)
        pts = np.array([[n, h, w] for n in range(2) for h in range(y.shape[2])
                        for w in range(y.shape[3])], np.int32)
        yp = orc.conv2d_points(xb, wb, None, pts, s, F16, RELU, CF)
        assert np.array_equal(yp, y.transpose(0, 2, 3, 1).reshape(-1, 4))


def pin_golden(orc):
    """Hand-worked examples (tests/golden/*.json; each file states its derivation)."""
    names = sorted(f for f in os.listdir(GOLDEN) if f.endswith(".json"))
    assert names, "no golden fixtures found"
    for name in names:
        with open(os.path.join(GOLDEN, name)) as fh:
            case = json.load(fh)
        dt = F16 if case["dtype"] == "f16" else BF16
        epi = {"none": NONE, "relu": RELU, "clamp1": CLAMP1}[case["epilogue"]]
        x = bits_of(np.array(case["x"], np.float64), dt)
        w = bits_of(np.array(case["w"], np.float64), dt)
        b = bits_of(np.array(case["b"], np.float64), dt) if case.get("b") is not None else None
        exp = np.array(case["y"], np.float64)
        if case["op"] == "conv2d":
            y = orc.conv2d(x, w, b, case["stride"], dt, epi, CF)
        elif case["op"] == "conv3d":
            y = orc.conv3d(x, w, b, case["stride"], dt, epi, CF)
        else:
            y = orc.head_split(x, w, b, dt, epi, CF)
        assert y.shape == exp.shape, name
        assert np.array_equal(y, exp), name


ALL_PINS = [
    pin_decode_all_patterns, pin_encode_matches_libraries, pin_encode_ties_by_hand,
    pin_delta_2d, pin_delta_3d, pin_ones_borders, pin_linearity, pin_stride2_is_subsampled_stride1,
    pin_split_equals_direct, pin_depth1_is_2d_centre_slice, pin_kd_only_is_per_frame_2d,
    pin_bias_and_epilogues, pin_torch_float64, pin_numpy_im2col, pin_points_match_full, pin_golden,
]
