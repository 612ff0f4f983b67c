"""Host logic of input regions: the band and causal-chunk helpers produce region parameters
whose sum (the region formula of conv3x3x3_fwd_region, evaluated here by brute force in fp64)
equals the oracle's plain convolution of the global tensor on the matching output piece.  No GPU.
"""
import numpy as np
import pytest

import oracle
from x3x3_convolution_amd.plan import band_rows, causal_frames


def region_conv(x, w, b, D_out, H_out, d_org, h_org, d_lo, d_hi, h_lo, h_hi):
    """y[n,od,oh,ow,co] = b[co] + sum w[co,ci,kd,ky,kx] X[n, od+d_org-1+kd, oh+h_org-1+ky,
    ow-1+kx, ci], X = x inside frames [d_lo, d_hi), rows [h_lo, h_hi), columns [0, W), else 0.
    Positions outside the valid ranges are never read (they may hold NaN)."""
    N, D_in, H_in, W, Ci = x.shape
    Co = w.shape[0]
    y = np.zeros((N, D_out, H_out, W, Co))
    for od in range(D_out):
        for oh in range(H_out):
            for ow in range(W):
                acc = np.array(b, np.float64).copy()[None, :].repeat(N, 0)
                for kd in range(3):
                    f = od + d_org - 1 + kd
                    if not d_lo <= f < d_hi:
                        continue
                    for ky in range(3):
                        r = oh + h_org - 1 + ky
                        if not h_lo <= r < h_hi:
                            continue
                        for kx in range(3):
                            c = ow - 1 + kx
                            if not 0 <= c < W:
                                continue
                            acc += x[:, f, r, c, :] @ w[:, :, kd, ky, kx].T
                y[:, od, oh, ow, :] = acc
    return y


def plain(X, w, b):
    """The oracle's pad-1 convolution (fp64 values, no epilogue) of X (N, D, H, W, C_in)."""
    enc = lambda a: oracle.encode(a, oracle.BF16)
    return oracle.conv3d(enc(X), enc(w), enc(b), 1, oracle.BF16, oracle.EPI_NONE,
                         oracle.CHANNELS_LAST)


def _case(seed, N=1, T=5, H=7, W=4, Ci=2, Co=3):
    rng = np.random.default_rng(seed)
    q = lambda s: rng.integers(-3, 4, size=s).astype(np.float64)   # exact in bf16
    return q((N, T, H, W, Ci)), q((Co, Ci, 3, 3, 3)), q((Co,))


@pytest.mark.parametrize("lo,rows,halo", [(0, 3, 1), (2, 3, 1), (4, 3, 2), (0, 7, 1), (6, 1, 2)])
def test_band_rows_reproduce_the_global_convolution(lo, rows, halo):
    X, w, b = _case(lo + 10 * rows)
    Hg = X.shape[2]
    H_in, h_org, h_lo, h_hi = band_rows(lo, rows, halo, Hg)
    xs = np.full(X.shape[:2] + (H_in,) + X.shape[3:], np.nan)
    for k in range(H_in):
        g = lo - halo + k
        if 0 <= g < Hg:
            xs[:, :, k] = X[:, :, g]
    got = region_conv(xs, w, b, X.shape[1], rows, 0, h_org, 0, X.shape[1], h_lo, h_hi)
    np.testing.assert_array_equal(got, plain(X, w, b)[:, :, lo:lo + rows])


@pytest.mark.parametrize("t0,Dc", [(0, 3), (1, 2), (2, 3), (4, 1)])
def test_causal_frames_reproduce_the_causal_convolution(t0, Dc):
    X, w, b = _case(100 + t0)
    T = X.shape[1]
    # causal: output frame t reads frames t-2 .. t; a zero frame in front of the sequence
    # turns the plain pad-1 convolution's output frame t into exactly that
    causal = plain(np.concatenate([np.zeros_like(X[:, :1]), X], axis=1), w, b)[:, :T]
    cached = min(2, t0)
    D_in, d_org, d_lo, d_hi = causal_frames(Dc, cached)
    xs = X[:, t0 - cached:t0 + Dc]
    assert xs.shape[1] == D_in
    got = region_conv(xs, w, b, Dc, X.shape[2], d_org, 0, d_lo, d_hi, 0, X.shape[2])
    np.testing.assert_array_equal(got, causal[:, t0:t0 + Dc])


def test_causal_reference_is_causal():
    """The zero-frame construction: changing a frame changes no earlier output frame, and output
    frame t equals a hand sum over frames t-2 .. t at one position."""
    X, w, b = _case(7)
    T = X.shape[1]
    z = np.zeros_like(X[:, :1])
    y0 = plain(np.concatenate([z, X], axis=1), w, b)[:, :T]
    X2 = X.copy()
    X2[:, 3] += 1.0
    y1 = plain(np.concatenate([z, X2], axis=1), w, b)[:, :T]
    np.testing.assert_array_equal(y0[:, :3], y1[:, :3])
    assert not np.array_equal(y0[:, 3], y1[:, 3])
    t, h, c = 1, 3, 2
    want = b.copy()
    for kd in range(3):
        f = t - 2 + kd
        if f < 0:
            continue
        for ky in range(3):
            for kx in range(3):
                cc = c - 1 + kx
                if 0 <= cc < X.shape[3]:
                    want += w[:, :, kd, ky, kx] @ X[0, f, h - 1 + ky, cc]
    np.testing.assert_array_equal(y0[0, t, h, c], want)


def test_causal_frames_rejects_bad_cache():
    with pytest.raises(ValueError):
        causal_frames(3, 3)
