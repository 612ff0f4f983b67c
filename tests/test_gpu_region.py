"""Parity of the 3D convolution over input regions (conv3x3x3_fwd_region) with the CPU oracle.

Each case builds a global tensor, runs the oracle's plain pad-1 convolution over it, and checks
that a region pass over a piece of that tensor reproduces the matching piece of the oracle's
output bit for bit (integer-valued inputs):

* row bands with halo rows: the band's input holds the global rows it needs plus ``halo`` rows
  each side; rows past the global height are filled with NaN and must never be read;
* causal temporal chunks: output frame t reads frames t-2 .. t of the whole sequence (zeros
  before frame 0); the oracle sees the sequence with one zero frame in front, so its output
  frame t is the causal one; a chunk carries up to two frames of the previous chunk;
* a NaN frame in front of the stored input, outside the valid frames (d_lo = 1).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from gpu_support import DEV, EPI, alloc_guarded, assert_bit_exact, check_guards, bits, odt
from x3x3_convolution_amd import conv as C
from x3x3_convolution_amd.plan import Conv3x3x3, band_rows, causal_frames

pytestmark = pytest.mark.gpu

NAN_BITS = {torch.bfloat16: 0x7FC0, torch.float16: 0x7E00}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _nan_like(t):
    return torch.full(t.shape, NAN_BITS[t.dtype], dtype=torch.int16, device=t.device).view(t.dtype)


def _oracle(x, w, b, epi):
    return oracle.conv3d(bits(x), bits(w), bits(b), 1, odt(x.dtype), EPI[epi], oracle.CHANNELS_LAST)


def _stored_rows(X, lo, rows, halo):
    """Global rows lo-halo .. lo+rows+halo-1 of X (N, D, Hg, W, C); rows outside [0, Hg) NaN."""
    Hg = X.shape[2]
    parts = []
    for r in range(lo - halo, lo + rows + halo):
        parts.append(X[:, :, r:r + 1] if 0 <= r < Hg else _nan_like(X[:, :, :1]))
    return torch.cat(parts, dim=2).contiguous()


def _run(op, x, D_in, H_in, d_org, h_org, d_lo, d_hi, h_lo, h_hi):
    buf, y = alloc_guarded(op.out_shape(), x.dtype)
    op.region(x, D_in, H_in, d_org, h_org, d_lo, d_hi, h_lo, h_hi, y=y)
    torch.cuda.synchronize()
    check_guards(buf, y.numel())
    return y


ALGOS = {
    # name: (C_in, C_out, dtype, algo)
    "mfma_w32": (32, 48, "bf16", C.ALGO_MFMA),
    "mfma_w32_f16_2mtiles": (16, 260, "f16", C.ALGO_MFMA),
    "mfma_narrow": (24, 12, "bf16", C.ALGO_MFMA),
    "fused_head": (64, 12, "bf16", C.ALGO_FUSED_HEAD),
    "fused_head_co7": (40, 7, "bf16", C.ALGO_FUSED_HEAD),
    "split_head": (32, 12, "bf16", C.ALGO_SPLIT_HEAD),
}


@pytest.mark.parametrize("name", list(ALGOS))
@pytest.mark.parametrize("lo,rows,halo", [(0, 7, 1), (5, 6, 1), (13, 7, 2), (0, 20, 1), (9, 2, 2)])
def test_row_band(name, lo, rows, halo):
    Ci, Co, dt, algo = ALGOS[name]
    N, D, Hg, W = 1, 3, 20, 130 if "head" in name else 40
    _say("region band %s lo=%d rows=%d halo=%d" % (name, lo, rows, halo))
    X, w, b = si.integer_case("3d", N, Ci, Co, Hg, W, D=D, dtype=dt, seed=lo * 7 + rows, device=DEV)
    want = _oracle(X, w, b, "clamp1")[:, :, lo:lo + rows]
    x = _stored_rows(X, lo, rows, halo)
    H_in, h_org, h_lo, h_hi = band_rows(lo, rows, halo, Hg)
    assert x.shape[2] == H_in
    op = Conv3x3x3(w, b, N, D, rows, W, epilogue="clamp1", algo=algo)
    y = _run(op, x, D, H_in, 0, h_org, 0, D, h_lo, h_hi)
    assert_bit_exact(y, want, x.dtype)


def _causal_reference(Xall, w, b, epi):
    """Causal temporal convolution of the whole sequence via the oracle: one zero frame in front
    makes the oracle's output frame t read frames t-2 .. t of the sequence."""
    z = torch.zeros_like(Xall[:, :1])
    return _oracle(torch.cat([z, Xall], dim=1).contiguous(), w, b, epi)[:, :Xall.shape[1]]


@pytest.mark.parametrize("name", list(ALGOS))
def test_causal_chunks(name):
    """A 9-frame sequence decoded in chunks of 4, 1 and 4 frames, each carrying the previous
    chunk's last two frames (or as many as exist), against the causal convolution of the whole
    sequence; the middle chunk also has a NaN frame in front, outside the valid frames."""
    Ci, Co, dt, algo = ALGOS[name]
    N, T, H, W = 2, 9, 11, 130 if "head" in name else 40
    epi = "relu" if Co > 12 else "clamp1"
    Xall, w, b = si.integer_case("3d", N, Ci, Co, H, W, D=T, dtype=dt, seed=5, device=DEV)
    want = _causal_reference(Xall, w, b, epi)
    t0 = 0
    for k, Dc in enumerate((4, 1, 4)):
        cached = min(2, t0)
        D_in, d_org, d_lo, d_hi = causal_frames(Dc, cached)
        x = Xall[:, t0 - cached:t0 + Dc].contiguous()
        if k == 1:   # a poisoned frame in front: shift the region by one
            x = torch.cat([_nan_like(x[:, :1]), x], dim=1).contiguous()
            D_in, d_org, d_lo, d_hi = D_in + 1, d_org + 1, d_lo + 1, d_hi + 1
        _say("region causal %s chunk %d frames %d..%d cached %d" % (name, k, t0, t0 + Dc, cached))
        op = Conv3x3x3(w, b, N, Dc, H, W, epilogue=epi, algo=algo)
        y = _run(op, x, D_in, H, d_org, 0, d_lo, d_hi, 0, H)
        assert_bit_exact(y, want[:, t0:t0 + Dc], x.dtype)
        t0 += Dc


@pytest.mark.parametrize("name", ["mfma_w32", "fused_head"])
def test_causal_chunk_of_a_row_band(name):
    """Both at once: rows [6, 14) of a 17-row frame with a 2-row halo, frames 3..6 of a causal
    sequence with two cached frames."""
    Ci, Co, dt, algo = ALGOS[name]
    N, T, Hg, W = 1, 7, 17, 130 if "head" in name else 40
    Xall, w, b = si.integer_case("3d", N, Ci, Co, Hg, W, D=T, dtype=dt, seed=9, device=DEV)
    want = _causal_reference(Xall, w, b, "none")[:, 3:7, 6:14]
    D_in, d_org, d_lo, d_hi = causal_frames(4, 2)
    H_in, h_org, h_lo, h_hi = band_rows(6, 8, 2, Hg)
    x = _stored_rows(Xall[:, 1:7].contiguous(), 6, 8, 2)
    _say("region causal band %s" % name)
    op = Conv3x3x3(w, b, N, 4, 8, W, epilogue="none", algo=algo)
    y = _run(op, x, D_in, H_in, d_org, h_org, d_lo, d_hi, h_lo, h_hi)
    assert_bit_exact(y, want, x.dtype)


def test_split_head_regions():
    """The split head on a causal chunk, a whole-height band (its plane needs no extra rows) and
    a band with data above and below it (its plane carries one more Z row each side)."""
    N, Ci, Co, T, H, W = 1, 32, 12, 6, 9, 50
    Xall, w, b = si.integer_case("3d", N, Ci, Co, H, W, D=T, dtype="bf16", seed=11, device=DEV)
    want = _causal_reference(Xall, w, b, "clamp1")
    D_in, d_org, d_lo, d_hi = causal_frames(4, 2)
    x = Xall[:, 0:6].contiguous()
    _say("region split head causal")
    op = Conv3x3x3(w, b, N, 4, H, W, epilogue="clamp1", algo=C.ALGO_SPLIT_HEAD)
    y = _run(op, x, D_in, H, d_org, 0, d_lo, d_hi, 0, H)
    assert_bit_exact(y, want[:, 2:6], x.dtype)
    # whole-height band with one (NaN) halo row each side
    xs = _stored_rows(x, 0, H, 1)
    H_in, h_org, h_lo, h_hi = band_rows(0, H, 1, H)
    y = _run(op, xs, D_in, H_in, d_org, h_org, d_lo, d_hi, h_lo, h_hi)
    assert_bit_exact(y, want[:, 2:6], x.dtype)
    # a band whose rows above and below hold data
    op2 = Conv3x3x3(w, b, N, 4, 4, W, epilogue="clamp1", algo=C.ALGO_SPLIT_HEAD)
    H_in, h_org, h_lo, h_hi = band_rows(3, 4, 1, H)
    y = _run(op2, _stored_rows(x, 3, 4, 1), D_in, H_in, d_org, h_org, d_lo, d_hi, h_lo, h_hi)
    assert_bit_exact(y, want[:, 2:6, 3:7], x.dtype)


def test_region_split_k():
    """A small position count makes the MFMA path split K over workgroups (fp32 partials in the
    workspace): the region reaches the split-K kernel too."""
    N, Ci, Co, T, Hg, W = 1, 256, 64, 4, 12, 8
    Xall, w, b = si.integer_case("3d", N, Ci, Co, Hg, W, D=T, dtype="bf16", seed=13, device=DEV)
    want = _causal_reference(Xall, w, b, "none")[:, 2:4, 4:8]
    op = Conv3x3x3(w, b, N, 2, 4, W, epilogue="none", algo=C.ALGO_MFMA)
    assert op.ws_bytes > 0, "expected a split-K plan"
    D_in, d_org, d_lo, d_hi = causal_frames(2, 2)
    H_in, h_org, h_lo, h_hi = band_rows(4, 4, 1, Hg)
    x = _stored_rows(Xall[:, 0:4].contiguous(), 4, 4, 1)
    _say("region split-K")
    y = _run(op, x, D_in, H_in, d_org, h_org, d_lo, d_hi, h_lo, h_hi)
    assert_bit_exact(y, want, x.dtype)


def test_region_stream_k():
    """The stream-K schedule (where the cost model sends 416 -> 300 channels over 5 frames of
    36 x 78): its stage order counts each output frame's live temporal taps in the region, so a
    causal first chunk (frames 0 and 1 with one and two taps) and a later chunk with two cached
    frames (three taps everywhere) divide differently; both on a band of rows at the bottom
    edge."""
    N, Ci, Co, T, Hg, W = 1, 416, 300, 10, 38, 78
    Xall, w, b = si.integer_case("3d", N, Ci, Co, Hg, W, D=T, dtype="bf16", seed=17, device=DEV)
    want = _causal_reference(Xall, w, b, "relu")
    lo, rows = 2, 36
    op = Conv3x3x3(w, b, N, 5, rows, W, epilogue="relu", algo=C.ALGO_AUTO)
    assert C.conv3x3x3_describe(N, Ci, Co, 5, rows, W).startswith("igemm32_sk ")
    H_in, h_org, h_lo, h_hi = band_rows(lo, rows, 1, Hg)
    for t0, cached in ((0, 0), (5, 2)):
        D_in, d_org, d_lo, d_hi = causal_frames(5, cached)
        x = _stored_rows(Xall[:, t0 - cached:t0 + 5].contiguous(), lo, rows, 1)
        _say("region stream-K frames %d..%d cached %d" % (t0, t0 + 5, cached))
        y = _run(op, x, D_in, H_in, d_org, h_org, d_lo, d_hi, h_lo, h_hi)
        assert_bit_exact(y, want[:, t0:t0 + 5, lo:lo + rows], x.dtype)


def test_full_region_equals_plain_call():
    """conv3x3x3_fwd_region over the full region is conv3x3x3_fwd, bit for bit (random inputs,
    AUTO algorithm: the fused head at C_out = 12)."""
    x, w, b = si.random_case("3d", 1, 64, 12, 33, 140, D=5, dtype="bf16", seed=3, device=DEV)
    op = Conv3x3x3(w, b, 1, 5, 33, 140, epilogue="clamp1")
    y0 = op(x)
    y1 = op.region(x, 5, 33, 0, 0, 0, 5, 0, 33)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y0), bits(y1))
