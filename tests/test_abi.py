"""The C ABI on the host: the library loads, exports every entry point its header declares, and
rejects every invalid request before it enqueues anything.  No compute calls (no GPU needed);
fake device addresses are only passed on paths that fail validation or return before a launch.
"""
import ctypes
import os
import re

import pytest
import torch

import x3x3_convolution_amd as cx
from x3x3_convolution_amd import conv as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "conv3x3.h")

A = 1 << 20           # a fake, 16-byte aligned "device address" (never dereferenced)
B = 1 << 30
WS = 1 << 34
HAS_GPU = torch.cuda.device_count() > 0


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(conv\w*)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = cx.library()
    declared = header_functions()
    assert len(declared) >= 12
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(n for n, _, _ in C.EXPORTS) == declared


def test_version_and_status_strings():
    assert cx.conv_abi_version() == C.ABI_VERSION == 1
    for st in (C.OK, C.E_INVAL, C.E_UNSUPPORTED, C.E_WORKSPACE, C.E_NODEVICE, C.E_LAUNCH):
        assert cx.conv_status_str(st) not in ("", "unknown status")
    assert cx.conv_status_str(12345) == "unknown status"


def test_out_size():
    for n in range(0, 40):
        for s in (1, 2):
            assert cx.conv_out_size(n, s) == (0 if n == 0 else (n - 1) // s + 1)
    assert cx.conv_out_size(256, 2) == 128 and cx.conv_out_size(255, 2) == 128
    assert cx.conv_out_size(-1, 1) == -1 and cx.conv_out_size(5, 3) == -1


def _st(fn, *a):
    try:
        fn(*a)
    except C.ConvError as e:
        return e.status
    return C.OK


def f2d(**kw):
    a = dict(x=A, w=B, bias=None, y=A + (1 << 28), N=1, C_in=16, C_out=16, H=8, W=8, stride=1,
             layout=0, dtype=0, epilogue=1, algo=0, stream=0)
    a.update(kw)
    return _st(cx.conv3x3_fwd, a["x"], a["w"], a["bias"], a["y"], a["N"], a["C_in"], a["C_out"],
               a["H"], a["W"], a["stride"], a["layout"], a["dtype"], a["epilogue"], a["algo"],
               a["stream"])


def f3d(**kw):
    a = dict(x=A, w=B, bias=None, y=A + (1 << 28), N=1, C_in=32, C_out=12, D=2, H=8, W=8,
             stride=1, layout=1, dtype=1, epilogue=2, algo=C.ALGO_MFMA, ws=None, wsb=0,
             stream=0)
    a.update(kw)
    return _st(cx.conv3x3x3_fwd, a["x"], a["w"], a["bias"], a["y"], a["N"], a["C_in"],
               a["C_out"], a["D"], a["H"], a["W"], a["stride"], a["layout"], a["dtype"],
               a["epilogue"], a["algo"], a["ws"], a["wsb"], a["stream"])


def test_2d_invalid_arguments():
    assert f2d(x=None) == C.E_INVAL
    assert f2d(w=None) == C.E_INVAL
    assert f2d(y=None) == C.E_INVAL
    assert f2d(stride=3) == C.E_INVAL
    assert f2d(stride=0) == C.E_INVAL
    assert f2d(dtype=7) == C.E_INVAL
    assert f2d(epilogue=3) == C.E_INVAL
    assert f2d(layout=5) == C.E_INVAL
    assert f2d(algo=9) == C.E_INVAL
    assert f2d(N=-1) == C.E_INVAL
    assert f2d(C_in=0) == C.E_INVAL
    assert f2d(x=A + 2) == C.E_INVAL            # misaligned
    assert f2d(bias=A + 1) == C.E_INVAL         # misaligned bias
    assert f2d(y=A + 64) == C.E_INVAL           # overlaps x
    assert "overlap" in cx.conv_last_error()
    # NHWC runs on the matrix-core kernel only: C_in a multiple of 8 up to 64, C_out up to 64
    assert f2d(layout=1, algo=C.ALGO_SIMT) == C.E_UNSUPPORTED
    assert f2d(layout=1, C_in=12) == C.E_UNSUPPORTED
    assert f2d(layout=1, C_out=65) == C.E_UNSUPPORTED
    assert f2d(layout=1, C_in=72) == C.E_UNSUPPORTED
    assert f2d(algo=C.ALGO_MFMA, C_in=12) == C.E_UNSUPPORTED     # C_in not a multiple of 8
    assert f2d(algo=C.ALGO_MFMA, C_in=72) == C.E_UNSUPPORTED     # C_in above 64
    assert f2d(algo=C.ALGO_MFMA, C_out=65) == C.E_UNSUPPORTED
    assert f2d(algo=C.ALGO_MFMA, W=12) == C.E_UNSUPPORTED        # W not a multiple of 8
    assert f2d(algo=C.ALGO_SPLIT_HEAD) == C.E_UNSUPPORTED


def test_2d_empty_is_noop():
    for kw in (dict(N=0), dict(C_out=0), dict(H=0), dict(W=0)):
        assert f2d(x=None, y=None, **kw) == C.OK


def test_3d_invalid_and_unsupported():
    assert f3d(x=None) == C.E_INVAL
    assert f3d(w=None) == C.E_INVAL
    assert f3d(y=None) == C.E_INVAL
    assert f3d(epilogue=-1) == C.E_INVAL
    assert f3d(algo=17) == C.E_INVAL
    assert f3d(D=-2) == C.E_INVAL
    assert f3d(C_in=0) == C.E_INVAL
    assert f3d(y=A + 16) == C.E_INVAL
    assert f3d(w=B + 8) == C.E_INVAL
    assert f3d(layout=0) == C.E_UNSUPPORTED     # NCDHW
    assert f3d(stride=2, algo=C.ALGO_FUSED_HEAD) == C.E_UNSUPPORTED   # heads: stride 1 only
    assert f3d(stride=2, algo=C.ALGO_SPLIT_HEAD) == C.E_UNSUPPORTED
    assert f3d(C_in=20) == C.E_UNSUPPORTED      # not a multiple of 8
    assert f3d(algo=C.ALGO_SIMT) == C.E_UNSUPPORTED
    assert f3d(algo=C.ALGO_SPLIT_HEAD, C_out=13) == C.E_UNSUPPORTED
    assert f3d(algo=C.ALGO_FUSED_HEAD, C_out=13) == C.E_UNSUPPORTED
    # a workgroup's six input frames must stay below 2 GiB for the head kernels' buffer
    # addressing (the number of frames does not matter)
    assert cx.conv3x3x3_is_supported(1, 256, 12, 32, 352, 624, 1, 1, 1, 2, C.ALGO_FUSED_HEAD) == C.OK
    assert cx.conv3x3x3_is_supported(1, 256, 12, 1, 1400, 1024, 1, 1, 1, 2, C.ALGO_FUSED_HEAD) == C.E_UNSUPPORTED
    assert cx.conv3x3x3_select_algo(1, 256, 12, 1, 1400, 1024, 1, 1, 1, 0) == C.ALGO_MFMA
    # the split head needs its plane in the workspace
    assert f3d(algo=C.ALGO_SPLIT_HEAD) == C.E_WORKSPACE
    need = cx.conv3x3x3_workspace_bytes(1, 32, 12, 2, 8, 8, 1, 1, 1, C.ALGO_SPLIT_HEAD)
    assert need == 2 * (8 + 2) * 8 * 112 * 2   # one plane row above and below the output rows
    assert f3d(algo=C.ALGO_SPLIT_HEAD, ws=WS, wsb=need - 1) == C.E_WORKSPACE
    assert f3d(algo=C.ALGO_SPLIT_HEAD, ws=WS + 4, wsb=need) == C.E_INVAL   # misaligned
    assert f3d(algo=C.ALGO_SPLIT_HEAD, ws=A, wsb=need) == C.E_INVAL        # overlaps x


def test_3d_empty_is_noop():
    for kw in (dict(N=0), dict(C_out=0), dict(D=0), dict(H=0), dict(W=0)):
        assert f3d(x=None, y=None, w=None, **kw) == C.OK
        assert f3d(x=None, y=None, w=None, stride=2, **kw) == C.OK


def test_2d_algo_selection():
    assert cx.conv3x3_select_algo(8, 64, 64, 256, 256, 1, 0, 0, C.ALGO_AUTO) == C.ALGO_MFMA
    assert cx.conv3x3_select_algo(8, 64, 64, 256, 256, 2, 0, 0, C.ALGO_AUTO) == C.ALGO_MFMA
    assert cx.conv3x3_select_algo(1, 16, 16, 64, 64, 1, 0, 0, C.ALGO_AUTO) == C.ALGO_MFMA
    assert cx.conv3x3_select_algo(2, 5, 7, 13, 37, 1, 0, 0, C.ALGO_AUTO) == C.ALGO_SIMT
    assert cx.conv3x3_select_algo(1, 64, 128, 32, 32, 1, 0, 0, C.ALGO_AUTO) == C.ALGO_SIMT
    assert cx.conv3x3_select_algo(8, 64, 64, 256, 256, 1, 0, 0, C.ALGO_SIMT) == C.ALGO_SIMT
    assert cx.conv3x3_is_supported(8, 64, 64, 256, 256, 1, 0, 0, 1, C.ALGO_MFMA) == C.OK
    assert cx.conv3x3_is_supported(1, 8, 8, 8, 20, 1, 0, 0, 1, C.ALGO_MFMA) == C.E_UNSUPPORTED
    with pytest.raises(C.ConvError):
        cx.conv3x3_select_algo(1, 8, 8, 8, 20, 1, 0, 0, C.ALGO_MFMA)
    # NHWC: always the matrix-core kernel, any width
    assert cx.conv3x3_select_algo(2, 8, 7, 13, 37, 1, 1, 0, C.ALGO_AUTO) == C.ALGO_MFMA
    with pytest.raises(C.ConvError):
        cx.conv3x3_select_algo(2, 8, 7, 13, 37, 1, 1, 0, C.ALGO_SIMT)
    with pytest.raises(C.ConvError):
        cx.conv3x3_select_algo(2, 5, 7, 13, 37, 1, 1, 0, C.ALGO_AUTO)
    # one image of x (64 x 4096 x W fp16) just below and just above 2 GiB: the matrix-core kernel
    # addresses an image through one 32-bit range, so past it AUTO falls back to SIMT (which takes
    # any size) and an explicit MFMA request is refused
    assert 64 * 4096 * 4088 * 2 < 1 << 31 <= 64 * 4096 * 4104 * 2
    assert cx.conv3x3_select_algo(3, 64, 64, 4096, 4088, 1, 0, 0, C.ALGO_AUTO) == C.ALGO_MFMA
    assert cx.conv3x3_select_algo(3, 64, 64, 4096, 4104, 1, 0, 0, C.ALGO_AUTO) == C.ALGO_SIMT
    assert cx.conv3x3_is_supported(3, 64, 64, 4096, 4104, 1, 0, 0, 1, C.ALGO_MFMA) == C.E_UNSUPPORTED


def test_is_supported_matches_fwd_checks():
    assert cx.conv3x3_is_supported(8, 64, 64, 256, 256, 2, 0, 0, 1, 0) == C.OK
    assert cx.conv3x3_is_supported(8, 64, 64, 256, 256, 2, 1, 0, 1, 0) == C.OK   # NHWC
    assert cx.conv3x3_is_supported(8, 64, 64, 256, 256, 2, 1, 0, 1, C.ALGO_SIMT) == C.E_UNSUPPORTED
    assert cx.conv3x3x3_is_supported(1, 256, 12, 16, 352, 624, 1, 1, 1, 2, 0) == C.OK
    assert cx.conv3x3x3_is_supported(1, 256, 12, 16, 352, 624, 1, 1, 1, 2, C.ALGO_SPLIT_HEAD) == C.OK
    assert cx.conv3x3x3_is_supported(1, 256, 256, 16, 176, 312, 1, 1, 1, 0, C.ALGO_SPLIT_HEAD) == C.E_UNSUPPORTED
    assert cx.conv3x3x3_is_supported(1, 256, 256, 16, 176, 312, 2, 1, 1, 0, 0) == C.OK   # stride 2
    assert cx.conv3x3x3_is_supported(1, 256, 12, 16, 176, 312, 2, 1, 1, 2, C.ALGO_FUSED_HEAD) == C.E_UNSUPPORTED


def test_algo_selection_and_buffer_sizes():
    # the output head: AUTO resolves to a concrete algorithm; split head needs its plane
    a = cx.conv3x3x3_select_algo(1, 256, 12, 16, 352, 624, 1, 1, 1, 0)
    assert a == C.ALGO_FUSED_HEAD
    assert cx.conv3x3x3_workspace_bytes(1, 256, 12, 16, 352, 624, 1, 1, 1, 0) == 0
    assert cx.conv3x3x3_select_algo(1, 256, 256, 16, 176, 312, 1, 1, 1, 0) == C.ALGO_MFMA
    assert cx.conv3x3x3_workspace_bytes(1, 256, 12, 16, 352, 624, 1, 1, 1,
                                        C.ALGO_SPLIT_HEAD) == 16 * 354 * 624 * 112 * 2
    # packed weights: 8 channel chunks x 27 taps x 16 rows x 32 (direct head)
    assert cx.conv3x3x3_packed_weight_bytes(1, 256, 12, 16, 352, 624, 1, 1, 1,
                                            C.ALGO_MFMA) == 8 * 27 * 16 * 32 * 2
    # split head: 8 chunks x 3 temporal taps x 128 rows (108 used) x 32; the fused head keeps
    # three row versions of each chunk
    assert cx.conv3x3x3_packed_weight_bytes(1, 256, 12, 16, 352, 624, 1, 1, 1,
                                            C.ALGO_SPLIT_HEAD) == 8 * 3 * 128 * 32 * 2
    assert cx.conv3x3x3_packed_weight_bytes(1, 256, 12, 16, 352, 624, 1, 1, 1,
                                            C.ALGO_FUSED_HEAD) == 3 * 8 * 3 * 128 * 32 * 2
    # mid-decoder conv fills the chip without split-K: no workspace
    assert cx.conv3x3x3_workspace_bytes(1, 256, 256, 16, 176, 312, 1, 1, 1, 0) == 0
    # the small low-res conv: one round of 240 half-size (128-position) tiles would wait for
    # the interior frames' three temporal taps, so 240 stream-K workgroups share the stages:
    # two 128 KiB partial slots per workgroup, then one counter per tile (60 tiles x 4 frames)
    assert cx.conv3x3x3_workspace_bytes(1, 512, 512, 4, 44, 78, 1, 1, 1, 0) == (
        240 * 2 * 256 * 128 * 4 + 60 * 4 * 4)
    # its first causal frame alone splits K over the four waves of each workgroup: no workspace
    assert cx.conv3x3x3_workspace_bytes(1, 512, 512, 1, 44, 78, 1, 1, 1, 0) == 0
    # fewer input channels over the same frame split K over workgroups: fp32 partials
    ws = cx.conv3x3x3_workspace_bytes(1, 264, 96, 1, 44, 78, 1, 1, 1, 0)
    assert ws > 0 and ws % (44 * 78 * 96 * 4) == 0
    assert cx.conv3x3x3_workspace_bytes(1, 512, 512, 4, 44, 78, 1, 1, 1, 9) == 0  # invalid
    assert cx.conv3x3x3_packed_weight_bytes(1, 20, 12, 1, 4, 4, 1, 1, 1, 0) == 0  # unsupported
    # spatial stride 2: AUTO is the MFMA path (the 32x32 family, 256 packed rows, even for the
    # head's 12 channels); the split-K partials cover the output positions
    assert cx.conv3x3x3_select_algo(1, 256, 12, 16, 352, 624, 2, 1, 1, 0) == C.ALGO_MFMA
    assert cx.conv3x3x3_packed_weight_bytes(1, 256, 12, 16, 352, 624, 2, 1, 1, 0) == 8 * 27 * 256 * 32 * 2
    ws = cx.conv3x3x3_workspace_bytes(1, 64, 5, 1, 9, 9, 2, 1, 1, 0)
    assert ws > 0 and ws % (5 * 5 * 5 * 4) == 0


def test_pack_invalid():
    st = _st(cx.conv3x3x3_pack_weights, None, B, 1, 32, 12, 2, 8, 8, 1, 1, 1, 0, 0)
    assert st == C.E_INVAL
    st = _st(cx.conv3x3x3_pack_weights, A, B + 8, 1, 32, 12, 2, 8, 8, 1, 1, 1, 0, 0)
    assert st == C.E_INVAL
    st = _st(cx.conv3x3x3_pack_weights, A, A, 1, 32, 12, 2, 8, 8, 1, 1, 1, 0, 0)
    assert st == C.E_INVAL


@pytest.mark.skipif(HAS_GPU, reason="checks the no-device path; a GPU is visible")
def test_no_device_reported_after_validation():
    assert f2d() == C.E_NODEVICE
    assert f3d(stride=2) == C.E_NODEVICE           # spatial stride 2 on the MFMA path
    assert f2d(layout=1) == C.E_NODEVICE           # NHWC
    assert f2d(layout=1, W=13, stride=2) == C.E_NODEVICE   # NHWC takes any width
    assert f3d() == C.E_NODEVICE
    assert "device" in cx.conv_last_error()


def f3r(**kw):
    """conv3x3x3_fwd_region with a valid default region: output (1, 4, 6, 8, 12) of a band
    of rows [2, 8) with one halo row each side (H_in = 8) and two cached frames (D_in = 6)."""
    a = dict(x=A, w=B, bias=None, y=A + (1 << 28), N=1, C_in=32, C_out=12, D_in=6, H_in=8, W=8,
             D_out=4, H_out=6, d_org=1, h_org=1, d_lo=0, d_hi=6, h_lo=0, h_hi=8, layout=1,
             dtype=1, epilogue=2, algo=C.ALGO_FUSED_HEAD, ws=None, wsb=0, stream=0)
    a.update(kw)
    return _st(cx.conv3x3x3_fwd_region, *[a[k] for k in (
        "x", "w", "bias", "y", "N", "C_in", "C_out", "D_in", "H_in", "W", "D_out", "H_out",
        "d_org", "h_org", "d_lo", "d_hi", "h_lo", "h_hi", "layout", "dtype", "epilogue", "algo",
        "ws", "wsb", "stream")])


def test_region_invalid_and_unsupported():
    assert f3r(x=None) == C.E_INVAL
    assert f3r(D_in=-1) == C.E_INVAL
    assert f3r(d_lo=-1) == C.E_INVAL
    assert f3r(d_hi=7) == C.E_INVAL              # past D_in
    assert f3r(d_lo=4, d_hi=3) == C.E_INVAL
    assert f3r(h_hi=9) == C.E_INVAL              # past H_in
    assert f3r(h_lo=5, h_hi=4) == C.E_INVAL
    # every output frame must read a valid frame
    assert f3r(d_lo=3) == C.E_UNSUPPORTED       # frame 0 reads 0..2 only
    assert f3r(d_hi=3) == C.E_UNSUPPORTED       # frame 3 reads 3..5 only
    assert f3r(d_lo=2, d_hi=2) == C.E_UNSUPPORTED
    assert f3r(d_org=4) == C.E_UNSUPPORTED       # frame 3 reads 6..8 only
    assert f3r(d_org=-2) == C.E_UNSUPPORTED      # frame 0 reads -3..-1 only
    assert f3r(algo=C.ALGO_SIMT) == C.E_UNSUPPORTED
    assert f3r(C_in=20) == C.E_UNSUPPORTED
    assert f3r(y=A + 16) == C.E_INVAL           # overlaps x (x is 6*8*8*32*2 bytes)
    # the split head's plane carries a row above and below the band: the workspace covers it
    ws = cx.conv3x3x3_workspace_bytes(1, 32, 12, 4, 6, 8, 1, 1, 1, C.ALGO_SPLIT_HEAD)
    assert ws == 4 * (6 + 2) * 8 * 112 * 2
    expect = C.OK if HAS_GPU else C.E_NODEVICE
    assert f3r(algo=C.ALGO_SPLIT_HEAD, ws=WS, wsb=ws, x=None) == C.E_INVAL
    assert f3r(algo=C.ALGO_SPLIT_HEAD, ws=WS, wsb=ws - 1) == C.E_WORKSPACE
    assert f3r(algo=C.ALGO_SPLIT_HEAD, ws=None, h_lo=1, h_hi=7) == C.E_WORKSPACE
    if not HAS_GPU:
        assert f3r(algo=C.ALGO_SPLIT_HEAD, ws=WS, wsb=ws) == expect
    # empty outputs are no-ops once the region itself is well formed
    assert f3r(x=None, y=None, D_out=0) == C.OK
    assert f3r(x=None, y=None, D_out=0, d_hi=7) == C.E_INVAL


def test_region_full_is_plain_validation():
    """The full region goes through the same checks as conv3x3x3_fwd."""
    full = dict(D_in=2, H_in=8, D_out=2, H_out=8, d_org=0, h_org=0, d_lo=0, d_hi=2, h_lo=0, h_hi=8)
    for kw in (dict(), dict(x=None), dict(epilogue=-1), dict(C_in=20), dict(algo=C.ALGO_SIMT),
               dict(algo=C.ALGO_SPLIT_HEAD), dict(algo=C.ALGO_MFMA, C_out=40), dict(y=A + 16)):
        assert f3d(**{"algo": C.ALGO_FUSED_HEAD, **kw}) == f3r(**{**full, **kw}), kw


def test_video_invalid_and_empty():
    ok = dict(y=A, rgb=A + (1 << 28), N=1, D=2, H=4, W=8, C=12, dtype=1, stream=0)

    def fv(**kw):
        a = dict(ok)
        a.update(kw)
        return _st(cx.conv_video_rgb8, a["y"], a["rgb"], a["N"], a["D"], a["H"], a["W"], a["C"],
                   a["dtype"], a["stream"])
    assert fv(C=11) == C.E_UNSUPPORTED
    assert fv(y=None) == C.E_INVAL
    assert fv(rgb=None) == C.E_INVAL
    assert fv(y=A + 8) == C.E_INVAL                 # misaligned
    assert fv(rgb=A + 16) == C.E_INVAL              # overlaps y
    assert fv(W=-1) == C.E_INVAL
    assert fv(dtype=7) == C.E_INVAL
    assert fv(y=None, rgb=None, D=0) == C.OK        # empty: no-op
    if not HAS_GPU:
        assert fv() == C.E_NODEVICE


def test_head_rgb8_invalid():
    def fr(**kw):
        a = dict(x=A, w=B, bias=None, rgb=A + (1 << 28), N=1, C_in=32, D=2, H=8, W=8, dtype=1,
                 epilogue=2, stream=0)
        a.update(kw)
        return _st(cx.conv3x3x3_head_rgb8, *[a[k] for k in (
            "x", "w", "bias", "rgb", "N", "C_in", "D", "H", "W", "dtype", "epilogue", "stream")])
    assert fr(x=None) == C.E_INVAL
    assert fr(rgb=A + (1 << 28) + 1) == C.E_INVAL     # odd address
    assert fr(rgb=A + 64) == C.E_INVAL                # overlaps x
    assert fr(C_in=20) == C.E_UNSUPPORTED
    assert fr(epilogue=5) == C.E_INVAL
    assert fr(x=None, rgb=None, D=0) == C.OK
    if not HAS_GPU:
        assert fr() == C.E_NODEVICE


def _band_by_enumeration(lo, rows, g_off, Hg):
    """The band's region fields worked out row by row: input row r of the band holds global row
    lo - g_off + r, and holds data exactly when that row lies inside the frame."""
    H_in = rows + 2 * g_off
    valid = [r for r in range(H_in) if 0 <= lo - g_off + r < Hg]
    h_lo, h_hi = (valid[0], valid[-1] + 1) if valid else (0, 0)
    return H_in, g_off, h_lo, h_hi


def test_band_region_matches_row_enumeration():
    for Hg in (1, 2, 5, 17, 44, 352):
        for g_off in (0, 1, 2, 3):
            for lo in range(0, Hg, max(1, Hg // 7)):
                for rows in sorted({0, 1, 2, Hg - lo, (Hg - lo) // 2}):
                    if rows < 0 or lo + rows > Hg:
                        continue
                    got = cx.conv_band_region(lo, rows, g_off, Hg)
                    H_in, h_org, h_lo, h_hi = _band_by_enumeration(lo, rows, g_off, Hg)
                    if h_lo == h_hi == 0 and got[2] >= got[3]:
                        # no row of the band's input holds data: any empty range is the same
                        assert got[:2] == (H_in, h_org)
                        continue
                    assert got == (H_in, h_org, h_lo, h_hi), (lo, rows, g_off, Hg)
    # the python helper is the C entry point
    from x3x3_convolution_amd.plan import band_rows
    assert band_rows(132, 44, 1, 352) == cx.conv_band_region(132, 44, 1, 352) == (46, 1, 0, 46)
    assert band_rows(0, 44, 1, 352) == (46, 1, 1, 46)
    assert band_rows(308, 44, 1, 352) == (46, 1, 0, 45)


def test_band_region_invalid():
    for args in ((-1, 4, 1, 10), (0, -1, 1, 10), (0, 4, -1, 10), (7, 4, 1, 10)):
        with pytest.raises(C.ConvError) as e:
            cx.conv_band_region(*args)
        assert e.value.status == C.E_INVAL
    lib = cx.library()
    import ctypes
    o = ctypes.c_int()
    assert lib.conv_band_region(0, 4, 1, 10, None, ctypes.byref(o), ctypes.byref(o),
                                ctypes.byref(o)) == C.E_INVAL
    assert lib.conv_causal_region(4, 1, ctypes.byref(o), None, ctypes.byref(o),
                                  ctypes.byref(o)) == C.E_INVAL


def test_causal_region_reads_the_causal_frames():
    """Output frame t of a chunk must read stored frames holding video frames t-2 .. t of the
    chunk (the cached frames of the previous chunk first), and nothing else."""
    for D_out in (0, 1, 2, 5, 16):
        for cached in (0, 1, 2):
            D_in, d_org, d_lo, d_hi = cx.conv_causal_region(D_out, cached)
            assert D_in == D_out + cached
            for t in range(D_out):
                # stored frame s holds chunk frame s - cached
                read = [t + d_org - 1 + kd for kd in range(3)]
                live = [s - cached for s in read if d_lo <= s < d_hi]
                assert live == [f for f in (t - 2, t - 1, t) if f >= -cached], (D_out, cached, t)
    for args in ((-1, 0), (4, 3), (4, -1)):
        with pytest.raises(C.ConvError):
            cx.conv_causal_region(*args)


def test_head_any_number_of_frames():
    """The head algorithms take any number of frames (a workgroup addresses only its own six
    input and four output frames); only frames too large for that window leave them."""
    for D in (16, 32, 200):
        assert cx.conv3x3x3_select_algo(1, 256, 12, D, 352, 624, 1, 1, 1, 0) == C.ALGO_FUSED_HEAD
        assert cx.conv3x3x3_is_supported(1, 256, 12, D, 352, 624, 1, 1, 1, 2, C.ALGO_SPLIT_HEAD) == C.OK
    # six 2048x1024x256 frames are 6 GiB: past the window's 32-bit range
    assert cx.conv3x3x3_select_algo(1, 256, 12, 2, 2048, 1024, 1, 1, 1, 0) == C.ALGO_MFMA
    assert cx.conv3x3x3_is_supported(1, 256, 12, 2, 2048, 1024, 1, 1, 1, 2,
                                     C.ALGO_FUSED_HEAD) == C.E_UNSUPPORTED


def test_describe_names_the_plan():
    d = C.conv3x3x3_describe
    assert d(1, 512, 512, 1, 44, 78) == "igemm32_kq tile=8x16 rows=64 splits=1 workgroups=240"
    assert d(1, 512, 512, 4, 44, 78) == "igemm32_sk tile=8x16 rows=256 splits=1 workgroups=240"
    assert d(1, 264, 96, 1, 44, 78) == "igemm32 tile=4x32 rows=256 splits=5 workgroups=165"
    # the head: 5 strips of 126 positions, 4 frame groups, 64 row ranges of <= 30 Z rows each
    assert d(1, 256, 12, 16, 352, 624) == (
        "fused_head strips=5 frame_groups=4 row_ranges=64 z_rows=30 workgroups=256")
    assert d(1, 256, 12, 16, 352, 624, algo=C.ALGO_SPLIT_HEAD).startswith(
        "split_head strips=5 frame_groups=4 row_ranges=64 ")
    assert d(1, 256, 12, 16, 352, 624, algo=C.ALGO_MFMA).startswith("igemm16_narrow tile=8x32 rows=16 ")
    assert d(1, 256, 12, 16, 352, 624, stride=2).startswith("igemm32 tile=4x32 rows=256 ")
    # truncation: the full length comes back, the buffer holds what fits
    lib = C.library()
    buf = ctypes.create_string_buffer(8)
    n = lib.conv3x3x3_describe(1, 512, 512, 1, 44, 78, 1, 1, 1, 0, buf, 8)
    assert n == len("igemm32_kq tile=8x16 rows=64 splits=1 workgroups=240") and buf.value == b"igemm32"
    # errors: no buffer, and what select_algo rejects
    assert lib.conv3x3x3_describe(1, 512, 512, 1, 44, 78, 1, 1, 1, 0, None, 8) == C.E_INVAL
    assert lib.conv3x3x3_describe(1, 512, 512, 1, 44, 78, 1, 1, 1, 0, buf, 0) == C.E_INVAL
    rejected = lib.conv3x3x3_select_algo(1, 20, 12, 1, 4, 4, 1, 1, 1, 0)
    assert rejected < 0 and lib.conv3x3x3_describe(1, 20, 12, 1, 4, 4, 1, 1, 1, 0, buf, 8) == rejected
    with pytest.raises(C.ConvError):
        d(1, 20, 12, 1, 4, 4)


def _head_plan(N, D, H, W, fused=True):
    txt = C.conv3x3x3_describe(N, 32, 12, D, H, W,
                               algo=C.ALGO_FUSED_HEAD if fused else C.ALGO_SPLIT_HEAD)
    f = dict(kv.split("=") for kv in txt.split()[1:])
    return {k: int(v) for k, v in f.items()}


@pytest.mark.parametrize("shape", [(1, 16, 352, 624), (1, 40, 37, 300), (2, 32, 17, 380),
                                   (1, 3, 9, 50), (1, 16, 44, 624), (1, 200, 352, 624),
                                   (3, 7, 1, 1), (1, 64, 1000, 130)])
@pytest.mark.parametrize("fused", [True, False])
def test_head_row_ranges_cover_and_balance(shape, fused):
    """The head's row ranges: one workgroup per (sample, frame group, range); no range costs more
    than a strip's rows plus its halo would if every range were a whole band of equal height, and
    the ranges fit the 256-workgroup rounds the plan chose."""
    N, D, H, W = shape
    p = _head_plan(N, D, H, W, fused)
    strip_out = 126 if fused else 128
    halo = 2 if fused else 0
    assert p["strips"] == -(-W // strip_out) and p["frame_groups"] == -(-D // 4)
    assert p["workgroups"] == N * p["frame_groups"] * p["row_ranges"]
    assert 1 <= p["row_ranges"] <= min(256, p["strips"] * H)
    # lower bound: the average cost; upper bound: whole bands of ceil(rows / ranges) rows
    total = p["strips"] * H
    assert p["z_rows"] >= -(-total // p["row_ranges"]) + halo
    assert p["z_rows"] <= -(-total // p["row_ranges"]) + 2 * halo + 1
    # at most four rounds of 256 workgroups
    assert p["workgroups"] <= 4 * 256 or p["row_ranges"] == 1
