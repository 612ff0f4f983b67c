"""CPU oracle for the pad-1 3x3 / 3x3x3 convolution -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package.  The product library (``x3x3_convolution_amd``) never imports it and shares
no code with it; the only module both sides use is ``synthetic_inputs`` (seeded input bits).

The arithmetic lives in ``conv_oracle.c`` (plain nested loops, fp64, OpenMP over output rows);
this module builds it with gcc and marshals numpy arrays through ctypes.  Inputs are fp16/bf16
*bit patterns* (``numpy.uint16``); the C code decodes them exactly.  Outputs are unrounded fp64.

What pins each function (the tests under ``tests/test_oracle_*.py``):

* ``decode`` / ``encode``: every one of the 65536 bit patterns against numpy's binary16 and
  torch's bfloat16 conversions; round-to-nearest-even ties and overflow at hand-picked values.
* ``conv2d`` / ``conv3d`` / ``*_points``: one-hot (delta) weights give shifted copies with zero
  fill (orientation and padding); all-ones inputs and weights give the closed-form border counts
  9/6/4 (2D) and 27/18/12/8 (3D) times C_in; linearity in x and in w; stride 2 equals stride 1
  sampled at [::2, ::2] with size floor((H-1)/2)+1; D=1 equals 2D with the centre temporal
  slice; weights live only at kd=1 give per-frame 2D convolutions; zero weights give E(bias);
  tiny random shapes against torch.nn.functional.conv2d/conv3d in float64 and a numpy
  im2col-times-matrix form; hand-worked examples stored under tests/golden/.
* ``head_split``: without rounding it equals ``conv3d`` (the split's algebra); with rounding the
  intermediate plane equals the encoded-then-decoded unrounded plane.
* ``video_rgb8`` (``video.py``, numpy): the head output as 8-bit RGB pixels; quantisation against
  exact rational arithmetic over every bf16 value, the pixel shuffle against
  torch.nn.functional.pixel_shuffle.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

F16, BF16 = 0, 1
CHANNELS_FIRST, CHANNELS_LAST = 0, 1
EPI_NONE, EPI_RELU, EPI_CLAMP1 = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "conv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()


def build(force: bool = True, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile conv_oracle.c (or another source ``src``) into a shared library with gcc (IEEE
    fp64: no fast-math, no FMA contraction).  Returns the library path."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-o", tmp, src, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def _bind(path: str):
    lib = ctypes.CDLL(path)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    f64p = ctypes.POINTER(ctypes.c_double)
    i32p = ctypes.POINTER(ctypes.c_int32)
    ci = ctypes.c_int
    lib.oracle_decode_one.argtypes = [ctypes.c_uint16, ci]
    lib.oracle_decode_one.restype = ctypes.c_double
    lib.oracle_encode_one.argtypes = [ctypes.c_double, ci]
    lib.oracle_encode_one.restype = ctypes.c_uint16
    lib.oracle_decode.argtypes = [u16p, f64p, ctypes.c_int64, ci]
    lib.oracle_decode.restype = None
    lib.oracle_encode.argtypes = [f64p, u16p, ctypes.c_int64, ci]
    lib.oracle_encode.restype = None
    lib.oracle_out_size.argtypes = [ci, ci]
    lib.oracle_out_size.restype = ci
    lib.oracle_conv2d.argtypes = [u16p, u16p, u16p, f64p] + [ci] * 9
    lib.oracle_conv2d.restype = ci
    lib.oracle_conv3d.argtypes = [u16p, u16p, u16p, f64p] + [ci] * 10
    lib.oracle_conv3d.restype = ci
    lib.oracle_conv3d_points.argtypes = [u16p, u16p, u16p, i32p, ctypes.c_int64, f64p] + [ci] * 10
    lib.oracle_conv3d_points.restype = ci
    lib.oracle_conv2d_points.argtypes = [u16p, u16p, u16p, i32p, ctypes.c_int64, f64p] + [ci] * 9
    lib.oracle_conv2d_points.restype = ci
    lib.oracle_head_split.argtypes = [u16p, u16p, u16p, f64p, f64p] + [ci] * 10
    lib.oracle_head_split.restype = ci
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ci
    lib.oracle_set_threads.argtypes = [ci]
    lib.oracle_set_threads.restype = None
    return lib


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("oracle inputs are uint16 bit patterns, got %s" % a.dtype)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16))


def _opt_u16(a):
    if a is None:
        return None, None
    return _u16(a)


def _f64p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _shape2d(x, layout):
    if layout == CHANNELS_FIRST:
        N, C, H, W = x.shape
    else:
        N, H, W, C = x.shape
    return N, C, H, W


def _shape3d(x, layout):
    if layout == CHANNELS_FIRST:
        N, C, D, H, W = x.shape
    else:
        N, D, H, W, C = x.shape
    return N, C, D, H, W


class Oracle:
    """The oracle's entry points bound to one compiled library (the default one is
    ``liboracle.so``; tests also bind deliberately broken copies to show the pins catch them)."""

    def __init__(self, path: str):
        self.lib = _bind(path)

    def max_threads(self) -> int:
        """Threads the OpenMP loops use (the calling thread's setting)."""
        return self.lib.oracle_max_threads()

    def set_threads(self, n: int) -> None:
        """Sets the thread count of the OpenMP loops for the calling thread."""
        self.lib.oracle_set_threads(int(n))

    def out_size(self, n: int, stride: int) -> int:
        return self.lib.oracle_out_size(int(n), int(stride))

    def decode(self, bits, dtype: int) -> np.ndarray:
        b, bp = _u16(bits)
        out = np.empty(b.shape, np.float64)
        self.lib.oracle_decode(bp, _f64p(out), b.size, dtype)
        return out

    def encode(self, values, dtype: int) -> np.ndarray:
        v = np.ascontiguousarray(values, dtype=np.float64)
        out = np.empty(v.shape, np.uint16)
        self.lib.oracle_encode(_f64p(v), out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)),
                               v.size, dtype)
        return out

    def conv2d(self, x, w, b, stride: int = 1, dtype: int = F16, epilogue: int = EPI_NONE,
               layout: int = CHANNELS_FIRST) -> np.ndarray:
        """x: (N,C,H,W) [NCHW] or (N,H,W,C) [NHWC] uint16 bits; w: (C_out,C_in,3,3);
        b: (C_out,) or None.  Returns fp64 y in the same layout."""
        x, xp = _u16(x)
        w, wp = _u16(w)
        b, bp = _opt_u16(b)
        N, C, H, W = _shape2d(x, layout)
        Co = w.shape[0]
        assert w.shape == (Co, C, 3, 3)
        Ho, Wo = self.out_size(H, stride), self.out_size(W, stride)
        shape = (N, Co, Ho, Wo) if layout == CHANNELS_FIRST else (N, Ho, Wo, Co)
        y = np.empty(shape, np.float64)
        rc = self.lib.oracle_conv2d(xp, wp, bp, _f64p(y), N, C, Co, H, W, stride, dtype,
                                    epilogue, layout)
        if rc:
            raise ValueError("oracle_conv2d rejected its arguments (%d)" % rc)
        return y

    def conv3d(self, x, w, b, stride: int = 1, dtype: int = BF16, epilogue: int = EPI_NONE,
               layout: int = CHANNELS_LAST) -> np.ndarray:
        """x: (N,D,H,W,C) [NDHWC] or (N,C,D,H,W) [NCDHW]; w: (C_out,C_in,3,3,3); returns fp64
        y in the same layout."""
        x, xp = _u16(x)
        w, wp = _u16(w)
        b, bp = _opt_u16(b)
        N, C, D, H, W = _shape3d(x, layout)
        Co = w.shape[0]
        assert w.shape == (Co, C, 3, 3, 3)
        Ho, Wo = self.out_size(H, stride), self.out_size(W, stride)
        shape = (N, Co, D, Ho, Wo) if layout == CHANNELS_FIRST else (N, D, Ho, Wo, Co)
        y = np.empty(shape, np.float64)
        rc = self.lib.oracle_conv3d(xp, wp, bp, _f64p(y), N, C, Co, D, H, W, stride, dtype,
                                    epilogue, layout)
        if rc:
            raise ValueError("oracle_conv3d rejected its arguments (%d)" % rc)
        return y

    def conv3d_points(self, x, w, b, pts, stride: int = 1, dtype: int = BF16,
                      epilogue: int = EPI_NONE, layout: int = CHANNELS_LAST) -> np.ndarray:
        """The 3D definition at output positions pts[i] = (n, od, oh, ow); returns
        (len(pts), C_out) fp64."""
        x, xp = _u16(x)
        w, wp = _u16(w)
        b, bp = _opt_u16(b)
        N, C, D, H, W = _shape3d(x, layout)
        Co = w.shape[0]
        p = np.ascontiguousarray(pts, dtype=np.int32).reshape(-1, 4)
        y = np.empty((p.shape[0], Co), np.float64)
        rc = self.lib.oracle_conv3d_points(
            xp, wp, bp, p.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), p.shape[0], _f64p(y),
            N, C, Co, D, H, W, stride, dtype, epilogue, layout)
        if rc:
            raise ValueError("oracle_conv3d_points rejected its arguments (%d)" % rc)
        return y

    def conv2d_points(self, x, w, b, pts, stride: int = 1, dtype: int = F16,
                      epilogue: int = EPI_NONE, layout: int = CHANNELS_FIRST) -> np.ndarray:
        """The 2D definition at output positions pts[i] = (n, oh, ow); returns
        (len(pts), C_out) fp64."""
        x, xp = _u16(x)
        w, wp = _u16(w)
        b, bp = _opt_u16(b)
        N, C, H, W = _shape2d(x, layout)
        Co = w.shape[0]
        p = np.ascontiguousarray(pts, dtype=np.int32).reshape(-1, 3)
        y = np.empty((p.shape[0], Co), np.float64)
        rc = self.lib.oracle_conv2d_points(
            xp, wp, bp, p.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), p.shape[0], _f64p(y),
            N, C, Co, H, W, stride, dtype, epilogue, layout)
        if rc:
            raise ValueError("oracle_conv2d_points rejected its arguments (%d)" % rc)
        return y

    def head_split(self, x, w, b, dtype: int = BF16, epilogue: int = EPI_CLAMP1,
                   layout: int = CHANNELS_LAST, round_g: bool = False, return_g: bool = False):
        """Split-head mode: temporal 3x1x1 conv into 9*C_out tap channels (optionally rounded
        to the activation dtype), then the nine-tap shifted sum + bias + epilogue.  Returns y
        (and G as an (N,D,H,W,9*C_out) fp64 array if return_g)."""
        x, xp = _u16(x)
        w, wp = _u16(w)
        b, bp = _opt_u16(b)
        N, C, D, H, W = _shape3d(x, layout)
        Co = w.shape[0]
        assert w.shape == (Co, C, 3, 3, 3)
        shape = (N, Co, D, H, W) if layout == CHANNELS_FIRST else (N, D, H, W, Co)
        y = np.empty(shape, np.float64)
        g = np.empty((N, D, H, W, 9 * Co), np.float64) if return_g else None
        rc = self.lib.oracle_head_split(xp, wp, bp, _f64p(y),
                                        _f64p(g) if g is not None else None, N, C, Co, D, H, W,
                                        dtype, epilogue, layout, int(bool(round_g)))
        if rc:
            raise ValueError("oracle_head_split rejected its arguments (%d)" % rc)
        return (y, g) if return_g else y


_default = None


def default() -> Oracle:
    """The oracle bound to liboracle.so (built with gcc on first use if absent)."""
    global _default
    with _lock:
        if _default is None:
            if not os.path.exists(_LIB_PATH):
                build(force=True)
            _default = Oracle(_LIB_PATH)
        return _default


def out_size(n, stride):
    return default().out_size(n, stride)


def max_threads():
    return default().max_threads()


def set_threads(n):
    return default().set_threads(n)


def decode(bits, dtype):
    return default().decode(bits, dtype)


def encode(values, dtype):
    return default().encode(values, dtype)


def conv2d(*a, **k):
    return default().conv2d(*a, **k)


def conv3d(*a, **k):
    return default().conv3d(*a, **k)


def conv2d_points(*a, **k):
    return default().conv2d_points(*a, **k)


def conv3d_points(*a, **k):
    return default().conv3d_points(*a, **k)


def head_split(*a, **k):
    return default().head_split(*a, **k)


from .video import pixel_shuffle2_nhwc, quantize_u8, video_rgb8  # noqa: E402,F401
