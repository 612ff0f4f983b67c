"""ctypes binding of libconv3x3.so.  Argument marshalling only.

Tensor arguments may be torch tensors (their ``data_ptr()`` is passed; they must be contiguous
device tensors in the layout the C ABI documents) or plain integers (device addresses).  A
``stream`` of None means torch's current HIP stream on the current device.  Every non-zero
status raises ``ConvError`` carrying the library's message.
"""
from __future__ import annotations

import ctypes
import os
import threading

ABI_VERSION = 1
DTYPE_F16, DTYPE_BF16 = 0, 1
LAYOUT_CHANNELS_FIRST, LAYOUT_CHANNELS_LAST = 0, 1
EPI_NONE, EPI_RELU, EPI_CLAMP1 = 0, 1, 2
ALGO_AUTO, ALGO_SIMT, ALGO_MFMA, ALGO_SPLIT_HEAD, ALGO_FUSED_HEAD = 0, 1, 2, 3, 4
OK, E_INVAL, E_UNSUPPORTED, E_WORKSPACE, E_NODEVICE, E_LAUNCH = 0, -1, -2, -3, -4, -5

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libconv3x3.so")
_lib = None
_lock = threading.Lock()

# (name, restype, argtypes) of every exported entry point of include/conv3x3.h
_P, _I, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
EXPORTS = [
    ("conv_abi_version", _I, []),
    ("conv_status_str", ctypes.c_char_p, [_I]),
    ("conv_last_error", ctypes.c_char_p, []),
    ("conv_out_size", _I, [_I, _I]),
    ("conv3x3_fwd", _I, [_P, _P, _P, _P] + [_I] * 10 + [_P]),
    ("conv3x3_is_supported", _I, [_I] * 10),
    ("conv3x3_select_algo", _I, [_I] * 9),
    ("conv3x3x3_fwd", _I, [_P, _P, _P, _P] + [_I] * 11 + [_P, _SZ, _P]),
    ("conv3x3x3_fwd_region", _I, [_P, _P, _P, _P] + [_I] * 18 + [_P, _SZ, _P]),
    ("conv3x3x3_select_algo", _I, [_I] * 10),
    ("conv3x3x3_is_supported", _I, [_I] * 11),
    ("conv3x3x3_workspace_bytes", _SZ, [_I] * 10),
    ("conv3x3x3_packed_weight_bytes", _SZ, [_I] * 10),
    ("conv3x3x3_pack_weights", _I, [_P, _P] + [_I] * 10 + [_P]),
    ("conv_head_temporal", _I, [_P, _P, _P] + [_I] * 7 + [_P]),
    ("conv_head_stencil", _I, [_P, _P, _P] + [_I] * 7 + [_P]),
    ("conv_video_rgb8", _I, [_P, _P] + [_I] * 6 + [_P]),
    ("conv3x3x3_head_rgb8", _I, [_P, _P, _P, _P] + [_I] * 7 + [_P]),
    ("conv_band_region", _I, [_I] * 4 + [ctypes.POINTER(ctypes.c_int)] * 4),
    ("conv_causal_region", _I, [_I] * 2 + [ctypes.POINTER(ctypes.c_int)] * 4),
    ("conv_calib_mfma_bf16", _I, [_P, _I, _I, _P]),
    ("conv3x3x3_fwd_noalloc", _I, [_P, _P, _P, _P] + [_I] * 11 + [_P]),
    ("conv_calib_lds_dma", _I, [_P, _SZ, _I, _I, _I, _P]),
    ("conv3x3x3_describe", _I, [_I] * 10 + [ctypes.c_char_p, _I]),
    ("conv_calib_lds_read", _I, [_P, _I, _I, _I, _P]),
]
NOALLOC_SCRATCH_BYTES = 80 << 20


class ConvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s (%d): %s" % (_status_text(status), status, message))
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def library():
    """Load libconv3x3.so (build it with hipcc first if it is absent).  Raises if it cannot be
    loaded: there is no other implementation to fall back on."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            from . import _build
            _build.build()
        lib = ctypes.CDLL(_LIB_PATH)
        for name, res, args in EXPORTS:
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if lib.conv_abi_version() != ABI_VERSION:
            raise ImportError("libconv3x3.so ABI %d, binding expects %d"
                              % (lib.conv_abi_version(), ABI_VERSION))
        _lib = lib
        return lib


def _status_text(status: int) -> str:
    try:
        return library().conv_status_str(status).decode()
    except Exception:  # noqa: BLE001 - message formatting must not mask the original error
        return "status"


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int):
    if status != OK:
        raise ConvError(status, library().conv_last_error().decode())
    return status


def conv_abi_version() -> int:
    return library().conv_abi_version()


def conv_status_str(status: int) -> str:
    return library().conv_status_str(status).decode()


def conv_last_error() -> str:
    return library().conv_last_error().decode()


def conv_out_size(n: int, stride: int) -> int:
    return library().conv_out_size(n, stride)


def conv3x3_fwd(x, w, bias, y, N, C_in, C_out, H, W, stride=1, layout=LAYOUT_CHANNELS_FIRST,
                dtype=DTYPE_F16, epilogue=EPI_NONE, algo=ALGO_AUTO, stream=None):
    return _check(library().conv3x3_fwd(_ptr(x), _ptr(w), _ptr(bias), _ptr(y), N, C_in, C_out,
                                        H, W, stride, layout, dtype, epilogue, algo,
                                        _stream(stream)))


def conv3x3_is_supported(N, C_in, C_out, H, W, stride=1, layout=LAYOUT_CHANNELS_FIRST,
                         dtype=DTYPE_F16, epilogue=EPI_NONE, algo=ALGO_AUTO) -> int:
    return library().conv3x3_is_supported(N, C_in, C_out, H, W, stride, layout, dtype, epilogue,
                                          algo)


def conv3x3_select_algo(N, C_in, C_out, H, W, stride=1, layout=LAYOUT_CHANNELS_FIRST,
                        dtype=DTYPE_F16, algo=ALGO_AUTO) -> int:
    r = library().conv3x3_select_algo(N, C_in, C_out, H, W, stride, layout, dtype, algo)
    if r < 0:
        _check(r)
    return r


def conv3x3x3_select_algo(N, C_in, C_out, D, H, W, stride=1, layout=LAYOUT_CHANNELS_LAST,
                          dtype=DTYPE_BF16, algo=ALGO_AUTO) -> int:
    r = library().conv3x3x3_select_algo(N, C_in, C_out, D, H, W, stride, layout, dtype, algo)
    if r < 0:
        _check(r)
    return r


def conv3x3x3_is_supported(N, C_in, C_out, D, H, W, stride=1, layout=LAYOUT_CHANNELS_LAST,
                           dtype=DTYPE_BF16, epilogue=EPI_NONE, algo=ALGO_AUTO) -> int:
    return library().conv3x3x3_is_supported(N, C_in, C_out, D, H, W, stride, layout, dtype,
                                            epilogue, algo)


def conv3x3x3_workspace_bytes(N, C_in, C_out, D, H, W, stride=1, layout=LAYOUT_CHANNELS_LAST,
                              dtype=DTYPE_BF16, algo=ALGO_AUTO) -> int:
    return library().conv3x3x3_workspace_bytes(N, C_in, C_out, D, H, W, stride, layout, dtype,
                                               algo)


def conv3x3x3_packed_weight_bytes(N, C_in, C_out, D, H, W, stride=1,
                                  layout=LAYOUT_CHANNELS_LAST, dtype=DTYPE_BF16,
                                  algo=ALGO_AUTO) -> int:
    return library().conv3x3x3_packed_weight_bytes(N, C_in, C_out, D, H, W, stride, layout,
                                                   dtype, algo)


def conv3x3x3_pack_weights(w_oidhw, w_packed, N, C_in, C_out, D, H, W, stride=1,
                           layout=LAYOUT_CHANNELS_LAST, dtype=DTYPE_BF16, algo=ALGO_AUTO,
                           stream=None):
    return _check(library().conv3x3x3_pack_weights(_ptr(w_oidhw), _ptr(w_packed), N, C_in, C_out,
                                                   D, H, W, stride, layout, dtype, algo,
                                                   _stream(stream)))


def conv3x3x3_fwd(x, w_packed, bias, y, N, C_in, C_out, D, H, W, stride=1,
                  layout=LAYOUT_CHANNELS_LAST, dtype=DTYPE_BF16, epilogue=EPI_NONE,
                  algo=ALGO_AUTO, workspace=None, workspace_bytes=0, stream=None):
    return _check(library().conv3x3x3_fwd(_ptr(x), _ptr(w_packed), _ptr(bias), _ptr(y), N, C_in,
                                          C_out, D, H, W, stride, layout, dtype, epilogue, algo,
                                          _ptr(workspace), workspace_bytes, _stream(stream)))


def conv3x3x3_fwd_region(x, w_packed, bias, y, N, C_in, C_out, D_in, H_in, W, D_out, H_out,
                         d_org, h_org, d_lo, d_hi, h_lo, h_hi, layout=LAYOUT_CHANNELS_LAST,
                         dtype=DTYPE_BF16, epilogue=EPI_NONE, algo=ALGO_AUTO, workspace=None,
                         workspace_bytes=0, stream=None):
    return _check(library().conv3x3x3_fwd_region(
        _ptr(x), _ptr(w_packed), _ptr(bias), _ptr(y), N, C_in, C_out, D_in, H_in, W, D_out, H_out,
        d_org, h_org, d_lo, d_hi, h_lo, h_hi, layout, dtype, epilogue, algo, _ptr(workspace),
        workspace_bytes, _stream(stream)))


def conv_head_temporal(x, w_packed, g, N, C_in, C_out, D, H, W, dtype=DTYPE_BF16, stream=None):
    return _check(library().conv_head_temporal(_ptr(x), _ptr(w_packed), _ptr(g), N, C_in, C_out,
                                               D, H, W, dtype, _stream(stream)))


def conv_head_stencil(g, bias, y, N, D, H, W, C_out, dtype=DTYPE_BF16, epilogue=EPI_CLAMP1,
                      stream=None):
    return _check(library().conv_head_stencil(_ptr(g), _ptr(bias), _ptr(y), N, D, H, W, C_out,
                                              dtype, epilogue, _stream(stream)))


def conv_video_rgb8(y, rgb, N, D, H, W, C=12, dtype=DTYPE_BF16, stream=None):
    return _check(library().conv_video_rgb8(_ptr(y), _ptr(rgb), N, D, H, W, C, dtype,
                                            _stream(stream)))


def conv3x3x3_head_rgb8(x, w_packed, bias, rgb, N, C_in, D, H, W, dtype=DTYPE_BF16,
                        epilogue=EPI_CLAMP1, stream=None):
    return _check(library().conv3x3x3_head_rgb8(_ptr(x), _ptr(w_packed), _ptr(bias), _ptr(rgb),
                                                N, C_in, D, H, W, dtype, epilogue,
                                                _stream(stream)))


def conv_band_region(lo, rows, g_off, H_global):
    """(H_in, h_org, h_lo, h_hi) of output rows [lo, lo + rows) of a frame of global height
    H_global whose input holds g_off extra rows each side (conv_band_region)."""
    out = [ctypes.c_int() for _ in range(4)]
    _check(library().conv_band_region(lo, rows, g_off, H_global, *[ctypes.byref(o) for o in out]))
    return tuple(o.value for o in out)


def conv_causal_region(D_out, cached):
    """(D_in, d_org, d_lo, d_hi) of a causal chunk of D_out frames with `cached` frames of the
    previous chunk in front (conv_causal_region)."""
    out = [ctypes.c_int() for _ in range(4)]
    _check(library().conv_causal_region(D_out, cached, *[ctypes.byref(o) for o in out]))
    return tuple(o.value for o in out)


def conv_calib_mfma_bf16(out, workgroups, iters, stream=None):
    """Enqueues the matrix-core calibration loop (a measurement aid, conv_calib_mfma_bf16)."""
    return _check(library().conv_calib_mfma_bf16(_ptr(out), workgroups, iters, _stream(stream)))


def conv3x3x3_fwd_noalloc(x, w_packed, bias, y, N, C_in, C_out, D, H, W, stride=1,
                          layout=LAYOUT_CHANNELS_LAST, dtype=DTYPE_BF16, epilogue=EPI_NONE,
                          algo=ALGO_AUTO, stream=None):
    """conv3x3x3_fwd without a workspace argument: the library's static per-device scratch
    serves as the workspace (conv3x3x3_fwd_noalloc)."""
    return _check(library().conv3x3x3_fwd_noalloc(_ptr(x), _ptr(w_packed), _ptr(bias), _ptr(y), N,
                                                  C_in, C_out, D, H, W, stride, layout, dtype,
                                                  epilogue, algo, _stream(stream)))


def conv_calib_lds_dma(src, src_bytes, whole_lines, workgroups, iters, stream=None):
    """Enqueues the global -> LDS copy calibration loop (a measurement aid, conv_calib_lds_dma)."""
    return _check(library().conv_calib_lds_dma(_ptr(src), src_bytes, int(whole_lines),
                                               workgroups, iters, _stream(stream)))


def conv3x3x3_describe(N, C_in, C_out, D, H, W, stride=1, layout=LAYOUT_CHANNELS_LAST,
                       dtype=DTYPE_BF16, algo=ALGO_AUTO):
    """The launch plan conv3x3x3_fwd would use for this request, as one line of text."""
    buf = ctypes.create_string_buffer(256)
    n = library().conv3x3x3_describe(N, C_in, C_out, D, H, W, stride, layout, dtype, algo, buf, 256)
    if n < 0:
        _check(n)
    return buf.value.decode()


def conv_calib_lds_read(out, workgroups, waves, iters, stream=None):
    """Enqueues the LDS read-rate calibration loop (a measurement aid, conv_calib_lds_read)."""
    return _check(library().conv_calib_lds_read(_ptr(out), workgroups, waves, iters,
                                                _stream(stream)))
