"""Convenience owners of the buffers the C ABI asks the caller for (plumbing only).

``Conv3x3x3`` packs a weight tensor once and keeps the packed copy and the workspace the chosen
algorithm needs; calling it runs ``conv3x3x3_fwd``.  ``Conv3x3`` does the same for the 2D call,
which needs neither.  Device memory comes from torch; every computation runs in libconv3x3.so.
"""
from __future__ import annotations

import torch

from . import conv as C

_DT = {torch.float16: C.DTYPE_F16, torch.bfloat16: C.DTYPE_BF16}
_EPI = {"none": C.EPI_NONE, "relu": C.EPI_RELU, "clamp1": C.EPI_CLAMP1}


def dtype_code(t: torch.dtype) -> int:
    if t not in _DT:
        raise TypeError("conv3x3 supports float16 and bfloat16 storage, got %s" % t)
    return _DT[t]


def epi_code(e) -> int:
    return _EPI[e] if isinstance(e, str) else int(e)


class Conv3x3:
    """2D pad-1 3x3 convolution of one fixed shape over NCHW tensors, or NHWC ones with
    channels_last=True (weights OIHW either way)."""

    def __init__(self, w, bias, N, H, W, stride=1, epilogue="none", algo=C.ALGO_AUTO,
                 channels_last=False):
        self.w, self.bias = w.contiguous(), None if bias is None else bias.contiguous()
        self.C_out, self.C_in = w.shape[0], w.shape[1]
        self.N, self.H, self.W, self.stride = N, H, W, stride
        self.dtype = dtype_code(w.dtype)
        self.epi = epi_code(epilogue)
        self.algo = algo
        self.layout = C.LAYOUT_CHANNELS_LAST if channels_last else C.LAYOUT_CHANNELS_FIRST
        self.H_out, self.W_out = C.conv_out_size(H, stride), C.conv_out_size(W, stride)

    def out_shape(self):
        if self.layout == C.LAYOUT_CHANNELS_LAST:
            return (self.N, self.H_out, self.W_out, self.C_out)
        return (self.N, self.C_out, self.H_out, self.W_out)

    def __call__(self, x, y=None, stream=None):
        if y is None:
            y = torch.empty(self.out_shape(), dtype=self.w.dtype, device=x.device)
        C.conv3x3_fwd(x, self.w, self.bias, y, self.N, self.C_in, self.C_out, self.H, self.W,
                      self.stride, self.layout, self.dtype, self.epi, self.algo, stream)
        return y


class Conv3x3x3:
    """3D pad-1 3x3x3 convolution over NDHWC tensors of one fixed input shape; stride 2 is
    spatial (H, W halve, the D frames stay)."""

    def __init__(self, w, bias, N, D, H, W, epilogue="none", algo=C.ALGO_AUTO, stream=None,
                 stride=1):
        self.C_out, self.C_in = w.shape[0], w.shape[1]
        self.N, self.D, self.H, self.W = N, D, H, W
        self.stride = stride
        self.H_out, self.W_out = C.conv_out_size(H, stride), C.conv_out_size(W, stride)
        self.dtype = dtype_code(w.dtype)
        self.torch_dtype = w.dtype
        self.epi = epi_code(epilogue)
        self.bias = None if bias is None else bias.contiguous()
        shape = (N, self.C_in, self.C_out, D, H, W, stride, C.LAYOUT_CHANNELS_LAST, self.dtype)
        self.algo = C.conv3x3x3_select_algo(*shape, algo)
        nbytes = C.conv3x3x3_packed_weight_bytes(*shape, self.algo)
        self.w_packed = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
        C.conv3x3x3_pack_weights(w.contiguous(), self.w_packed, *shape, self.algo, stream=stream)
        self.ws_bytes = C.conv3x3x3_workspace_bytes(*shape, self.algo)
        self.workspace = (torch.empty(self.ws_bytes, dtype=torch.uint8, device=w.device)
                          if self.ws_bytes else None)
        self._shape = shape

    def out_shape(self):
        return (self.N, self.D, self.H_out, self.W_out, self.C_out)

    def __call__(self, x, y=None, stream=None):
        if y is None:
            y = torch.empty(self.out_shape(), dtype=self.torch_dtype, device=x.device)
        N, Ci, Co, D, H, W, s, lay, dt = self._shape
        C.conv3x3x3_fwd(x, self.w_packed, self.bias, y, N, Ci, Co, D, H, W, s, lay, dt, self.epi,
                        self.algo, self.workspace, self.ws_bytes, stream)
        return y

    def region(self, x, D_in, H_in, d_org, h_org, d_lo, d_hi, h_lo, h_hi, y=None, stream=None):
        """The convolution over an input region of x (N, D_in, H_in, W, C_in) into an output of
        this plan's extent (N, D, H, W, C_out): conv3x3x3_fwd_region (stride 1)."""
        if self.stride != 1:
            raise ValueError("regions are stride-1 convolutions")
        if y is None:
            y = torch.empty(self.out_shape(), dtype=self.torch_dtype, device=x.device)
        N, Ci, Co, D, H, W, s, lay, dt = self._shape
        C.conv3x3x3_fwd_region(x, self.w_packed, self.bias, y, N, Ci, Co, D_in, H_in, W, D, H,
                               d_org, h_org, d_lo, d_hi, h_lo, h_hi, lay, dt, self.epi, self.algo,
                               self.workspace, self.ws_bytes, stream)
        return y


    def rgb8(self, x, rgb=None, stream=None):
        """The fused head writing the RGB frames of its output (conv3x3x3_head_rgb8); the plan
        must be a C_out = 12 fused head."""
        if self.algo != C.ALGO_FUSED_HEAD or self.C_out != 12:
            raise ValueError("rgb8 needs a fused head with 12 output channels")
        N, Ci, Co, D, H, W, s, lay, dt = self._shape
        if rgb is None:
            rgb = torch.empty((N, D, 2 * H, 2 * W, 3), dtype=torch.uint8, device=x.device)
        C.conv3x3x3_head_rgb8(x, self.w_packed, self.bias, rgb, N, Ci, D, H, W, dt, self.epi,
                              stream)
        return rgb


def band_rows(lo, rows, halo, H_global):
    """Region rows of an output band [lo, lo + rows) of a global height H_global whose input
    holds global rows lo - halo .. lo + rows + halo - 1 (rows outside the global height may
    hold anything): (H_in, h_org, h_lo, h_hi) for conv3x3x3_fwd_region (conv_band_region)."""
    return C.conv_band_region(lo, rows, halo, H_global)


def causal_frames(D_out, cached):
    """Region frames of a causal temporal pass (output frame t reads input frames t-2 .. t) over
    D_out new frames, with `cached` (0..2) frames of the previous chunk stored in front of them
    and zeros in place of the rest: (D_in, d_org, d_lo, d_hi) for conv3x3x3_fwd_region
    (conv_causal_region)."""
    if not 0 <= cached <= 2:
        raise ValueError("cached must be 0, 1 or 2")
    return C.conv_causal_region(D_out, cached)
