"""Seeded synthetic inputs for the convolution workloads -- shared by the tests, the benchmark and
the smoke check.  It holds none of the convolution's arithmetic: it only draws numbers and rounds
them to the storage dtype, so both the HIP library and the CPU oracle can be fed the same bits.

Workloads (shapes, layouts and distributions of the image/video decoder convolutions the pages
describe: TAESD-style low-channel fp16 NCHW 2D convs, Wan2.2-style bf16 channels-last 3D convs
and the 256->12 output head).  "N(0, v)" means variance v.  Values are drawn in fp32 with a
seeded torch generator and rounded to the dtype with round-to-nearest-even (``Tensor.to``).
Seeds: 20261200 + 10*id + {x: 0, w: 1, b: 2}.

Activations are returned in their physical layout as contiguous tensors:
NCHW -> (N, C, H, W); NDHWC -> (N, D, H, W, C).  Weights are (C_out, C_in, 3, 3[, 3]).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

SEED_BASE = 20261200


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "2d" | "3d"
    N: int
    C_in: int
    C_out: int
    H: int
    W: int
    D: int = 1
    stride: int = 1
    dtype: str = "f16"   # "f16" | "bf16"
    epilogue: str = "relu"   # "none" | "relu" | "clamp1"
    x_dist: str = "normal"   # "normal" | "uniform" | "relu_normal"
    w_var: float = 1.0
    b_var: float = 0.1
    x_id: int = 0
    w_id: int = 0
    notes: str = field(default="", compare=False)

    @property
    def torch_dtype(self):
        return torch.float16 if self.dtype == "f16" else torch.bfloat16

    @property
    def H_out(self):
        return (self.H - 1) // self.stride + 1

    @property
    def W_out(self):
        return (self.W - 1) // self.stride + 1

    def x_shape(self):
        if self.kind == "2d":
            return (self.N, self.C_in, self.H, self.W)
        return (self.N, self.D, self.H, self.W, self.C_in)

    def y_shape(self):
        if self.kind == "2d":
            return (self.N, self.C_out, self.H_out, self.W_out)
        return (self.N, self.D, self.H_out, self.W_out, self.C_out)

    def w_shape(self):
        if self.kind == "2d":
            return (self.C_out, self.C_in, 3, 3)
        return (self.C_out, self.C_in, 3, 3, 3)


WORKLOADS = {
    # TAESD-style smallest case: 16->16 at 64x64, fp16 NCHW, bias + ReLU, x ~ U(-1,1).
    "c1": Workload("c1", "2d", N=1, C_in=16, C_out=16, H=64, W=64, dtype="f16", epilogue="relu",
                   x_dist="uniform", w_var=2.0 / (9 * 16), x_id=1, w_id=1),
    # TAESD-style 64->64 at 8x256x256, fp16 NCHW, bias + ReLU, x ~ ReLU(N(0,1)).
    "c2": Workload("c2", "2d", N=8, C_in=64, C_out=64, H=256, W=256, dtype="f16",
                   epilogue="relu", x_dist="relu_normal", w_var=2.0 / (9 * 64), x_id=2, w_id=2),
    # its stride-2 variant 256x256 -> 128x128 (own seeds)
    "c2s2": Workload("c2s2", "2d", N=8, C_in=64, C_out=64, H=256, W=256, stride=2, dtype="f16",
                     epilogue="relu", x_dist="relu_normal", w_var=2.0 / (9 * 64), x_id=21,
                     w_id=21),
    # Wan2.2-style output head 256->12 over a 16-frame 352x624 latent-upsampled plane, clamp.
    "c3": Workload("c3", "3d", N=1, C_in=256, C_out=12, D=16, H=352, W=624, dtype="bf16",
                   epilogue="clamp1", x_dist="normal", w_var=1.0 / (27 * 256), x_id=3, w_id=3),
    # mid-decoder 256->256 3D conv at 16x176x312, identity epilogue.
    "c4": Workload("c4", "3d", N=1, C_in=256, C_out=256, D=16, H=176, W=312, dtype="bf16",
                   epilogue="none", x_dist="normal", w_var=1.0 / (27 * 256), x_id=4, w_id=4),
    # low-res high-channel 512->512 at 4x44x78, identity epilogue ...
    "c5": Workload("c5", "3d", N=1, C_in=512, C_out=512, D=4, H=44, W=78, dtype="bf16",
                   epilogue="none", x_dist="normal", w_var=1.0 / (27 * 512), x_id=5, w_id=5),
    # ... and the same weights at D=1 (the first causal frame of a chunked decode).
    "c5d1": Workload("c5d1", "3d", N=1, C_in=512, C_out=512, D=1, H=44, W=78, dtype="bf16",
                     epilogue="none", x_dist="normal", w_var=1.0 / (27 * 512), x_id=51, w_id=5),
}


def seed_for(cfg_id: int, which: str) -> int:
    return SEED_BASE + 10 * cfg_id + {"x": 0, "w": 1, "b": 2}[which]


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(seed)
    return g


def _draw_x(wl: Workload, shape, seed: int, device) -> torch.Tensor:
    g = _gen(seed, device)
    if wl.x_dist == "uniform":
        v = torch.rand(shape, generator=g, device=device, dtype=torch.float32) * 2.0 - 1.0
    else:
        v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if wl.x_dist == "relu_normal":
            v.clamp_(min=0.0)
    return v.to(wl.torch_dtype)


def make_inputs(wl: Workload, device="cpu", x_device=None, with_bias: bool = True):
    """Return (x, w, b) tensors in the workload's dtype and physical layout.  x is drawn on
    ``x_device`` (default ``device``): drawing the large video tensors on the GPU is fast; the
    result differs from a CPU draw with the same seed but is equally seeded and recorded."""
    x_device = device if x_device is None else x_device
    x = _draw_x(wl, wl.x_shape(), seed_for(wl.x_id, "x"), x_device)
    gw = _gen(seed_for(wl.w_id, "w"), "cpu")
    w = (torch.randn(wl.w_shape(), generator=gw, dtype=torch.float32) * math.sqrt(wl.w_var))
    w = w.to(wl.torch_dtype).to(device)
    b = None
    if with_bias:
        gb = _gen(seed_for(wl.w_id, "b"), "cpu")
        b = (torch.randn((wl.C_out,), generator=gb, dtype=torch.float32) * math.sqrt(wl.b_var))
        b = b.to(wl.torch_dtype).to(device)
    return x, w, b


def random_case(kind: str, N: int, C_in: int, C_out: int, H: int, W: int, D: int = 1,
                dtype: str = "bf16", seed: int = 0, x_std: float = 1.0, device="cpu",
                with_bias: bool = True):
    """A small random case for parity tests: x ~ N(0, x_std^2), w ~ N(0, 1/(taps*C_in)),
    b ~ N(0, 0.1).  Returns (x, w, b) in the physical layouts above."""
    td = torch.float16 if dtype == "f16" else torch.bfloat16
    g = _gen(SEED_BASE + 7919 * seed + 13, "cpu")
    xs = (N, C_in, H, W) if kind == "2d" else (N, D, H, W, C_in)
    ws = (C_out, C_in, 3, 3) if kind == "2d" else (C_out, C_in, 3, 3, 3)
    taps = 9 if kind == "2d" else 27
    x = (torch.randn(xs, generator=g) * x_std).to(td)
    w = (torch.randn(ws, generator=g) * math.sqrt(1.0 / (taps * C_in))).to(td)
    b = (torch.randn((C_out,), generator=g) * math.sqrt(0.1)).to(td) if with_bias else None
    mv = (lambda t: None if t is None else t.to(device))
    return mv(x), mv(w), mv(b)


def integer_case(kind: str, N: int, C_in: int, C_out: int, H: int, W: int, D: int = 1,
                 dtype: str = "bf16", seed: int = 0, max_nnz: int = 255, device="cpu",
                 with_bias: bool = True):
    """Integer-valued inputs for which every partial sum is exact in fp32 and in the storage
    dtype, in any order: w in {-1,0,1} with at most ``max_nnz`` non-zeros per output channel
    (and per output channel and spatial tap for the split head), b in {-1,0,1};
    x in {-1,0,1} for bf16 (|sums| <= 256 fit bf16's 8-bit significand) and in {-2..2} for fp16
    (|sums| <= 511 < 2048).  Any correct kernel must reproduce the oracle bit for bit."""
    td = torch.float16 if dtype == "f16" else torch.bfloat16
    rng = np.random.default_rng(SEED_BASE + 104729 * seed + 17)
    xs = (N, C_in, H, W) if kind == "2d" else (N, D, H, W, C_in)
    ws = (C_out, C_in, 3, 3) if kind == "2d" else (C_out, C_in, 3, 3, 3)
    xmax = 2 if dtype == "f16" else 1
    x = rng.integers(-xmax, xmax + 1, size=xs).astype(np.float32)
    K = int(np.prod(ws[1:]))
    p = min(0.5, max_nnz / (2.0 * K))
    w = (rng.integers(-1, 2, size=ws) * (rng.random(ws) < 2 * p)).astype(np.float32)
    wf = w.reshape(C_out, -1)
    for co in range(C_out):  # cap the non-zeros per output channel
        nz = np.flatnonzero(wf[co])
        if nz.size > max_nnz:
            wf[co, rng.choice(nz, nz.size - max_nnz, replace=False)] = 0.0
    w = wf.reshape(ws)
    b = rng.integers(-1, 2, size=(C_out,)).astype(np.float32) if with_bias else None
    tt = (lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(td).to(device))
    return tt(x), tt(w), tt(b)


def bits(t: torch.Tensor) -> np.ndarray:
    """The fp16/bf16 bit patterns of a tensor as a host numpy uint16 array (same shape)."""
    if t is None:
        return None
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
