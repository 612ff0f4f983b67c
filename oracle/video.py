"""The step after the head: its 12-channel output as an 8-bit RGB video -- TEST INFRASTRUCTURE.

[head.cu, header comment: the clamped 12-channel plane is what the video writer consumes;
commit summary: the decoded RGB video's frames are copied to the host once.]  The pages do not
say how 12 channels become RGB pixels or how values become bytes; the readings taken:

* **pixel shuffle, factor 2**: 12 = 3 colours x 2 x 2 sub-pixels; channel k = 4*c + 2*dy + dx of
  position (h, w) is colour c of output pixel (2h + dy, 2w + dx) -- the channel order of PyTorch's
  ``pixel_shuffle`` (colour outermost, then the sub-pixel row, then its column);
* **quantisation**: [-1, 1] maps linearly onto [0, 255]: ``u8 = clamp(RNE(127.5 * (v + 1)), 0,
  255)`` evaluated exactly (round half to even of the exact value), NaN -> 0, +inf -> 255,
  -inf -> 0.  In fp64, ``v * 127.5 + 127.5`` is exact for every fp16/bf16 value except the tiny
  ones (|v| below about 2^-38), where the sum rounds to 127.5 itself; the exact value then lies
  just above or below the tie, which the sign of v decides.

Output layout: (N, D, 2H, 2W, 3) uint8, channels-last (the per-frame HWC RGB a video writer
takes).  Plain numpy; pinned by ``tests/test_oracle_video.py``.
"""
from __future__ import annotations

import numpy as np


def quantize_u8(values) -> np.ndarray:
    """fp16/bf16 values (as float64 or float32 arrays) -> uint8 codes, exactly rounded."""
    v = np.asarray(values, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        t = v * 127.5 + 127.5                         # exact unless |v| is tiny (see above)
        q = np.rint(t)                                # round half to even
        q = np.where((v < 0) & (t == 127.5), 127.0, q)
        q = np.where(np.isnan(q), 0.0, q)
    return np.clip(q, 0, 255).astype(np.uint8)


def pixel_shuffle2_nhwc(q) -> np.ndarray:
    """(..., H, W, 12) -> (..., 2H, 2W, 3): channel 4c + 2dy + dx -> pixel (2h+dy, 2w+dx), colour c."""
    q = np.asarray(q)
    *lead, H, W, C = q.shape
    assert C == 12, "12 channels (3 colours x 2 x 2) expected"
    t = q.reshape(*lead, H, W, 3, 2, 2)                       # (..., h, w, c, dy, dx)
    n = len(lead)
    perm = list(range(n)) + [n, n + 3, n + 1, n + 4, n + 2]   # (..., h, dy, w, dx, c)
    return np.ascontiguousarray(t.transpose(perm)).reshape(*lead, 2 * H, 2 * W, 3)


def video_rgb8(y_values) -> np.ndarray:
    """Head output values (N, D, H, W, 12) -> RGB bytes (N, D, 2H, 2W, 3)."""
    return pixel_shuffle2_nhwc(quantize_u8(y_values))
