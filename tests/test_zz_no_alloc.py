"""The allocation-free entry point (conv3x3x3_fwd_noalloc) against conv3x3x3_fwd.

Both run the same kernels; the allocation-free one takes its workspace from the library's static
per-device scratch.  Two calls in a row that need that scratch (split-K partial sums), the second
with a smaller input, must each give the same bits as conv3x3x3_fwd with a caller-owned
workspace; a request without a workspace (the fused head) must too, and one that needs more
than the scratch holds (the split head's plane at full head size) is refused with nothing
enqueued.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from gpu_support import DEV, alloc_guarded, assert_bit_exact, bits, check_guards, oracle_3d
from x3x3_convolution_amd import conv as C
from x3x3_convolution_amd.plan import Conv3x3x3

pytestmark = pytest.mark.gpu


def _both(x, w, b, epilogue, algo=C.ALGO_AUTO):
    N, D, H, W, Ci = x.shape
    op = Conv3x3x3(w, b, N, D, H, W, epilogue=epilogue, algo=algo)
    ref = op(x)
    buf, y = alloc_guarded(op.out_shape(), x.dtype)
    C.conv3x3x3_fwd_noalloc(x, op.w_packed, op.bias, y, N, Ci, op.C_out, D, H, W, 1,
                            C.LAYOUT_CHANNELS_LAST, op.dtype, op.epi, op.algo)
    torch.cuda.synchronize()
    check_guards(buf, y.numel())
    return op, ref, y


def test_noalloc_matches_fwd_two_calls_smaller_second():
    # 1) a low-resolution frame pair with 384 channels: K split six ways, 16 MB of partials
    x, w, b = si.random_case("3d", 1, 384, 136, 40, 60, D=2, dtype="bf16", seed=900, device=DEV)
    op, ref, y = _both(x, w, b, "none")
    assert 0 < op.ws_bytes <= C.NOALLOC_SCRATCH_BYTES
    assert torch.equal(ref.view(torch.int16), y.view(torch.int16))
    # 2) a smaller split-K request right after it (the scratch still holds the first call's
    #    partials): integer inputs, so both must also equal the oracle bit for bit
    x2, w2, b2 = si.integer_case("3d", 2, 96, 20, 9, 13, D=1, dtype="bf16", seed=901, device=DEV)
    op2, ref2, y2 = _both(x2, w2, b2, "relu")
    assert 0 < op2.ws_bytes < op.ws_bytes
    assert torch.equal(ref2.view(torch.int16), y2.view(torch.int16))
    assert_bit_exact(y2, oracle_3d(x2, w2, b2, "relu"), x2.dtype)


def test_noalloc_without_workspace_and_split_plane():
    # the fused head needs no workspace; the split head's plane of a small frame fits the scratch
    x, w, b = si.integer_case("3d", 1, 32, 12, 9, 50, D=3, dtype="bf16", seed=902, device=DEV)
    for algo in (C.ALGO_FUSED_HEAD, C.ALGO_SPLIT_HEAD):
        op, ref, y = _both(x, w, b, "clamp1", algo)
        assert torch.equal(ref.view(torch.int16), y.view(torch.int16))
        assert_bit_exact(y, oracle_3d(x, w, b, "clamp1"), x.dtype)


def test_noalloc_stream_k():
    # the MFMA path's stream-K schedule: partial tiles and arrival counters in the scratch (the
    # counters cleared by the call itself), against conv3x3x3_fwd and the oracle
    x, w, b = si.integer_case("3d", 1, 416, 300, 36, 78, D=5, dtype="bf16", seed=903, device=DEV)
    assert C.conv3x3x3_describe(1, 416, 300, 5, 36, 78).startswith("igemm32_sk ")
    op, ref, y = _both(x, w, b, "relu")
    assert 0 < op.ws_bytes <= C.NOALLOC_SCRATCH_BYTES
    assert torch.equal(ref.view(torch.int16), y.view(torch.int16))
    assert_bit_exact(y, oracle_3d(x, w, b, "relu"), x.dtype)


def test_noalloc_refuses_more_than_the_scratch():
    N, Ci, Co, D, H, W = 1, 256, 12, 16, 352, 624
    need = C.conv3x3x3_workspace_bytes(N, Ci, Co, D, H, W, algo=C.ALGO_SPLIT_HEAD)
    assert need > C.NOALLOC_SCRATCH_BYTES
    y = torch.full((8,), 0x7FFF, dtype=torch.int16, device=DEV)
    with pytest.raises(C.ConvError) as e:
        C.conv3x3x3_fwd_noalloc(1 << 20, 1 << 30, None, y, N, Ci, Co, D, H, W, 1,
                                C.LAYOUT_CHANNELS_LAST, C.DTYPE_BF16, C.EPI_CLAMP1,
                                C.ALGO_SPLIT_HEAD)
    assert e.value.status == C.E_WORKSPACE and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(y == 0x7FFF)
