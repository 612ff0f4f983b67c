"""Helpers of the GPU parity tests: run the HIP path through the C ABI, evaluate the oracle on the
same bits, and compare (bit-exact, or by the max|d| / rms / rel-rms tolerances)."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synthetic_inputs as si
from x3x3_convolution_amd import conv as C
from x3x3_convolution_amd.plan import Conv3x3, Conv3x3x3

DEV = "cuda:0"
EPI = {"none": oracle.EPI_NONE, "relu": oracle.EPI_RELU, "clamp1": oracle.EPI_CLAMP1}
# tolerances of the fp16/bf16 paths against the fp64 oracle
TOL_ACT = dict(max_abs=1.6e-2, rms=2e-3)     # clamped / activated outputs
TOL_LINEAR = dict(rel_rms=4e-3)              # unclamped outputs


def odt(torch_dtype):
    return oracle.F16 if torch_dtype == torch.float16 else oracle.BF16


def bits(t):
    return si.bits(t)


def alloc_guarded(shape, dtype, guard=256, fill_bits=0x7FFF):
    """An output tensor inside a larger buffer whose guard bands (and the tensor itself) are
    pre-filled with a NaN pattern: unwritten outputs and out-of-bounds writes both show."""
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * guard,), fill_bits, dtype=torch.int16, device=DEV)
    y = buf[guard:guard + n].view(dtype).view(shape)
    return buf, y


def check_guards(buf, n, guard=256, fill_bits=0x7FFF):
    g = buf.cpu().numpy().view(np.uint16)
    assert np.all(g[:guard] == fill_bits), "write before the output buffer"
    assert np.all(g[guard + n:] == fill_bits), "write past the output buffer"


def run_2d(x, w, b, stride, epilogue, guarded=False, algo=C.ALGO_SIMT):
    N, Ci, H, W = x.shape
    op = Conv3x3(w, b, N, H, W, stride=stride, epilogue=epilogue, algo=algo)
    if guarded:
        buf, y = alloc_guarded(op.out_shape(), x.dtype)
        op(x, y)
        torch.cuda.synchronize()
        check_guards(buf, y.numel())
        return y
    y = op(x)
    torch.cuda.synchronize()
    return y


def run_3d(x, w, b, epilogue, algo, guarded=False):
    N, D, H, W, Ci = x.shape
    op = Conv3x3x3(w, b, N, D, H, W, epilogue=epilogue, algo=algo)
    if guarded:
        buf, y = alloc_guarded(op.out_shape(), x.dtype)
        op(x, y)
        torch.cuda.synchronize()
        check_guards(buf, y.numel())
        return y
    y = op(x)
    torch.cuda.synchronize()
    return y


def oracle_2d(x, w, b, stride, epilogue):
    return oracle.conv2d(bits(x), bits(w), bits(b), stride, odt(x.dtype), EPI[epilogue],
                         oracle.CHANNELS_FIRST)


def oracle_3d(x, w, b, epilogue):
    return oracle.conv3d(bits(x), bits(w), bits(b), 1, odt(x.dtype), EPI[epilogue],
                         oracle.CHANNELS_LAST)


def assert_bit_exact(y_gpu, y_ref, dtype):
    """The GPU bits must equal the oracle's value rounded once to the storage dtype."""
    got = bits(y_gpu)
    exp = oracle.encode(y_ref, odt(dtype)).reshape(got.shape)
    bad = np.flatnonzero(got != exp)
    assert bad.size == 0, "%d of %d outputs differ; first at flat index %d: got %s want %s" % (
        bad.size, got.size, bad[0], hex(got.flat[bad[0]]), hex(exp.flat[bad[0]]))


def metrics(y_gpu_bits, y_ref, dtype):
    g = oracle.decode(np.ascontiguousarray(y_gpu_bits), odt(dtype)).reshape(-1)
    r = np.asarray(y_ref, np.float64).reshape(-1)
    assert np.all(np.isfinite(g)), "non-finite output"
    d = g - r
    rms = float(np.sqrt(np.mean(d * d)))
    return dict(max_abs=float(np.max(np.abs(d))), rms=rms,
                rel_rms=rms / max(float(np.sqrt(np.mean(r * r))), 1e-30))


def assert_within(m, activated):
    if activated:
        assert m["max_abs"] <= TOL_ACT["max_abs"] and m["rms"] <= TOL_ACT["rms"], m
    else:
        assert m["rel_rms"] <= TOL_LINEAR["rel_rms"], m


def sample_points_3d(N, D, H, W, n_random, seed):
    """Output positions to check at full size: every combination of border / near-border /
    middle coordinates, plus uniformly random ones."""
    rng = np.random.default_rng(seed)

    def picks(n):
        return sorted({0, 1, n // 2, n - 2, n - 1} & set(range(n)))
    pts = [(nn, d, h, w) for nn in sorted({0, N - 1}) for d in picks(D) for h in picks(H)
           for w in picks(W)]
    pts += [tuple(int(v) for v in (rng.integers(N), rng.integers(D), rng.integers(H),
                                   rng.integers(W))) for _ in range(n_random)]
    return np.array(sorted(set(pts)), np.int32)


def sample_points_2d(N, Ho, Wo, n_random, seed):
    rng = np.random.default_rng(seed)

    def picks(n):
        return sorted({0, 1, n // 2, n - 2, n - 1} & set(range(n)))
    pts = [(nn, h, w) for nn in sorted({0, N - 1}) for h in picks(Ho) for w in picks(Wo)]
    pts += [tuple(int(v) for v in (rng.integers(N), rng.integers(Ho), rng.integers(Wo)))
            for _ in range(n_random)]
    return np.array(sorted(set(pts)), np.int32)


def gather_3d(y, pts):
    """y[n, d, h, w, :] at the sampled positions, as uint16 bits (len(pts), C)."""
    idx = torch.from_numpy(pts.astype(np.int64)).to(y.device)
    sel = y[idx[:, 0], idx[:, 1], idx[:, 2], idx[:, 3], :]
    return bits(sel)


def gather_2d(y, pts):
    idx = torch.from_numpy(pts.astype(np.int64)).to(y.device)
    sel = y[idx[:, 0], :, idx[:, 1], idx[:, 2]]
    return bits(sel)
