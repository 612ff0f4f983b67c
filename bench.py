#!/usr/bin/env python3
"""Benchmark of the 3x3x3 video output head on one MI355X: ms per 704x1248 VAE-head pass.

The workload is the Wan2.2-style output head at its full size: x [1,16,352,624,256] bf16 NDHWC
(channels-last) -> y [1,16,352,624,12], bias, clamp to [-1,1], seeded synthetic N(0,1)
activations and N(0, 1/(27*256)) weights (no trained weights or real latents exist here).  One
step is one head pass, computed by the algorithm AUTO selects; the three head algorithms -- the
direct 27-tap MFMA implicit GEMM, the split head (3x1x1 temporal conv into a 112-channel plane,
then the nine-tap stencil) and the fused head -- are timed and reported.  Inputs are resident in
HBM before the timed region; each step's launches run back to back on one stream.  Every timed
region follows untimed warm-up steps -- at least --warmup of them and at least --settle-ms of
them -- so the chip's clock has settled under that load before the timing starts.

The default line also carries:
  * cpu_baseline: the oracle timed over one whole head pass on the host cores, and one thread
    over the small 2D workload; parity: the pass's every output against that oracle pass;
  * workloads: the other workloads (2D 16->16 and 64->64 at stride 1 and 2, the mid-decoder and
    low-res 3D convolutions), each timed with the same protocol, with its roofline fraction and
    its parity against the oracle (every output; a seeded sample of the mid-decoder conv);
  * calibration: a plain 1 GiB device copy and a loop of nothing but matrix-core instructions,
    what this machine's HBM and matrix cores sustain (context beside the published peaks),
    and the time of a launch that does almost nothing (the floor of any one-launch figure).

Prints one JSON line (see --help).  `--workload` times another of the synthetic workloads with
the same protocol (for measurements outside the default line).
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "conv TFLOP/s + HBM GB/s (roofline %), ms per 704x1248 VAE-head pass"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2516.6    # MI355X dense bf16 matrix-core peak
VALU_FP32_PEAK_TFS = 157.3     # MI355X fp32 vector peak (dot2/packed rate)
KERNEL_SOURCES = {             # dominant-kernel name -> the source file it is built from
    "igemm3d": "x3x3_convolution_amd/csrc/igemm3d.hip",
    "head_stencil": "x3x3_convolution_amd/csrc/stencil.hip",
    "head_fused": "x3x3_convolution_amd/csrc/head.hip",
    "simt2d": "x3x3_convolution_amd/csrc/simt2d.hip",
    "mfma2d": "x3x3_convolution_amd/csrc/mfma2d.hip",
    "video_rgb8": "x3x3_convolution_amd/csrc/video.hip",
}


class no_gc:
    """Python's cyclic garbage collector off for a timed region: a full collection costs tens of
    ms of host time, which the wall time per step would otherwise carry.  No collection runs at
    the start either: the GPU would sit idle meanwhile, and after an idle spell of that length
    the clock goes through its transient again, right in the timed steps."""

    def __enter__(self):
        gc.disable()
        return self

    def __exit__(self, *exc):
        gc.enable()
        return False


def warm_up(step, args):
    """Untimed steps before a timed region: at least args.warmup of them, in doubling batches
    until at least args.settle_ms of wall time has passed.  After an idle spell (another
    workload's oracle check, the process start) the chip's clock under a new load takes tens of
    ms to settle -- per-launch times first rise, then fall below where they started -- so a
    fixed handful of steps would time the transient instead of the sustained rate.  Returns the
    number of steps run."""
    import torch
    n, batch = 0, max(1, args.warmup)
    t0 = time.perf_counter()
    while n < args.warmup or (time.perf_counter() - t0) * 1e3 < args.settle_ms:
        for _ in range(batch):
            step()
        n += batch
        batch *= 2
        torch.cuda.synchronize()
    return n


def live_taps(n, stride=1):
    """Sum over output coordinates of the taps that land inside a pad-1 3-tap dimension."""
    nout = (n - 1) // stride + 1
    return sum(sum(1 for t in range(3) if 0 <= stride * o - 1 + t < n) for o in range(nout))


def source_sha(kernel):
    with open(os.path.join(ROOT, KERNEL_SOURCES[kernel]), "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def traffic_from_profiles(kernel, workload, algo):
    """HBM bytes per launch from the committed counter summary, if it was taken on the current
    kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh).get("%s/%s/%s" % (kernel, workload, algo))
    if not rec or rec.get("source_sha") != source_sha(kernel):
        return None
    return rec.get("bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="keep warming up (past --warmup steps) until this many ms of untimed "
                         "launches have run: after an idle spell the clock under a new load goes "
                         "through a transient of up to ~100 ms before it settles")
    ap.add_argument("--workload", default="c3",
                    choices=["c3", "c4", "c5", "c5d1", "c1", "c2", "c2s2"])
    ap.add_argument("--algo", default="auto", choices=["auto", "mfma", "split", "fused"],
                    help="auto: time every head algorithm and report AUTO's choice; otherwise "
                         "time only the named one")
    ap.add_argument("--region", default="none", choices=["none", "band8", "causal"],
                    help="3D workloads only: time a region pass instead of the plain one -- "
                         "band8: the middle eighth of the rows with a one-row halo each side "
                         "(one GPU's share when the rows are split over eight); causal: every "
                         "frame with causal temporal padding and two cached frames in front")
    ap.add_argument("--stride3d", type=int, default=1, choices=[1, 2],
                    help="3D workloads other than the head: spatial stride (2 halves H and W)")
    ap.add_argument("--flush", action="store_true",
                    help="workloads other than the head: overwrite a 512 MiB buffer before every "
                         "timed step (outside the timed events), so inputs and weights start "
                         "outside the L2s and the 256 MB last-level cache; the line's value is "
                         "then the kernel time")
    ap.add_argument("--channels-last", action="store_true",
                    help="2D workloads only: NHWC activations instead of NCHW")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (used for profiler runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--mfma-calibration", action="store_true",
                    help="only run the matrix-core calibration loop (bf16 32x32x16 MFMAs on "
                         "register operands) and the global -> LDS copy rates, and exit")
    ap.add_argument("--no-workloads", action="store_true",
                    help="default line only: skip the other workloads' entries")
    return ap.parse_args()


def copy_calibration():
    """A plain 1 GiB device copy: the counter calibration (FETCH_SIZE / WRITE_SIZE of a known
    byte count) and the HBM rate a plain stream reaches on this machine (HIP events)."""
    import torch
    n = 1 << 30
    a = torch.ones(n // 2, dtype=torch.int16, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    s.record()
    for _ in range(reps):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    del a, b
    torch.cuda.empty_cache()
    return {"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
            "copy_ms": round(ms, 4), "copy_gbs": round(2 * n / (ms * 1e-3) / 1e9, 1),
            "copy_hbm_frac": round(2 * n / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def mfma_calibration(stream):
    """The rate of a loop of nothing but bf16 32x32x16 MFMAs on register operands (one wave per
    SIMD on every CU), timed with HIP events on the launch stream: what this machine's matrix
    cores sustain under a pure matrix-core load, clock and power included.  A calibration beside
    the published peak, not a denominator.  The same kernel with one pass of its loop, on one
    and on 240 workgroups, gives the time of a launch with almost no work."""
    import torch
    from x3x3_convolution_amd import conv as C
    wgs, iters = 256 * 8, 2000
    out = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    for _ in range(2):
        C.conv_calib_mfma_bf16(out, wgs, iters, stream)
    torch.cuda.synchronize()
    tm = Timer(torch.cuda.current_stream())
    for _ in range(5):
        s0 = tm.start()
        C.conv_calib_mfma_bf16(out, wgs, iters, stream)
        tm.stop("mfma", s0)
    torch.cuda.synchronize()
    ms = tm.stats("mfma")["median"]
    flop = wgs * 4.0 * iters * 8 * 2 * 32 * 32 * 16
    tf = flop / (ms * 1e-3) / 1e12
    floor = {}
    for w in (1, 240):
        # the same kernel with one pass of its loop: what one launch costs with (almost) no work,
        # timed like the workloads (back to back, HIP events on the launch stream)
        for _ in range(3):
            C.conv_calib_mfma_bf16(out, w, 1, stream)
        torch.cuda.synchronize()
        for _ in range(20):
            s0 = tm.start()
            C.conv_calib_mfma_bf16(out, w, 1, stream)
            tm.stop(f"floor{w}", s0)
        torch.cuda.synchronize()
        floor[f"launch_floor_ms_{w}wg"] = round(tm.stats(f"floor{w}")["median"], 5)
    return dict({"mfma_loop_flop": flop, "mfma_loop_ms": ms, "mfma_loop_tflops": round(tf, 1),
                 "mfma_loop_frac_of_peak": round(tf / MFMA_BF16_PEAK_TFS, 4)}, **floor)


def lds_dma_calibration(stream):
    """The rate of global -> LDS copies (16 bytes per lane, the way the kernels stage operands)
    with every CU busy: whole 128-byte lines and half lines (64 bytes, the pattern of a
    32-channel slice of 256-channel positions), from an L2-resident 4 MiB source and from a
    1 GiB source that streams from HBM."""
    import torch
    from x3x3_convolution_amd import conv as C
    src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    wgs, iters = 256, 400
    out = {}
    for label, nbytes in (("l2", 4 << 20), ("hbm", 1 << 30)):
        for whole in (1, 0):
            C.conv_calib_lds_dma(src, nbytes, whole, wgs, iters, stream)
            torch.cuda.synchronize()
            tm = Timer(torch.cuda.current_stream())
            for _ in range(3):
                s0 = tm.start()
                C.conv_calib_lds_dma(src, nbytes, whole, wgs, iters, stream)
                tm.stop("dma", s0)
            torch.cuda.synchronize()
            ms = tm.stats("dma")["median"]
            gbs = wgs * 4.0 * iters * 16 * 1024 / (ms * 1e-3) / 1e9
            out["lds_dma_%s_%s_gbs" % (label, "whole_lines" if whole else "half_lines")] = round(gbs, 1)
    del src
    torch.cuda.empty_cache()
    return out


def lds_read_calibration(stream):
    """The rate of conflict-free LDS reads (16 bytes per lane) with 8 and 16 waves per CU: what
    the LDS can deliver to fragment reads, summed over the chip (TB/s; divided by 256 CUs and
    the clock it is bytes per clock per CU)."""
    import torch
    from x3x3_convolution_amd import conv as C
    wgs, iters = 256 * 4, 4000
    out = torch.empty(wgs * 512 * 4, dtype=torch.int32, device="cuda")
    res = {}
    for waves in (4, 8):
        C.conv_calib_lds_read(out, wgs, waves, iters, stream)
        torch.cuda.synchronize()
        tm = Timer(torch.cuda.current_stream())
        for _ in range(3):
            s0 = tm.start()
            C.conv_calib_lds_read(out, wgs, waves, iters, stream)
            tm.stop("lds", s0)
        torch.cuda.synchronize()
        ms = tm.stats("lds")["median"]
        tbs = wgs * waves * 64 * 16 * 8.0 * iters / (ms * 1e-3) / 1e12
        res["lds_read_%dwaves_per_cu_tbs" % (2 * waves)] = round(tbs, 1)
    del out
    return res


class Timer:
    """HIP events on one stream around a sequence of launches."""

    def __init__(self, stream):
        import torch
        self.torch = torch
        self.stream = stream
        self.pairs = []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        return e

    def stop(self, name, s):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        self.pairs.append((name, s, e))

    def times(self):
        out = {}
        for name, s, e in self.pairs:
            out.setdefault(name, []).append(s.elapsed_time(e))
        return out

    def summary(self):
        return {k: sum(v) / len(v) for k, v in self.times().items()}

    def stats(self, name):
        """median / min / p90 of one kernel's per-step times (ms)."""
        v = sorted(self.times()[name])
        return dict(median=round(v[len(v) // 2], 5), min=round(v[0], 5),
                    p90=round(v[min(len(v) - 1, (9 * len(v)) // 10)], 5))


def time_pack(op, w, stream, reps=5):
    """The one-time repack of the OIDHW weights into the plan's order (not part of a pass):
    average of a few re-packs, HIP events on the launch stream."""
    import torch
    from x3x3_convolution_amd import conv as C
    wc = w.contiguous()
    torch.cuda.synchronize()
    tm = Timer(torch.cuda.current_stream())
    for _ in range(reps):
        s0 = tm.start()
        C.conv3x3x3_pack_weights(wc, op.w_packed, *op._shape, op.algo, stream=stream)
        tm.stop("pack", s0)
    torch.cuda.synchronize()
    return tm.summary()["pack"]


def run_head(args, wl, stream):
    """Times every head algorithm; returns per-algorithm results and the AUTO choice."""
    import torch

    import synthetic_inputs as si
    from x3x3_convolution_amd import conv as C
    from x3x3_convolution_amd.plan import Conv3x3x3

    x, w, b = si.make_inputs(wl, device="cuda")
    P = wl.N * wl.D * wl.H * wl.W
    y = torch.empty(wl.y_shape(), dtype=wl.torch_dtype, device="cuda")
    shape = (wl.N, wl.C_in, wl.C_out, wl.D, wl.H, wl.W)
    auto = C.conv3x3x3_select_algo(*shape, 1, C.LAYOUT_CHANNELS_LAST, C.DTYPE_BF16, C.ALGO_AUTO)
    algos = {"mfma": C.ALGO_MFMA, "split": C.ALGO_SPLIT_HEAD, "fused": C.ALGO_FUSED_HEAD}
    if args.algo != "auto":   # time only the requested algorithm (profiler runs)
        auto = algos[args.algo]
        algos = {args.algo: auto}
    flop_live = 2.0 * wl.C_in * wl.C_out * live_taps(wl.D) * live_taps(wl.H) * live_taps(wl.W)
    xb, yb = P * wl.C_in * 2, P * wl.C_out * 2
    wb, bb = wl.C_out * wl.C_in * 27 * 2, wl.C_out * 2
    gb = P * 112 * 2
    results = {}
    for name, code in algos.items():
        op = Conv3x3x3(w, b, wl.N, wl.D, wl.H, wl.W, epilogue=wl.epilogue, algo=code)
        pack_ms = time_pack(op, w, stream)
        if code == C.ALGO_SPLIT_HEAD:
            g = op.workspace

            def step(tm=None):
                s0 = tm.start() if tm else None
                C.conv_head_temporal(x, op.w_packed, g, wl.N, wl.C_in, wl.C_out, wl.D, wl.H,
                                     wl.W, C.DTYPE_BF16, stream)
                if tm:
                    tm.stop("head_temporal", s0)
                    s1 = tm.start()
                C.conv_head_stencil(g, b, y, wl.N, wl.D, wl.H, wl.W, wl.C_out, C.DTYPE_BF16,
                                    C.EPI_CLAMP1, stream)
                if tm:
                    tm.stop("head_stencil", s1)
        else:
            kname = "head_fused" if code == C.ALGO_FUSED_HEAD else "igemm3d_direct"

            def step(tm=None, kname=kname, op=op):
                s0 = tm.start() if tm else None
                op(x, y, stream=stream)
                if tm:
                    tm.stop(kname, s0)
        nwarm = warm_up(step, args)
        tm = Timer(torch.cuda.current_stream())
        with no_gc():
            t0 = time.perf_counter()
            for _ in range(args.steps):
                step(tm)
            torch.cuda.synchronize()
            wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        k = tm.summary()
        results[name] = dict(ms_per_pass=wall_ms, kernel_ms=k, weight_pack_ms=pack_ms,
                             kernel_stats={kk: tm.stats(kk) for kk in k}, warmup_steps=nwarm)
        del op
        torch.cuda.empty_cache()

    # roofline of the dominant kernel of the chosen algorithm
    flop_t = 2.0 * wl.C_in * 9 * wl.C_out * live_taps(wl.D) * wl.H * wl.W   # temporal GEMM
    if auto == C.ALGO_FUSED_HEAD:
        kms = results["fused"]["kernel_ms"]["head_fused"]
        bytes_f = xb + yb + wl.C_out * wl.C_in * 27 * 2 + bb
        ach = bytes_f / (kms * 1e-3) / 1e9
        roof = dict(kernel="head_gemm_kernel (fused: temporal GEMM + in-register nine-tap stencil + clamp)",
                    bound="hbm", achieved=ach, peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=ach / HBM_PEAK_GBS, mfma_tflops=flop_t / (kms * 1e-3) / 1e12,
                    mfma_frac=flop_t / (kms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS,
                    algorithmic_bytes=bytes_f, algorithmic_flop=flop_t, avg_launch_ms=kms,
                    launch_ms_stats=results["fused"]["kernel_stats"]["head_fused"],
                    traffic=traffic_from_profiles("head_fused", wl.name, "fused"))
    elif auto == C.ALGO_SPLIT_HEAD:
        kms = results["split"]["kernel_ms"]["head_temporal"]
        bytes_t = xb + gb + wl.C_out * wl.C_in * 27 * 2
        ach = bytes_t / (kms * 1e-3) / 1e9
        roof = dict(kernel="head_gemm_kernel (split-head temporal 3x1x1, 112-channel plane)",
                    bound="hbm", achieved=ach, peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=ach / HBM_PEAK_GBS, mfma_tflops=flop_t / (kms * 1e-3) / 1e12,
                    algorithmic_bytes=bytes_t, algorithmic_flop=flop_t, avg_launch_ms=kms,
                    traffic=traffic_from_profiles("head_fused", wl.name, "split"))
    else:
        kms = results["mfma"]["kernel_ms"]["igemm3d_direct"]
        ach = flop_live / (kms * 1e-3) / 1e12
        bytes_d = xb + yb + wb + bb
        roof = dict(kernel="igemm3d (direct 27-tap head, 16-row tiles)", bound="mfma",
                    achieved=ach, peak=MFMA_BF16_PEAK_TFS, unit="TFLOP/s",
                    frac=ach / MFMA_BF16_PEAK_TFS,
                    hbm_gbs=bytes_d / (kms * 1e-3) / 1e9,
                    hbm_frac=bytes_d / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    algorithmic_bytes=bytes_d, algorithmic_flop=flop_live, avg_launch_ms=kms,
                    traffic=traffic_from_profiles("igemm3d", wl.name, "mfma"))
    chosen = {C.ALGO_SPLIT_HEAD: "split", C.ALGO_FUSED_HEAD: "fused"}.get(auto, "mfma")
    pass_ms = results[chosen]["ms_per_pass"]

    # the step after the pass: the 12-channel output as 704x1248 RGB bytes (timed on its own,
    # not part of the pass's value)
    video = None
    if wl.C_out == 12 and args.algo == "auto":
        rgb = torch.empty((wl.N, wl.D, 2 * wl.H, 2 * wl.W, 3), dtype=torch.uint8, device="cuda")
        warm_up(lambda: C.conv_video_rgb8(y, rgb, wl.N, wl.D, wl.H, wl.W, 12, C.DTYPE_BF16,
                                          stream), args)
        tm = Timer(torch.cuda.current_stream())
        for _ in range(args.steps):
            s0 = tm.start()
            C.conv_video_rgb8(y, rgb, wl.N, wl.D, wl.H, wl.W, 12, C.DTYPE_BF16, stream)
            tm.stop("video_rgb8", s0)
        torch.cuda.synchronize()
        vms = tm.summary()["video_rgb8"]
        vbytes = yb + rgb.numel()
        video = dict(kernel="video_rgb8_kernel", avg_launch_ms=round(vms, 5),
                     algorithmic_bytes=vbytes, gbs=round(vbytes / (vms * 1e-3) / 1e9, 1),
                     hbm_frac=round(vbytes / (vms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     traffic=traffic_from_profiles("video_rgb8", wl.name, "auto"))
        # the fused head writing the RGB frames straight from its registers (no y round trip)
        opf = Conv3x3x3(w, b, wl.N, wl.D, wl.H, wl.W, epilogue=wl.epilogue,
                        algo=C.ALGO_FUSED_HEAD)
        warm_up(lambda: opf.rgb8(x, rgb, stream=stream), args)
        tm = Timer(torch.cuda.current_stream())
        for _ in range(args.steps):
            s0 = tm.start()
            opf.rgb8(x, rgb, stream=stream)
            tm.stop("head_rgb8", s0)
        torch.cuda.synchronize()
        video["fused_head_rgb8_ms"] = round(tm.summary()["head_rgb8"], 5)
        video["separate_head_plus_video_ms"] = round(results["fused"]["kernel_ms"]["head_fused"] + vms, 5) \
            if "fused" in results else None
        del rgb, opf
    extra = dict(
        pass_tflops=flop_live / (pass_ms * 1e-3) / 1e12,
        pass_gbs=((xb + 2 * gb + yb + wb + bb) if chosen == "split" else (xb + yb + wb + bb))
        / (pass_ms * 1e-3) / 1e9,
        algos={k: dict(ms_per_pass=round(v["ms_per_pass"], 4),
                       kernel_ms={kk: round(vv, 4) for kk, vv in v["kernel_ms"].items()},
                       weight_pack_ms=round(v["weight_pack_ms"], 4),
                       warmup_steps=v["warmup_steps"])
               for k, v in results.items()})
    if video is not None:
        extra["video_step"] = video
    return chosen, pass_ms, roof, extra, (x, w, b), y


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def parity_of(y_bits, ref, dtype_code, activated):
    """d = y_gpu - y_oracle over the given outputs (the cpu_baseline leg's comparison): max|d|,
    rms(d) and rel-rms = rms(d) / rms(y_oracle), with the workload text's bound."""
    import numpy as np

    import oracle
    g = oracle.decode(np.ascontiguousarray(y_bits), dtype_code).reshape(-1)
    r = np.asarray(ref, np.float64).reshape(-1)
    d = g - r
    rms = float(np.sqrt(np.mean(d * d)))
    out = dict(max_abs=float(np.max(np.abs(d))), rms=rms,
               rel_rms=rms / max(float(np.sqrt(np.mean(r * r))), 1e-30), outputs=int(r.size),
               finite=bool(np.all(np.isfinite(g))))
    if activated:
        out["bound"] = dict(max_abs=1.6e-2, rms=2e-3)
        out["ok"] = out["finite"] and out["max_abs"] <= 1.6e-2 and out["rms"] <= 2e-3
    else:
        out["bound"] = dict(rel_rms=4e-3)
        out["ok"] = out["finite"] and out["rel_rms"] <= 4e-3
    for k in ("max_abs", "rms", "rel_rms"):
        out[k] = float("%.4g" % out[k])
    return out


def cpu_baseline(wl, tensors, y):
    """The cpu_baseline leg of the default line: the oracle (as it stands, plain loops, OpenMP
    over output rows) timed on the host cores over one whole head pass, its output compared with
    the GPU's at every output (parity of the line's value), and the oracle on one thread over
    the small 2D workload."""
    import oracle
    import synthetic_inputs as si

    x, w, b = tensors
    xb, wbits, bbits = si.bits(x), si.bits(w), si.bits(b)
    epi = {"none": oracle.EPI_NONE, "relu": oracle.EPI_RELU, "clamp1": oracle.EPI_CLAMP1}
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    ref = oracle.conv3d(xb, wbits, bbits, 1, oracle.BF16, epi[wl.epilogue], oracle.CHANNELS_LAST)
    dt = time.perf_counter() - t0
    parity = parity_of(si.bits(y), ref, oracle.BF16, wl.epilogue != "none")
    parity["positions"] = int(ref.size // wl.C_out)
    del ref, xb
    # one thread, the small 2D workload (input generation outside the timing)
    c1 = si.WORKLOADS["c1"]
    x1, w1, b1 = si.make_inputs(c1, device="cpu")
    oracle.set_threads(1)
    try:
        t1 = time.perf_counter()
        oracle.conv2d(si.bits(x1), si.bits(w1), si.bits(b1), c1.stride, oracle.F16,
                      epi[c1.epilogue], oracle.CHANNELS_FIRST)
        c1_ms = (time.perf_counter() - t1) * 1e3
    finally:
        oracle.set_threads(threads)
    base = dict(value=round(dt * 1e3, 1), unit="ms", cores=threads, kind="oracle",
                cpu_model=cpu_model(),
                sample="one whole head pass (%d positions x %d channels), timed end to end; the "
                       "oracle's OpenMP loops on %d threads" % (wl.N * wl.D * wl.H * wl.W,
                                                               wl.C_out, threads),
                single_thread_c1_ms=round(c1_ms, 2))
    return base, parity


def cpu_parity_sample(wl, tensors, y, full, channels_last=False):
    """Part of the cpu_baseline leg: the oracle over a workload's outputs (all of them, or for the
    largest one a seeded sample of positions) compared with the GPU's."""
    import numpy as np
    import torch

    import oracle
    import synthetic_inputs as si

    x, w, b = tensors
    epi = {"none": oracle.EPI_NONE, "relu": oracle.EPI_RELU, "clamp1": oracle.EPI_CLAMP1}[wl.epilogue]
    od = oracle.F16 if wl.dtype == "f16" else oracle.BF16
    t0 = time.perf_counter()
    if wl.kind == "2d":
        layout = oracle.CHANNELS_LAST if channels_last else oracle.CHANNELS_FIRST
        ref = oracle.conv2d(si.bits(x), si.bits(w), si.bits(b), wl.stride, od, epi, layout)
        got, n_pos = si.bits(y), wl.N * wl.H_out * wl.W_out
    elif full:
        ref = oracle.conv3d(si.bits(x), si.bits(w), si.bits(b), 1, od, epi, oracle.CHANNELS_LAST)
        got, n_pos = si.bits(y), wl.N * wl.D * wl.H * wl.W
    else:
        rng = np.random.default_rng(11)
        n_pos = 16384
        pts = np.stack([rng.integers(0, wl.N, n_pos), rng.integers(0, wl.D, n_pos),
                        rng.integers(0, wl.H, n_pos), rng.integers(0, wl.W, n_pos)], 1).astype(np.int32)
        ref = oracle.conv3d_points(si.bits(x), si.bits(w), si.bits(b), pts, 1, od, epi,
                                   oracle.CHANNELS_LAST)
        idx = torch.from_numpy(pts.astype(np.int64)).to(y.device)
        got = si.bits(y[idx[:, 0], idx[:, 1], idx[:, 2], idx[:, 3], :])
    p = parity_of(got, ref, od, wl.epilogue != "none")
    p["positions"] = int(n_pos)
    p["sampled"] = not (full or wl.kind == "2d")
    p["oracle_s"] = round(time.perf_counter() - t0, 2)
    return p


def run_other(args, wl, stream):
    """Same timing protocol for the other workloads (one algorithm each)."""
    import torch

    import synthetic_inputs as si
    from x3x3_convolution_amd import conv as C
    from x3x3_convolution_amd.plan import Conv3x3, Conv3x3x3

    x, w, b = si.make_inputs(wl, device="cuda")
    if wl.kind == "2d":
        if args.channels_last:
            x = x.permute(0, 2, 3, 1).contiguous()
        op = Conv3x3(w, b, wl.N, wl.H, wl.W, stride=wl.stride, epilogue=wl.epilogue,
                     channels_last=args.channels_last)
        P = wl.N * wl.H_out * wl.W_out
        flop = 2.0 * wl.C_in * wl.C_out * wl.N * live_taps(wl.H, wl.stride) * live_taps(wl.W, wl.stride)
        algo2d = C.conv3x3_select_algo(wl.N, wl.C_in, wl.C_out, wl.H, wl.W, wl.stride, op.layout,
                                       C.DTYPE_F16, C.ALGO_AUTO)
        if algo2d == C.ALGO_MFMA:
            # a stream at the HBM / matrix-core ridge: graded against HBM, MFMA reported beside
            kname, bound, peak, unit = "mfma2d", "hbm", HBM_PEAK_GBS, "GB/s"
        else:
            kname, bound, peak, unit = "simt2d", "alu", VALU_FP32_PEAK_TFS, "TFLOP/s"
    else:
        s3 = args.stride3d
        op = Conv3x3x3(w, b, wl.N, wl.D, wl.H, wl.W, epilogue=wl.epilogue, stride=s3)
        pack_ms = time_pack(op, w, stream)
        P = wl.N * wl.D * op.H_out * op.W_out
        flop = (2.0 * wl.C_in * wl.C_out * wl.N * live_taps(wl.D) * live_taps(wl.H, s3)
                * live_taps(wl.W, s3))
        kname, bound, peak, unit = "igemm3d", "mfma", MFMA_BF16_PEAK_TFS, "TFLOP/s"
    y = torch.empty(op.out_shape(), dtype=wl.torch_dtype, device="cuda")
    nbytes = (x.numel() + y.numel() + w.numel() + b.numel()) * 2
    nwarm = warm_up(lambda: op(x, y, stream=stream), args)
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda") if args.flush else None
    torch.cuda.synchronize()
    tm = Timer(torch.cuda.current_stream())
    with no_gc():
        t0 = time.perf_counter()
        for _ in range(args.steps):
            if scratch is not None:
                scratch.fill_(1)
            s = tm.start()
            op(x, y, stream=stream)
            tm.stop(kname, s)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    kms = tm.summary()[kname]
    kstats = tm.stats(kname)
    if scratch is not None:
        wall_ms = kms    # the flushes are not part of the step
    tflops = flop / (kms * 1e-3) / 1e12
    gbs = nbytes / (kms * 1e-3) / 1e9
    ach = gbs if unit == "GB/s" else tflops
    roof = dict(kernel=kname, bound=bound, achieved=ach, peak=peak, unit=unit, frac=ach / peak,
                hbm_gbs=gbs, hbm_frac=gbs / HBM_PEAK_GBS, algorithmic_flop=flop,
                algorithmic_bytes=nbytes, avg_launch_ms=kms, launch_ms_stats=kstats, positions=P,
                warmup_steps=nwarm,
                traffic=traffic_from_profiles(
                    kname, wl.name, "nhwc" if args.channels_last else
                    ("stride2" if wl.kind == "3d" and args.stride3d == 2 else "auto")))
    if kname == "mfma2d":
        roof.update(mfma_tflops=tflops, mfma_frac=tflops / MFMA_BF16_PEAK_TFS)
    if wl.kind == "3d":
        roof["weight_pack_ms"] = pack_ms
        roof["mfma_tflops"] = tflops
        roof["plan"] = C.conv3x3x3_describe(wl.N, wl.C_in, wl.C_out, wl.D, wl.H, wl.W, s3)
    return wall_ms, roof, y, (x, w, b)


WORKLOAD_NOTES = {
    "c1": "TAESD-style 2D conv 16->16, [1,16,64,64] fp16 NCHW, bias + ReLU (launch scale)",
    "c2": "TAESD-style 2D conv 64->64, [8,64,256,256] fp16 NCHW, bias + ReLU",
    "c2s2": "its stride-2 variant, [8,64,256,256] -> [8,64,128,128]",
    "c4": "mid-decoder 3D conv 256->256, [1,256,16,176,312] bf16 NDHWC, bias, identity",
    "c5": "low-res 3D conv 512->512, [1,512,4,44,78] bf16 NDHWC, bias, identity",
    "c5d1": "the same at D=1 (the first causal frame)",
}


def run_workloads(args, stream):
    """The other workloads, each timed with the default line's protocol (kernel time per step,
    HIP events on the launch stream) and, in the cpu_baseline leg, compared with the oracle."""
    import torch

    import synthetic_inputs as si

    out = {}
    for name in ("c1", "c2", "c2s2", "c4", "c5", "c5d1"):
        wl = si.WORKLOADS[name]
        wall_ms, roof, y, tensors = run_other(args, wl, stream)
        ent = dict(config=WORKLOAD_NOTES[name], kernel=roof["kernel"],
                   ms=dict(avg=round(roof["avg_launch_ms"], 5), **roof["launch_ms_stats"]),
                   bound=roof["bound"], achieved=round(roof["achieved"], 1), peak=roof["peak"],
                   unit=roof["unit"], frac=round(roof["frac"], 4),
                   hbm_gbs=round(roof["hbm_gbs"], 1), hbm_frac=round(roof["hbm_frac"], 4),
                   algorithmic_flop=roof["algorithmic_flop"],
                   algorithmic_bytes=roof["algorithmic_bytes"],
                   warmup_steps=roof["warmup_steps"])
        if "mfma_tflops" in roof:
            ent["mfma_tflops"] = round(roof["mfma_tflops"], 1)
            ent["mfma_frac"] = round(roof["mfma_tflops"] / MFMA_BF16_PEAK_TFS, 4)
        if "weight_pack_ms" in roof:
            ent["weight_pack_ms"] = round(roof["weight_pack_ms"], 4)
        if not args.no_cpu_baseline:
            ent["parity"] = cpu_parity_sample(wl, tensors, y, full=name != "c4",
                                              channels_last=args.channels_last)
        out[name] = ent
        print("workload %s: %.4f ms" % (name, roof["avg_launch_ms"]), file=sys.stderr, flush=True)
        del y, tensors
        torch.cuda.empty_cache()
    return out


def region_of(kind, D, H):
    """(D_in, H_in, d_org, h_org, d_lo, d_hi, h_lo, h_hi, D_out, H_out, band_lo) of a region
    pass over a workload of D frames and H rows."""
    from x3x3_convolution_amd.plan import band_rows, causal_frames
    if kind == "band8":
        rows = H // 8
        lo = 3 * rows
        H_in, h_org, h_lo, h_hi = band_rows(lo, rows, 1, H)
        return (D, H_in, 0, h_org, 0, D, h_lo, h_hi, D, rows, lo)
    D_in, d_org, d_lo, d_hi = causal_frames(D, 2)
    return (D_in, H, d_org, 0, d_lo, d_hi, 0, H, D, H, 0)


def run_region(args, wl, stream):
    """A region pass of a 3D workload (the --algo algorithm), timed like the plain pass."""
    import torch

    import synthetic_inputs as si
    from x3x3_convolution_amd import conv as C
    from x3x3_convolution_amd.plan import Conv3x3x3

    D_in, H_in, d_org, h_org, d_lo, d_hi, h_lo, h_hi, D, H, lo = region_of(args.region, wl.D, wl.H)
    # drawn on the GPU: a multi-threaded draw of this size on the host runs the process into its
    # CPU quota, and the throttling that follows lands in the timed steps
    _, w, b = si.make_inputs(wl, device="cuda")
    torch.cuda.empty_cache()
    g = torch.Generator("cuda").manual_seed(si.SEED_BASE + 7)
    x = torch.randn((wl.N, D_in, H_in, wl.W, wl.C_in), generator=g, device="cuda",
                    dtype=torch.float32).to(wl.torch_dtype)
    algo = {"auto": C.ALGO_AUTO, "mfma": C.ALGO_MFMA, "split": C.ALGO_SPLIT_HEAD,
            "fused": C.ALGO_FUSED_HEAD}[args.algo]
    op = Conv3x3x3(w, b, wl.N, D, H, wl.W, epilogue=wl.epilogue, algo=algo)
    y = torch.empty(op.out_shape(), dtype=wl.torch_dtype, device="cuda")
    kname = {C.ALGO_FUSED_HEAD: "head_fused", C.ALGO_SPLIT_HEAD: "head_split"}.get(op.algo, "igemm3d")

    def live(n_out, org, lo_, hi_):
        return sum(sum(1 for t in range(3) if lo_ <= o + org - 1 + t < hi_) for o in range(n_out))
    flop = (2.0 * wl.C_in * wl.C_out * wl.N * live(D, d_org, d_lo, d_hi) * live(H, h_org, h_lo, h_hi)
            * live_taps(wl.W))
    nbytes = (x.numel() + y.numel() + w.numel() + b.numel()) * 2

    def call():
        op.region(x, D_in, H_in, d_org, h_org, d_lo, d_hi, h_lo, h_hi, y=y, stream=stream)
    warm_up(call, args)
    tm = Timer(torch.cuda.current_stream())
    with no_gc():
        t0 = time.perf_counter()
        for _ in range(args.steps):
            s0 = tm.start()
            call()
            tm.stop(kname, s0)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    kms = tm.summary()[kname]
    tflops, gbs = flop / (kms * 1e-3) / 1e12, nbytes / (kms * 1e-3) / 1e9
    if kname == "igemm3d":
        bound, ach, peak, unit = "mfma", tflops, MFMA_BF16_PEAK_TFS, "TFLOP/s"
    else:
        bound, ach, peak, unit = "hbm", gbs, HBM_PEAK_GBS, "GB/s"
    roof = dict(kernel=kname, bound=bound, achieved=ach, peak=peak, unit=unit, frac=ach / peak,
                hbm_gbs=gbs, mfma_tflops=tflops, mfma_frac=tflops / MFMA_BF16_PEAK_TFS,
                algorithmic_flop=flop, algorithmic_bytes=nbytes, avg_launch_ms=kms,
                traffic=None)
    cfg = dict(workload="%s %s" % (wl.name, args.region), N=wl.N, C_in=wl.C_in, C_out=wl.C_out,
               D_out=D, H_out=H, W=wl.W, D_in=D_in, H_in=H_in, d_org=d_org, h_org=h_org,
               band_lo=lo, algo=kname)
    return wall_ms, roof, cfg


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        print(json.dumps(copy_calibration()))
        return
    import torch

    import synthetic_inputs as si

    torch.cuda.set_device(0)
    # a dedicated stream (default priority): the library's launches and the timing events
    # both go on it
    strm = torch.cuda.Stream()
    torch.cuda.set_stream(strm)
    stream = strm.cuda_stream
    if args.mfma_calibration:
        print(json.dumps(dict(mfma_calibration(stream), **lds_dma_calibration(stream),
                              **lds_read_calibration(stream))))
        return
    wl = si.WORKLOADS[args.workload]
    line = dict(metric=METRIC, n_gpus=1, steps=args.steps, warmup=args.warmup,
                warmup_settle_ms=args.settle_ms,
                higher_is_better=False, scaling="weak", vs_baseline=None, dtype=wl.dtype,
                data="synthetic (seeded; no trained weights or real activations)")
    if args.region != "none":
        if wl.kind != "3d":
            print("--region applies to the 3D workloads", file=sys.stderr)
            sys.exit(2)
        wall_ms, roof, cfg = run_region(args, wl, stream)
        line.update(value=round(wall_ms, 4), unit="ms", ms_per_step=round(wall_ms, 4), config=cfg,
                    roofline={k: (round(v, 6) if isinstance(v, float) else v)
                              for k, v in roof.items()})
    elif wl.name == "c3":
        chosen, pass_ms, roof, extra, tensors, y_head = run_head(args, wl, stream)
        line.update(value=round(pass_ms, 4), unit="ms", ms_per_step=round(pass_ms, 4),
                    config=dict(workload="wan2.2 output head 3x3x3 256->12, x [1,16,352,624,256] "
                                "bf16 NDHWC, bias + clamp[-1,1], one 704x1248 head pass",
                                algo=chosen, N=wl.N, C_in=wl.C_in, C_out=wl.C_out, D=wl.D,
                                H=wl.H, W=wl.W),
                    roofline={k: (round(v, 6) if isinstance(v, float) else v)
                              for k, v in roof.items()})
        line.update({k: (round(v, 4) if isinstance(v, float) else v) for k, v in extra.items()})
        if not args.no_cpu_baseline:
            line["cpu_baseline"], line["parity"] = cpu_baseline(wl, tensors, y_head)
            line["parity"]["algo"] = chosen   # y holds the last algorithm timed: AUTO's choice
        del tensors, y_head
        torch.cuda.empty_cache()
        if not args.no_workloads and args.algo == "auto":
            line["workloads"] = run_workloads(args, stream)
            line["calibration"] = dict(copy_calibration(), **mfma_calibration(stream),
                                       **lds_dma_calibration(stream),
                                       **lds_read_calibration(stream))
    else:
        wall_ms, roof, _, _ = run_other(args, wl, stream)
        layout = ("NHWC" if args.channels_last else "NCHW") if wl.kind == "2d" else "NDHWC"
        line.update(value=round(wall_ms, 4), unit="ms", ms_per_step=round(wall_ms, 4),
                    config=dict(workload=wl.name, N=wl.N, C_in=wl.C_in, C_out=wl.C_out, D=wl.D,
                                H=wl.H, W=wl.W,
                                stride=wl.stride if wl.kind == "2d" else args.stride3d,
                                epilogue=wl.epilogue, layout=layout, caches_flushed=args.flush),
                    roofline={k: (round(v, 6) if isinstance(v, float) else v)
                              for k, v in roof.items()})
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
