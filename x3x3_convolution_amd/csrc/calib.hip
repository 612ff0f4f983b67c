// Measurement aids, not part of the convolution: the rate the matrix cores reach on a loop of
// nothing but bf16 32x32x16 MFMAs with register operands, the rate of global -> LDS copies
// (the way the kernels stage their operands) for whole and half cache lines, and the rate of
// conflict-free LDS reads.  The benchmark
// reports them beside the plain-copy rate as what this machine sustains (clock and power
// included); the roofline fractions are still taken against the published peaks.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "conv3x3.h"

namespace cx {
namespace {

constexpr int kChains = 8;   // independent accumulators: back-to-back issue, no dependency stalls

__global__ __launch_bounds__(256) void mfma_loop_kernel(float *out, int iters) {
    using E = Elem<true>;
    typedef E::vec8 vec8;
    // operands that depend on the lane, so nothing folds; small values, so nothing overflows
    vec8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (float)((threadIdx.x + i) & 7));
        b[i] = (__bf16)(0.001f * (float)((threadIdx.x * 3 + i) & 7));
    }
    f32x16_t acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = f32x16_t{};
#pragma unroll 1
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = E::mfma32x32x16(a, b, acc[c]);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) s += acc[c][i];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Global -> LDS copies (buffer_load ... lds, 16 bytes per lane): each wave keeps copying 16 KiB
// slices of `src` into its own 16 KiB of LDS, up to 32 copies in flight.  LINE = 1: one copy
// is 1 KiB of consecutive bytes (eight whole 128-byte lines); LINE = 0: 16 pieces of 64 bytes
// 512 bytes apart (half lines, the pattern of a 32-channel slice of channels-last positions with
// 256 channels).  Offsets stay inside the first half of `src` (plus one copy's span).
template <int LINE>
__global__ __launch_bounds__(256, 1) void lds_dma_kernel(const unsigned char *src,
                                                        unsigned src_bytes, int iters) {
    typedef __attribute__((address_space(3))) void lds_void;
    __shared__ __attribute__((aligned(16))) uint4 buf[4][16][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc((void *)src, (short)0, (int)src_bytes, 0x00020000);
    const unsigned span = src_bytes / 2;
    const unsigned wbase = ((blockIdx.x * 4u + (unsigned)wave) * 2654435761u) % span;
    const unsigned lo = LINE ? (unsigned)lane * 16u : (unsigned)(lane >> 2) * 512u + (lane & 3) * 16u;
    const unsigned step = LINE ? 1024u : 8192u;
#pragma unroll 1
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const unsigned off = ((wbase + (unsigned)(it * 16 + j) * step) % span) & ~15u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)&buf[wave][j][0], 16, off + lo,
                                                     0, 0, 0);
            if (j % 4 == 3)   // at most 32 copies in flight
                __builtin_amdgcn_s_waitcnt((32 & 15) | ((32 >> 4) << 14) | (7 << 4) | (15 << 8));
        }
    }
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
}

// LDS reads: every wave keeps reading 1 KiB slices (16 bytes per lane, conflict-free: the 64
// lanes read 1 KiB of consecutive bytes) of a 64 KiB LDS array, eight per iteration, folding the
// values into one register so that nothing is dropped.  WAVES waves per workgroup; with 64 KiB
// per workgroup two workgroups share a CU.
template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) void lds_read_kernel(uint4 *out, int iters) {
    __shared__ uint4 buf[4096];
    for (int i = threadIdx.x; i < 4096; i += 64 * WAVES) buf[i] = uint4{(unsigned)i, 1u, 2u, 3u};
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint4 acc = {0u, 0u, 0u, 0u};
    int base = wave * 512 + lane;
#pragma unroll 1
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const uint4 v = buf[(base + s * 64) & 4095];
            acc.x ^= v.x, acc.y ^= v.y, acc.z ^= v.z, acc.w ^= v.w;
        }
        base += 512;
    }
    out[(size_t)blockIdx.x * 64 * WAVES + threadIdx.x] = acc;
}

}  // namespace
}  // namespace cx

extern "C" int conv_calib_lds_read(void *out, int workgroups, int waves, int iters, void *stream) {
    if (!out || workgroups < 1 || workgroups > (1 << 20) || iters < 1 || (waves != 4 && waves != 8))
        return CONV_E_INVAL;
    uint4 *o = static_cast<uint4 *>(out);
    if (waves == 4)
        hipLaunchKernelGGL(cx::lds_read_kernel<4>, dim3((unsigned)workgroups), dim3(256), 0,
                           (hipStream_t)stream, o, iters);
    else
        hipLaunchKernelGGL(cx::lds_read_kernel<8>, dim3((unsigned)workgroups), dim3(512), 0,
                           (hipStream_t)stream, o, iters);
    return hipGetLastError() == hipSuccess ? CONV_OK : CONV_E_LAUNCH;
}

extern "C" int conv_calib_lds_dma(const void *src, size_t src_bytes, int whole_lines,
                                  int workgroups, int iters, void *stream) {
    if (!src || src_bytes < (1u << 20) || src_bytes > (1ull << 31) - 1 || workgroups < 1 ||
        workgroups > (1 << 20) || iters < 1)
        return CONV_E_INVAL;
    const unsigned char *s = static_cast<const unsigned char *>(src);
    if (whole_lines)
        hipLaunchKernelGGL(cx::lds_dma_kernel<1>, dim3((unsigned)workgroups), dim3(256), 0,
                           (hipStream_t)stream, s, (unsigned)src_bytes, iters);
    else
        hipLaunchKernelGGL(cx::lds_dma_kernel<0>, dim3((unsigned)workgroups), dim3(256), 0,
                           (hipStream_t)stream, s, (unsigned)src_bytes, iters);
    return hipGetLastError() == hipSuccess ? CONV_OK : CONV_E_LAUNCH;
}

extern "C" int conv_calib_mfma_bf16(void *out, int workgroups, int iters, void *stream) {
    if (!out || workgroups < 1 || iters < 1 || workgroups > (1 << 20))
        return CONV_E_INVAL;
    hipLaunchKernelGGL(cx::mfma_loop_kernel, dim3((unsigned)workgroups), dim3(256), 0,
                       (hipStream_t)stream, static_cast<float *>(out), iters);
    return hipGetLastError() == hipSuccess ? CONV_OK : CONV_E_LAUNCH;
}
