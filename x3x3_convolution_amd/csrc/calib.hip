// Measurement aid, not part of the convolution: the rate the matrix cores reach on a loop of
// nothing but bf16 32x32x16 MFMAs with register operands.  The benchmark reports it beside the
// plain-copy rate as what this machine's matrix cores sustain (clock and power included); the
// roofline fractions are still taken against the published peak.
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

}  // namespace
}  // namespace cx

extern "C" int conv_calib_mfma_bf16(void *out, int workgroups, int iters, void *stream) {
    if (!out || workgroups < 1 || iters < 1 || workgroups > (1 << 20))
        return CONV_E_INVAL;
    hipLaunchKernelGGL(cx::mfma_loop_kernel, dim3((unsigned)workgroups), dim3(256), 0,
                       (hipStream_t)stream, static_cast<float *>(out), iters);
    return hipGetLastError() == hipSuccess ? CONV_OK : CONV_E_LAUNCH;
}
