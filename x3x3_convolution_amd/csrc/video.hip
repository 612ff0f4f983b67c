// The step after the output head: its 12-channel NDHWC output as 8-bit RGB video frames.
//
// [head.cu, header comment: the clamped 12-channel plane is what the video writer consumes;
// commit summary: the decoded RGB video's frames are copied to the host once.]  Channel
// k = 4*c + 2*dy + dx of position (h, w) becomes colour c of pixel (2h + dy, 2w + dx) (a factor-2
// pixel shuffle, colour outermost), and a value v becomes the byte clamp(RNE(127.5*(v + 1)), 0,
// 255) of its exact value (NaN -> 0): [-1, 1] onto [0, 255].  Output (N, D, 2H, 2W, 3) uint8.
//
// HBM-bound streaming (24 bytes in, 12 bytes out per position).  A workgroup takes 256
// consecutive positions of one input row: each thread reads its position's 24 bytes, forms the
// 12 bytes of its 2 x 2 pixel block and puts them into the two output rows staged in LDS; the
// rows then leave in 16-byte stores (the two output rows of the block are 6*nw contiguous bytes
// each).  The code is rgb_code (common.hpp): exact for every fp16/bf16 value.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "launch.hpp"

namespace cx {
namespace {

constexpr int kVidPos = 256;   // positions per workgroup

template <bool BF>
__global__ __launch_bounds__(256) void video_rgb8_kernel(const u16 *__restrict__ y,
                                                         uint8_t *__restrict__ rgb, int H, int W,
                                                         int chunks, bool vec16) {
    using E = Elem<BF>;
    __shared__ __attribute__((aligned(16))) uint8_t rows[2][kVidPos * 6];
    const long long b = blockIdx.x;
    const int chunk = (int)(b % chunks);
    const long long r = b / chunks;              // input row: (n*D + d)*H + h
    const int w0 = chunk * kVidPos;
    const int nw = min(kVidPos, W - w0);
    const int t = threadIdx.x;
    if (t < nw) {
        const uint2 *src = reinterpret_cast<const uint2 *>(y + ((size_t)r * W + w0 + t) * 12);
        uint32_t v[6];
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const uint2 p = src[i];
            v[2 * i] = p.x, v[2 * i + 1] = p.y;
        }
        uint32_t q[12];
#pragma unroll
        for (int k = 0; k < 12; ++k)
            q[k] = rgb_code(E::to_f32((u16)(v[k >> 1] >> (16 * (k & 1)))));
        // pixel (2h + dy, 2w + dx), colour c <- channel 4c + 2dy + dx
#pragma unroll
        for (int dy = 0; dy < 2; ++dy)
#pragma unroll
            for (int dx = 0; dx < 2; ++dx)
#pragma unroll
                for (int c = 0; c < 3; ++c) rows[dy][(2 * t + dx) * 3 + c] = (uint8_t)q[4 * c + 2 * dy + dx];
    }
    __syncthreads();
    // output rows 2h and 2h+1 of this frame, from pixel column 2*w0
    const long long nd = r / H;
    const int h = (int)(r - nd * H);
    uint8_t *dst0 = rgb + ((size_t)(nd * 2 * H + 2 * h) * (2 * (size_t)W) + 2 * (size_t)w0) * 3;
    const size_t row_bytes = (size_t)W * 6;
    const int nbytes = nw * 6;
    if (vec16) {   // rows start 16-byte aligned: whole 16-byte pieces, then the byte tail
        const int pieces = nbytes >> 4;
        for (int i = t; i < 2 * pieces; i += 256) {
            const int dy = i >= pieces, p = i - dy * pieces;
            *reinterpret_cast<uint4 *>(dst0 + dy * row_bytes + 16 * p) =
                *reinterpret_cast<const uint4 *>(&rows[dy][16 * p]);
        }
        const int tail = nbytes - 16 * pieces;
        if (t < 2 * tail) {
            const int dy = t >= tail, i = 16 * pieces + (t - dy * tail);
            dst0[dy * row_bytes + i] = rows[dy][i];
        }
    } else {
        for (int i = t; i < 2 * nbytes; i += 256) {
            const int dy = i >= nbytes, p = i - dy * nbytes;
            dst0[dy * row_bytes + p] = rows[dy][p];
        }
    }
}

}  // namespace

hipError_t launch_video_rgb8(const VideoParams &p, hipStream_t stream) {
    const int chunks = (p.W + kVidPos - 1) / kVidPos;
    const long long wgs = (long long)p.N * p.D * p.H * chunks;
    const bool vec16 = (p.W % 8) == 0 && (reinterpret_cast<uintptr_t>(p.rgb) & 15) == 0;
    const dim3 grid((unsigned)wgs), block(256);
    if (p.bf16)
        video_rgb8_kernel<true><<<grid, block, 0, stream>>>(static_cast<const u16 *>(p.y),
                                                            static_cast<uint8_t *>(p.rgb), p.H,
                                                            p.W, chunks, vec16);
    else
        video_rgb8_kernel<false><<<grid, block, 0, stream>>>(static_cast<const u16 *>(p.y),
                                                             static_cast<uint8_t *>(p.rgb), p.H,
                                                             p.W, chunks, vec16);
    return hipGetLastError();
}

}  // namespace cx
