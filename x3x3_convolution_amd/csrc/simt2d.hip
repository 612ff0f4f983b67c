// Direct 3x3 convolution, NCHW fp16/bf16, stride 1 or 2, on the vector ALUs of gfx950.
//
// (musetalk-bench patches/taesd_conv.cuh.new: the operator contract in its header comment, and
// the design ideas of taesd_conv3x3_impl / _ocb_impl / _reg_impl -- an input halo staged once in
// shared memory, several output channels per thread so each staged value feeds several weights,
// and a micro-tile of output pixels per thread.)
//
// Re-designed for CDNA4: a workgroup is 4 wave64s.  Each wave owns 16 output channels (OCG
// channel groups per workgroup) and each lane a 2x2 block of output pixels; a lane's 64 fp32
// accumulators take every staged input value four ways (pixels) times sixteen (channels).
// Input channels are consumed in pairs with v_dot2_f32_{f16,bf16} (two products added into an
// fp32 accumulator per instruction), so the LDS halo stores channel pairs (c, c+1) of one pixel
// as one dword, and the weights are staged per chunk as [pair][tap][channel] dwords that a wave
// reads as uniform (broadcast) 16-byte LDS loads.  Input channels stream through LDS in chunks
// of 8 pairs, so any C_in fits.
#include "common.hpp"
#include "launch.hpp"

namespace cx {

namespace {

constexpr int kPairsPerChunk = 8;

struct Simt2dKArgs {
    const u16 *x, *w, *bias;
    u16 *y;
    int N, C_in, C_out, H, W, Hout, Wout;
    int tiles_w, tiles_h, oc_passes;
    uint32_t total_wg;
};

// OCG: 16-channel groups per workgroup (1, 2 or 4); the remaining waves split the pixels.
// Lanes form a 16 x 4 grid of 2x2-pixel blocks: one pixel group is 8 rows x 32 columns.
template <bool BF, int S, int OCG, int EPI>
__global__ __launch_bounds__(256) void simt2d_kernel(Simt2dKArgs a) {
    using E = Elem<BF>;
    typedef typename E::vec2 vec2;
    constexpr int PXG = 4 / OCG;
    constexpr int OCP = OCG * 16;
    constexpr int TH = 8 * PXG, TW = 32;
    constexpr int IH = (TH - 1) * S + 3, IW = (TW - 1) * S + 3;
    constexpr int PR = S + 3;  // input rows/cols one 2x2 block reads
    __shared__ uint32_t s_in[kPairsPerChunk][IH][IW];
    __shared__ __attribute__((aligned(16))) uint32_t s_w[kPairsPerChunk][9][OCP];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ocg = wave % OCG, pxg = wave / OCG;
    const int bx = lane & 15, by = lane >> 4;

    uint32_t lin = xcd_remap(blockIdx.x, a.total_wg);
    const int pass = lin % a.oc_passes;
    lin /= a.oc_passes;
    const int tw = lin % a.tiles_w;
    lin /= a.tiles_w;
    const int th = lin % a.tiles_h;
    const int n = lin / a.tiles_h;
    const int oh0 = th * TH, ow0 = tw * TW;
    const int ih0 = oh0 * S - 1, iw0 = ow0 * S - 1;
    const int oc_base = pass * OCP;
    const int orow = pxg * 8 + by * 2, ocol = bx * 2;  // this lane's block inside the tile

    float acc[16][4];
#pragma unroll
    for (int o = 0; o < 16; ++o) {
        const int co = oc_base + ocg * 16 + o;
        const float b = (a.bias != nullptr && co < a.C_out) ? E::to_f32(a.bias[co]) : 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[o][k] = b;
    }

    const int npairs = (a.C_in + 1) / 2;
    const size_t plane = (size_t)a.H * a.W;
    for (int p0 = 0; p0 < npairs; p0 += kPairsPerChunk) {
        __syncthreads();
        // stage the input halo of this chunk: dword = (channel 2p, channel 2p+1) of one pixel
        for (int i = tid; i < kPairsPerChunk * IH * IW; i += 256) {
            const int cp = i / (IH * IW);
            const int rem = i - cp * (IH * IW);
            const int r = rem / IW, c = rem - r * IW;
            const int ci = 2 * (p0 + cp);
            const int ih = ih0 + r, iw = iw0 + c;
            uint32_t lo = 0, hi = 0;
            if ((unsigned)ih < (unsigned)a.H && (unsigned)iw < (unsigned)a.W) {
                const u16 *src = a.x + ((size_t)n * a.C_in + ci) * plane + (size_t)ih * a.W + iw;
                if (ci < a.C_in) lo = src[0];
                if (ci + 1 < a.C_in) hi = src[plane];
            }
            s_in[cp][r][c] = lo | (hi << 16);
        }
        // stage the weights of this chunk: [pair][tap][channel] dwords
        for (int i = tid; i < kPairsPerChunk * 9 * OCP; i += 256) {
            const int oc = i % OCP;
            const int t = (i / OCP) % 9;
            const int cp = i / (9 * OCP);
            const int co = oc_base + oc, ci = 2 * (p0 + cp);
            uint32_t lo = 0, hi = 0;
            if (co < a.C_out) {
                const u16 *src = a.w + ((size_t)co * a.C_in + ci) * 9 + t;
                if (ci < a.C_in) lo = src[0];
                if (ci + 1 < a.C_in) hi = src[9];
            }
            s_w[cp][t][oc] = lo | (hi << 16);
        }
        __syncthreads();

        const int cpn = min(kPairsPerChunk, npairs - p0);
        for (int cp = 0; cp < cpn; ++cp) {
            vec2 patch[PR][PR];
#pragma unroll
            for (int i = 0; i < PR; ++i)
#pragma unroll
                for (int j = 0; j < PR; ++j)
                    patch[i][j] = __builtin_bit_cast(vec2, s_in[cp][orow * S + i][ocol * S + j]);
#pragma unroll
            for (int t = 0; t < 9; ++t) {
                const int ky = t / 3, kx = t % 3;
                vec2 wv[16];
                const uint4 *wsrc = reinterpret_cast<const uint4 *>(&s_w[cp][t][ocg * 16]);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint4 u = wsrc[q];
                    wv[4 * q + 0] = __builtin_bit_cast(vec2, u.x);
                    wv[4 * q + 1] = __builtin_bit_cast(vec2, u.y);
                    wv[4 * q + 2] = __builtin_bit_cast(vec2, u.z);
                    wv[4 * q + 3] = __builtin_bit_cast(vec2, u.w);
                }
#pragma unroll
                for (int py = 0; py < 2; ++py)
#pragma unroll
                    for (int px = 0; px < 2; ++px) {
                        const vec2 xin = patch[py * S + ky][px * S + kx];
#pragma unroll
                        for (int o = 0; o < 16; ++o)
                            acc[o][py * 2 + px] = E::dot2(xin, wv[o], acc[o][py * 2 + px]);
                    }
            }
        }
    }

    // epilogue: activation, one rounding, NCHW store
#pragma unroll
    for (int o = 0; o < 16; ++o) {
        const int co = oc_base + ocg * 16 + o;
        if (co >= a.C_out) continue;
#pragma unroll
        for (int py = 0; py < 2; ++py) {
            const int oh = oh0 + orow + py;
            if (oh >= a.Hout) continue;
            const int ow = ow0 + ocol;
            u16 *dst = a.y + (((size_t)n * a.C_out + co) * a.Hout + oh) * a.Wout + ow;
            const u16 v0 = E::from_f32(epilogue<EPI>(acc[o][py * 2 + 0]));
            const u16 v1 = E::from_f32(epilogue<EPI>(acc[o][py * 2 + 1]));
            if (ow + 1 < a.Wout && (a.Wout & 1) == 0) {
                *reinterpret_cast<uint32_t *>(dst) = (uint32_t)v0 | ((uint32_t)v1 << 16);
            } else {
                if (ow < a.Wout) dst[0] = v0;
                if (ow + 1 < a.Wout) dst[1] = v1;
            }
        }
    }
}

template <bool BF, int S, int OCG>
void launch_ocg(const Simt2dKArgs &a, int epi, dim3 grid, hipStream_t s) {
    if (epi == EPI_RELU)
        simt2d_kernel<BF, S, OCG, EPI_RELU><<<grid, dim3(256), 0, s>>>(a);
    else if (epi == EPI_CLAMP1)
        simt2d_kernel<BF, S, OCG, EPI_CLAMP1><<<grid, dim3(256), 0, s>>>(a);
    else
        simt2d_kernel<BF, S, OCG, EPI_NONE><<<grid, dim3(256), 0, s>>>(a);
}

template <bool BF, int S>
void launch_stride(Simt2dKArgs a, int ocg, int epi, hipStream_t s) {
    const int TH = 8 * (4 / ocg), TW = 32;
    a.tiles_h = (a.Hout + TH - 1) / TH;
    a.tiles_w = (a.Wout + TW - 1) / TW;
    a.oc_passes = (a.C_out + 16 * ocg - 1) / (16 * ocg);
    const long long wgs = (long long)a.N * a.tiles_h * a.tiles_w * a.oc_passes;
    a.total_wg = (uint32_t)wgs;
    const dim3 grid((unsigned)wgs);
    if (ocg == 1)
        launch_ocg<BF, S, 1>(a, epi, grid, s);
    else if (ocg == 2)
        launch_ocg<BF, S, 2>(a, epi, grid, s);
    else
        launch_ocg<BF, S, 4>(a, epi, grid, s);
}

}  // namespace

hipError_t launch_simt2d(const Simt2dParams &p, hipStream_t stream) {
    Simt2dKArgs a{};
    a.x = static_cast<const u16 *>(p.x);
    a.w = static_cast<const u16 *>(p.w);
    a.bias = static_cast<const u16 *>(p.bias);
    a.y = static_cast<u16 *>(p.y);
    a.N = p.N, a.C_in = p.C_in, a.C_out = p.C_out, a.H = p.H, a.W = p.W;
    a.Hout = p.Hout, a.Wout = p.Wout;
    // channel groups per workgroup: as many as C_out fills, the other waves take more pixels
    const int ocg = p.C_out <= 16 ? 1 : (p.C_out <= 32 ? 2 : 4);
    if (p.bf16) {
        if (p.stride == 1) launch_stride<true, 1>(a, ocg, p.epilogue, stream);
        else launch_stride<true, 2>(a, ocg, p.epilogue, stream);
    } else {
        if (p.stride == 1) launch_stride<false, 1>(a, ocg, p.epilogue, stream);
        else launch_stride<false, 2>(a, ocg, p.epilogue, stream);
    }
    return hipGetLastError();
}

}  // namespace cx
