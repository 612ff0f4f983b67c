// Split head, stage 2: the nine-tap spatial stencil over the 112-channel intermediate plane.
//
//   y[n,d,h,w,co] = E( b[co] + sum_{ky,kx} g[n,d,h+ky-1,w+kx-1,(ky*3+kx)*C_out+co] ),
//   g = 0 outside the plane (the 3x3x3 convolution's spatial zero padding), fp32 sum of the nine
//   bf16/fp16 values, bias in fp32, one round-to-nearest-even on the store.
// (FastVideo head.cu: header comment on the value path, and head_stencil_kernel for the channel
// order (i*3+j)*12+c of the plane, i = row tap, j = column tap.)
//
// Every element of g is read by exactly one output, so the kernel is a pure HBM stream: 224 B
// in per position, 2*C_out B out.  Instead of nine scattered 24-byte reads per position, a
// workgroup walks down a 64-column strip of one frame and keeps a ring of three staged rows of g
// (66 positions with the column halo) in LDS; each row is fetched once with coalesced 16-byte
// loads, and output row h is summed from the ring rows h-1, h, h+1.
#include "common.hpp"
#include "launch.hpp"

namespace cx {

namespace {

constexpr int kStripW = 64;                        // output columns per workgroup
constexpr int kRowPos = kStripW + 2;               // staged positions per row (column halo)
constexpr int kPosPieces = kHeadPlaneChannels / 8;  // 16-byte pieces per position (14)
constexpr int kRowPieces = kRowPos * kPosPieces;   // 924

struct StencilKArgs {
    const u16 *g;
    const u16 *bias;
    u16 *y;
    int N, D, H, W, C_out;
    int rows_per_band, bands, strips;
    uint32_t total_wg;
};

template <bool BF, int EPI>
__global__ __launch_bounds__(256) void head_stencil_kernel(StencilKArgs a) {
    using E = Elem<BF>;
    __shared__ uint4 ring[3][kRowPieces];
    const int tid = threadIdx.x;

    uint32_t lin = xcd_remap(blockIdx.x, a.total_wg);
    const int strip = lin % a.strips;
    lin /= a.strips;
    const int band = lin % a.bands;
    lin /= a.bands;
    const int d = lin % a.D;
    const int n = lin / a.D;
    const int w0 = strip * kStripW;
    const int h_begin = band * a.rows_per_band;
    const int h_end = min(a.H, h_begin + a.rows_per_band);
    const size_t frame = ((size_t)n * a.D + d) * a.H;

    auto stage_row = [&](int h) {
        uint4 *dst = ring[(h + 3) % 3];
        for (int i = tid; i < kRowPieces; i += 256) {
            const int p = i / kPosPieces, q = i - p * kPosPieces;
            const int w = w0 - 1 + p;
            uint4 v = {0u, 0u, 0u, 0u};
            if ((unsigned)h < (unsigned)a.H && (unsigned)w < (unsigned)a.W)
                v = *reinterpret_cast<const uint4 *>(
                    a.g + ((frame + h) * a.W + w) * kHeadPlaneChannels + q * 8);
            dst[i] = v;
        }
    };

    // thread -> (output column p, group of 4 output channels)
    const int groups = (a.C_out + 3) / 4;
    const int p = tid / groups, grp = tid - p * groups;
    const bool active = p < kStripW && w0 + p < a.W;
    const int c0 = grp * 4;
    const bool vec = (a.C_out & 3) == 0;
    float b4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        b4[i] = (a.bias != nullptr && c0 + i < a.C_out) ? E::to_f32(a.bias[c0 + i]) : 0.f;

    stage_row(h_begin - 1);
    stage_row(h_begin);
    for (int h = h_begin; h < h_end; ++h) {
        stage_row(h + 1);
        __syncthreads();
        if (active) {
            float s[4] = {b4[0], b4[1], b4[2], b4[3]};
#pragma unroll
            for (int ky = 0; ky < 3; ++ky) {
                const u16 *row = reinterpret_cast<const u16 *>(ring[(h - 1 + ky + 3) % 3]);
#pragma unroll
                for (int kx = 0; kx < 3; ++kx) {
                    const u16 *src = row + (p + kx) * kHeadPlaneChannels + (ky * 3 + kx) * a.C_out + c0;
                    if (vec) {
                        const uint2 v = *reinterpret_cast<const uint2 *>(src);
                        s[0] += E::to_f32((u16)(v.x & 0xffffu));
                        s[1] += E::to_f32((u16)(v.x >> 16));
                        s[2] += E::to_f32((u16)(v.y & 0xffffu));
                        s[3] += E::to_f32((u16)(v.y >> 16));
                    } else {
                        for (int i = 0; i < 4; ++i)
                            if (c0 + i < a.C_out) s[i] += E::to_f32(src[i]);
                    }
                }
            }
            u16 *dst = a.y + ((frame + h) * a.W + w0 + p) * a.C_out + c0;
            u16 o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = E::from_f32(epilogue<EPI>(s[i]));
            if (vec) {
                uint2 pk;
                pk.x = (uint32_t)o[0] | ((uint32_t)o[1] << 16);
                pk.y = (uint32_t)o[2] | ((uint32_t)o[3] << 16);
                *reinterpret_cast<uint2 *>(dst) = pk;
            } else {
                for (int i = 0; i < 4; ++i)
                    if (c0 + i < a.C_out) dst[i] = o[i];
            }
        }
        __syncthreads();  // ring slot of row h-1 is overwritten next
    }
}

}  // namespace

hipError_t launch_head_stencil(const StencilParams &p, hipStream_t stream) {
    StencilKArgs a{};
    a.g = static_cast<const u16 *>(p.g);
    a.bias = static_cast<const u16 *>(p.bias);
    a.y = static_cast<u16 *>(p.y);
    a.N = p.N, a.D = p.D, a.H = p.H, a.W = p.W, a.C_out = p.C_out;
    a.strips = (p.W + kStripW - 1) / kStripW;
    // Bands of rows: enough workgroups to cover the chip several times, each long enough that
    // the two halo rows it re-reads are a small fraction of its traffic.
    const long long frames = (long long)p.N * p.D;
    int bands = (int)((2048 + frames * a.strips - 1) / (frames * a.strips));
    if (bands < 1) bands = 1;
    if (bands > p.H) bands = p.H;
    a.rows_per_band = (p.H + bands - 1) / bands;
    a.bands = (p.H + a.rows_per_band - 1) / a.rows_per_band;
    const long long wgs = frames * a.bands * a.strips;
    a.total_wg = (uint32_t)wgs;
    const dim3 grid((unsigned)wgs), block(256);
#define CX_ST(BFV, EPIV) head_stencil_kernel<BFV, EPIV><<<grid, block, 0, stream>>>(a)
    if (p.bf16) {
        if (p.epilogue == EPI_RELU) CX_ST(true, EPI_RELU);
        else if (p.epilogue == EPI_CLAMP1) CX_ST(true, EPI_CLAMP1);
        else CX_ST(true, EPI_NONE);
    } else {
        if (p.epilogue == EPI_RELU) CX_ST(false, EPI_RELU);
        else if (p.epilogue == EPI_CLAMP1) CX_ST(false, EPI_CLAMP1);
        else CX_ST(false, EPI_NONE);
    }
#undef CX_ST
    return hipGetLastError();
}

}  // namespace cx
