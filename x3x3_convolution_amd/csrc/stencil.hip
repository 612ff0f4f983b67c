// Split head, stage 2: the nine-tap spatial stencil over the 112-channel intermediate plane.
//
//   y[n,d,h,w,co] = E( b[co] + sum_{ky,kx} g[n,d,h+g_off+ky-1,w+kx-1,(ky*3+kx)*C_out+co] ),
//   g = 0 outside the plane (the 3x3x3 convolution's spatial zero padding), fp32 sum of the nine
//   bf16/fp16 values, bias in fp32, one round-to-nearest-even on the store.  The plane has
//   gH = H + 2*g_off rows per frame: g_off = 1 carries the Z rows just above and below an output
//   band (head.cu, head_stencil: a band's plane with g_off halo rows each side).
// (FastVideo head.cu: header comment on the value path, and head_stencil_kernel for the channel
// order (i*3+j)*12+c of the plane, i = row tap, j = column tap.)
//
// Every element of g is read by exactly one output, so the kernel is a pure HBM stream: 224 B
// in per position, 2*C_out B out.  Instead of nine scattered 24-byte reads per position, a
// workgroup walks down a 64-column strip of one frame and keeps a ring of three staged rows of g
// (66 positions with the column halo) in LDS; each row is fetched once with coalesced 16-byte
// buffer loads (pieces outside the plane read as zero) and output row h is summed from the ring
// rows h-1, h, h+1.
//
// Keeping HBM busy: two rows are in flight in registers while a third is summed (two register
// sets that alternate, so no copy between them ever waits on a load), the plane is read with
// non-temporal loads (it streams through once; caching it only evicts other lines), and the
// bands are tall: the grid is sized to be resident at once at two workgroups per CU (the LDS
// would hold three; two measured faster), so a band re-reads only its two halo rows and pays its
// pipeline start once.
#include "common.hpp"
#include "launch.hpp"

namespace cx {

namespace {

constexpr int kStripW = 64;                        // output columns per workgroup
constexpr int kRowPos = kStripW + 2;               // staged positions per row (column halo)
constexpr int kPosPieces = kHeadPlaneChannels / 8;  // 16-byte pieces per position (14)
constexpr int kRowPieces = kRowPos * kPosPieces;   // 924
constexpr int kRPT = (kRowPieces + 255) / 256;     // pieces per thread and row (4)
constexpr int kResidentPerCU = 2;                  // workgroups per CU the grid is sized for
constexpr uint32_t kNoPiece = 0xFFFFFFFFu;         // an offset past any buffer range
constexpr int kCacheNT = 2;                        // buffer-op cache policy: non-temporal

struct StencilKArgs {
    const u16 *g;
    const u16 *bias;
    u16 *y;
    int N, D, H, W, C_out;
    int g_off, gH;     // plane rows above the first output row; plane rows per frame
    int rows_per_band, bands, strips;
    uint32_t total_wg;
};

template <bool BF, int EPI, bool VEC>
__global__ __launch_bounds__(256) void head_stencil_kernel(StencilKArgs a) {
    using E = Elem<BF>;
    // rows padded to 1024 pieces so that every thread stores all of its pieces (no branches)
    __shared__ uint4 ring[3][kRPT * 256];
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
    const size_t row_elems = (size_t)a.W * kHeadPlaneChannels;
    const u16 *gframe = a.g + ((size_t)n * a.D + d) * a.gH * row_elems;   // plane row 0
    const uint32_t row_bytes = (uint32_t)(row_elems * 2);
    // one frame of y
    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.y + ((size_t)n * a.D + d) * a.H * a.W * a.C_out), (short)0,
        (int)((uint32_t)a.H * (uint32_t)a.W * (uint32_t)a.C_out * 2u), 0x00020000);

    // This thread's pieces of a staged row: piece i = tid + 256*j is 16-byte piece i % 14 of
    // staged position i / 14 (column w0 - 1 + i / 14); the byte offset inside a plane row is the
    // same for every row, kNoPiece where the column is outside the frame or i is past the row.
    uint32_t off[kRPT];
#pragma unroll
    for (int j = 0; j < kRPT; ++j) {
        const int i = tid + 256 * j;
        const int p = i / kPosPieces, q = i - p * kPosPieces;
        const int w = w0 - 1 + p;
        off[j] = (i < kRowPieces && (unsigned)w < (unsigned)a.W)
                     ? (uint32_t)(w * kHeadPlaneChannels * 2 + q * 16) : kNoPiece;
    }
    // Row h (output coordinates) into registers.  Rows outside the plane, and rows past the
    // band's lower halo row h_end, read as zero without touching memory (a resource of size 0),
    // so the loads are issued unconditionally.
    auto fetch = [&](int h, uint4 (&r)[kRPT]) __attribute__((always_inline)) {
        const int gr = h + a.g_off;
        const bool ok = (unsigned)gr < (unsigned)a.gH && h <= h_end;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(gframe + (size_t)(ok ? gr : 0) * row_elems), (short)0,
            ok ? (int)row_bytes : 0, 0x00020000);
        // non-temporal: every piece of the plane is read once (the halo rows twice, far apart)
#pragma unroll
        for (int j = 0; j < kRPT; ++j)
            r[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off[j], 0, kCacheNT));
    };
    auto commit = [&](int h, const uint4 (&r)[kRPT]) __attribute__((always_inline)) {
        uint4 *dst = ring[(h + 3) % 3];
#pragma unroll
        for (int j = 0; j < kRPT; ++j) dst[tid + j * 256] = r[j];
    };

    // thread -> (output column p, group of 4 output channels)
    const int groups = (a.C_out + 3) / 4;
    const int p = tid / groups, grp = tid - p * groups;
    const bool active = p < kStripW && w0 + p < a.W;
    const int c0 = grp * 4;
    float b4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        b4[i] = (a.bias != nullptr && c0 + i < a.C_out) ? E::to_f32(a.bias[c0 + i]) : 0.f;
    const int pc = active ? p : 0;     // inactive threads read a valid slot and store nothing
    const uint32_t col_off = (uint32_t)(((w0 + pc) * a.C_out + c0) * 2);

    // Output row h (stored only when h < h_end: the loop runs whole pairs of rows).
    auto sum_row = [&](int h) __attribute__((always_inline)) {
        float s[4] = {b4[0], b4[1], b4[2], b4[3]};
#pragma unroll
        for (int ky = 0; ky < 3; ++ky) {
            const u16 *row = reinterpret_cast<const u16 *>(ring[(h - 1 + ky + 3) % 3]);
#pragma unroll
            for (int kx = 0; kx < 3; ++kx) {
                const u16 *src = row + (pc + kx) * kHeadPlaneChannels + (ky * 3 + kx) * a.C_out + c0;
                if (VEC) {
                    const uint2 v = *reinterpret_cast<const uint2 *>(src);
                    s[0] += E::to_f32((u16)(v.x & 0xffffu));
                    s[1] += E::to_f32((u16)(v.x >> 16));
                    s[2] += E::to_f32((u16)(v.y & 0xffffu));
                    s[3] += E::to_f32((u16)(v.y >> 16));
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) s[i] += E::to_f32(src[min(i, a.C_out - 1 - c0)]);
                }
            }
        }
        u16 o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = E::from_f32(epilogue<EPI>(s[i]));
        const bool st = active && h < h_end;
        const uint32_t yo = (uint32_t)h * (uint32_t)a.W * (uint32_t)a.C_out * 2u + col_off;
        if (VEC) {
            const uint32_t v0 = (uint32_t)o[0] | ((uint32_t)o[1] << 16);
            const uint32_t v1 = (uint32_t)o[2] | ((uint32_t)o[3] << 16);
            __builtin_amdgcn_raw_buffer_store_b32(v0, yr, st ? yo : kNoPiece, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(v1, yr, st ? yo + 4u : kNoPiece, 0, 0);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __builtin_amdgcn_raw_buffer_store_b16(o[i], yr, st && c0 + i < a.C_out ? yo + 2u * i : kNoPiece,
                                                      0, 0);
        }
    };
    // One output row: publish row h+1 (held in r) to the ring, refill r with row h+3, sum row h.
    auto step = [&](int h, uint4 (&r)[kRPT]) __attribute__((always_inline)) {
        __syncthreads();      // nobody still reads slot (h+1) mod 3 = (h-2) mod 3
        commit(h + 1, r);
        __syncthreads();
        fetch(h + 3, r);
        sum_row(h);
    };

    uint4 ra[kRPT], rb[kRPT];
    fetch(h_begin - 1, ra);
    fetch(h_begin, rb);
    commit(h_begin - 1, ra);
    fetch(h_begin + 1, ra);
    commit(h_begin, rb);
    fetch(h_begin + 2, rb);
    // the ring holds rows h-1 and h; ra (row h+1) and rb (row h+2) are in flight
    for (int h = h_begin; h < h_end; h += 2) {
        step(h, ra);
        step(h + 1, rb);
    }
}

}  // namespace

hipError_t launch_head_stencil(const StencilParams &p, hipStream_t stream) {
    StencilKArgs a{};
    a.g = static_cast<const u16 *>(p.g);
    a.bias = static_cast<const u16 *>(p.bias);
    a.y = static_cast<u16 *>(p.y);
    a.N = p.N, a.D = p.D, a.H = p.H, a.W = p.W, a.C_out = p.C_out;
    a.g_off = p.g_off, a.gH = p.H + 2 * p.g_off;
    // a plane row and a frame of y are each addressed by one buffer resource (32-bit range)
    if ((long long)p.W * kHeadPlaneChannels * 2 >= (1ll << 31) ||
        (long long)p.H * p.W * p.C_out * 2 >= (1ll << 31))
        return hipErrorInvalidValue;
    a.strips = (p.W + kStripW - 1) / kStripW;
    // Bands of rows: as few as keep the grid within 256 CUs x kResidentPerCU workgroups, so
    // every band is as tall as possible; more columns than that run as several rounds of
    // whole-height bands.
    const long long cols = (long long)p.N * p.D * a.strips;
    long long bands = (256 * kResidentPerCU) / (cols > 0 ? cols : 1);
    if (bands < 1) bands = 1;
    if (bands > p.H) bands = p.H;
    a.rows_per_band = (int)((p.H + bands - 1) / bands);
    a.bands = (p.H + a.rows_per_band - 1) / a.rows_per_band;
    const long long wgs = cols * a.bands;
    a.total_wg = (uint32_t)wgs;
    const dim3 grid((unsigned)wgs), block(256);
#define CX_ST(BFV, EPIV)                                                                  \
    do {                                                                                  \
        if (p.C_out % 4 == 0) head_stencil_kernel<BFV, EPIV, true><<<grid, block, 0, stream>>>(a);  \
        else head_stencil_kernel<BFV, EPIV, false><<<grid, block, 0, stream>>>(a);        \
    } while (0)
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
