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

    // Row h of the plane (66 positions incl. the column halo) is fetched into registers one
    // iteration before it is needed and written to its ring slot (h mod 3) after a barrier.
    constexpr int RPT = (kRowPieces + 255) / 256;
    uint4 rstg[RPT];
    auto fetch_row = [&](int h) {
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            const int i = tid + j * 256;
            uint4 v = {0u, 0u, 0u, 0u};
            if (i < kRowPieces) {
                const int p = i / kPosPieces, q = i - p * kPosPieces;
                const int w = w0 - 1 + p;
                if ((unsigned)h < (unsigned)a.H && (unsigned)w < (unsigned)a.W)
                    v = *reinterpret_cast<const uint4 *>(
                        a.g + ((frame + h) * a.W + w) * kHeadPlaneChannels + q * 8);
            }
            rstg[j] = v;
        }
    };
    auto commit_row = [&](int h) {
        uint4 *dst = ring[(h + 3) % 3];
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            const int i = tid + j * 256;
            if (i < kRowPieces) dst[i] = rstg[j];
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

    fetch_row(h_begin - 1);
    commit_row(h_begin - 1);
    fetch_row(h_begin);
    commit_row(h_begin);
    fetch_row(h_begin + 1);
    for (int h = h_begin; h < h_end; ++h) {
        __syncthreads();      // nobody still reads slot (h+1) mod 3 = (h-2) mod 3
        commit_row(h + 1);
        __syncthreads();
        if (h + 1 < h_end) fetch_row(h + 2);  // in flight while row h is summed
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
    }
}

// ---------------------------------------------------------------------------------------------
// The head's temporal GEMM: Z[p, m] = sum_{kd, ci} Wt[m, (kd, ci)] * X[frame(p)-1+kd, h(p), w(p), ci]
// with m = (ky*3+kx)*C_out + co over 112 rows (108 used), K = 3 * C_in.  [head.cu, header
// comment: the 3x1x1 convolution whose output channels are the nine spatial taps.]
//
// A workgroup (4 waves) owns a strip of 80 computed columns of one frame and walks down a band
// of rows, four rows (one per wave) per step.  Per step each wave accumulates a 112 x 80 tile
// (7 x 5 MFMA 16x16x32 blocks) over K.  The K loop is one continuous pipeline over all steps of
// the band: 32-channel chunks, each with its three temporal taps as k32 steps.
//   * B (activations): every lane fetches its 16-byte fragment slices with raw buffer loads --
//     out-of-range positions, frames and channels read as zero without branches (the
//     convolution's zero padding) -- three k-steps ahead of use into a register ring.
//   * A (weights, 3 taps x 112 rows x 32 channels = 21 KiB per chunk): fetched one chunk ahead
//     into registers and written to one of two LDS buffers (rows of 64 B with an XOR swizzle of
//     the 16-byte slots, so the 16 rows one fragment read touches fall on distinct banks).
//
// PLANE mode writes Z rounded to the storage type into the 112-channel plane of the split head.
// FUSED mode keeps the last six Z rows of the strip (rounded the same way, 108 channels) in an LDS
// ring and applies the nine-tap stencil + bias + epilogue itself: output row h needs Z rows
// h-1..h+1 and columns w-1..w+1, so a strip computes 80 columns for 78 outputs and a band
// computes two extra rows.  The split head's 787 MB plane never touches HBM.
// ---------------------------------------------------------------------------------------------
constexpr int kRows = 112;                 // 7 x 16 A rows
constexpr int kMB = 7;
constexpr int kNBW = 5;                    // 5 x 16 = 80 positions per wave
constexpr int kStripPos = kNBW * 16;       // computed columns per strip
constexpr int kAChunkPieces = 3 * kRows * 4;                 // 1344 16-byte pieces per chunk
constexpr int kWavesPerRow = 1;           // 1: a wave owns all 112 rows of its Z row;
                                           // 2: two waves split them as 4 + 3 blocks
constexpr int kThreads = 256 * kWavesPerRow;
constexpr int kAPPT = (kAChunkPieces + kThreads - 1) / kThreads;   // A pieces per thread
constexpr int kABufPieces = kAPPT * kThreads;                      // room for the over-fetch
constexpr int kMBW = kWavesPerRow == 1 ? kMB : 4;                  // A row blocks per wave
constexpr int kZCh = 108;                  // Z channels kept for the stencil (9 taps x 12)
constexpr int kZPosBytes = kZCh * 2;
constexpr int kZRing = 6;
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;  // a buffer offset past any resource range
constexpr int kChunksPerIter = 2;          // chunks of B fragments in flight
constexpr int kBRing = 3 * kChunksPerIter; // ring slots, one per k-step (chunk, temporal tap)

struct HeadGemmKArgs {
    const u16 *x;
    const u16 *wp;
    const u16 *bias;
    u16 *out;          // the plane (PLANE) or y (FUSED)
    int N, C_in, C_out, D, H, W;
    int nchunks;
    int rows_per_band, bands, strips, strip_out;
    uint32_t sample_bytes;  // bytes of one sample of x (buffer-resource range)
    uint32_t wp_bytes;
    uint32_t total_wg;
};

__device__ __forceinline__ int aswz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

template <bool BF, bool FUSED, int EPI>
__global__ __launch_bounds__(kThreads, 1) void head_gemm_kernel(HeadGemmKArgs a) {
    using E = Elem<BF>;
    typedef typename E::vec8 vec8;
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    __shared__ __attribute__((aligned(16))) uint4 As[2][kABufPieces];
    __shared__ __attribute__((aligned(16))) uint8_t Zr[FUSED ? kZRing * kStripPos * kZPosBytes : 16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int zrw = wave & 3;                 // Z row of the step this wave computes
    const int mhalf = wave >> 2;              // with two waves per row: blocks 0-3 or 4-6
    const int mb0 = mhalf * kMBW;
    const int mcnt = mhalf == 0 ? kMBW : kMB - kMBW;

    uint32_t lin = xcd_remap(blockIdx.x, a.total_wg);
    const int od = lin % a.D;          // frames of one (strip, band) are consecutive: they share
    lin /= a.D;                        // input frames, so they run on one XCD's L2
    const int strip = lin % a.strips;
    lin /= a.strips;
    const int band = lin % a.bands;
    const int n = lin / a.bands;

    const int HW = a.H * a.W;
    const int col0 = FUSED ? strip * a.strip_out - 1 : strip * kStripPos;
    const int h_begin = band * a.rows_per_band;
    const int h_end = min(a.H, h_begin + a.rows_per_band);
    const int zrow0 = FUSED ? h_begin - 1 : h_begin;
    const int zrows = FUSED ? h_end - h_begin + 2 : h_end - h_begin;
    const int nsteps = (zrows + 3) / 4;
    const int kofs = (lane >> 4) * 8;

    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.x + (size_t)n * a.D * HW * a.C_in), (short)0, (int)a.sample_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)a.wp, (short)0, (int)a.wp_bytes, 0x00020000);

    // Byte offset of this lane's B slice = a per-lane column part (fixed for the whole band)
    // + a wave-uniform part for (row, frame, chunk).  Anything outside the tensor -- rows,
    // columns, frames in the temporal padding, channels past C_in -- gets an offset past the
    // buffer range and reads as zero.
    uint32_t colpart[kNBW];
#pragma unroll
    for (int nb = 0; nb < kNBW; ++nb) {
        const int w = col0 + nb * 16 + (lane & 15);
        colpart[nb] = (unsigned)w < (unsigned)a.W ? (uint32_t)(w * a.C_in + kofs) * 2u : kOutOfRange;
    }
    auto load_b = [&](int s, vec8 (&dst)[kNBW]) {   // k-step s = 3 * (global chunk) + kd
        const int g = s / 3, kd = s - 3 * g;
        const int st = g / a.nchunks, c = g - st * a.nchunks;
        const int h = zrow0 + st * 4 + zrw;
        const int f = od - 1 + kd;
        const bool ok = (unsigned)h < (unsigned)a.H && (unsigned)f < (unsigned)a.D &&
                        c * 32 + kofs < a.C_in;
        const uint32_t upart = (uint32_t)(((size_t)f * HW + (size_t)h * a.W) * a.C_in + c * 32) * 2u;
#pragma unroll
        for (int nb = 0; nb < kNBW; ++nb) {
            const uint32_t off = (ok && colpart[nb] != kOutOfRange) ? upart + colpart[nb] : kOutOfRange;
            dst[nb] = __builtin_bit_cast(vec8, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
        }
    };
    auto stage_a = [&](int cc, uint4 (&dst)[kAPPT]) {
#pragma unroll
        for (int j = 0; j < kAPPT; ++j) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(
                wr, (uint32_t)(cc * kAChunkPieces + tid + j * kThreads) * 16u, 0, 0);
            dst[j] = uint4{v.x, v.y, v.z, v.w};
        }
    };
    auto publish_a = [&](int buf, const uint4 (&src)[kAPPT]) {
#pragma unroll
        for (int j = 0; j < kAPPT; ++j) {
            const int i = tid + j * kThreads, r = i >> 2;
            As[buf][r * 4 + ((i & 3) ^ aswz(r))] = src[j];
        }
    };

    f32x4_t acc[kMBW][kNBW];
    vec8 bq[kBRing][kNBW];       // B ring over k-steps (k-step = (chunk, temporal tap))
    uint4 ast[kAPPT];

    // prologue: weights of chunk 0, B of k-steps 0 .. kBRing-1
    stage_a(0, ast);
#pragma unroll
    for (int u = 0; u < kBRing; ++u) load_b(u, bq[u]);
    publish_a(0, ast);
    __syncthreads();

    // Per step: a 112 x 80 x (4 rows) Z tile, K walked kChunksPerIter chunks per iteration so
    // that ring slots and temporal taps are compile-time constants.  After k-step s's MFMAs its
    // ring slot is refilled with k-step s + kBRing -- the next step's first k-steps are already
    // in flight while this step's epilogue runs.  Loads past the band's last k-step are harmless
    // (they fetch rows of the next band, or read as zero past the tensor), so there are no
    // per-lane branches in the pipeline.  nchunks is a multiple of kChunksPerIter (the host pads
    // C_in with zero chunks).
#pragma unroll 1
    for (int step = 0; step < nsteps; ++step) {
#pragma unroll
        for (int i = 0; i < kMBW; ++i)
#pragma unroll
            for (int j = 0; j < kNBW; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
        for (int cp = 0; cp < a.nchunks; cp += kChunksPerIter) {
            const int g0 = step * a.nchunks + cp;
#pragma unroll
            for (int u = 0; u < kBRing; ++u) {
                const int kd = u % 3;
                const int cc = cp + u / 3;
                const int buf = (g0 + u / 3) & 1;
                if (kd == 0) stage_a(cc + 1 == a.nchunks ? 0 : cc + 1, ast);
#pragma unroll
                for (int mb = 0; mb < kMBW; ++mb) {
                    if (mb < mcnt) {
                        const int r = kd * kRows + (mb0 + mb) * 16 + (lane & 15);
                        const vec8 A = __builtin_bit_cast(vec8, As[buf][r * 4 + ((lane >> 4) ^ aswz(r))]);
#pragma unroll
                        for (int nb = 0; nb < kNBW; ++nb)
                            acc[mb][nb] = E::mfma16x16x32(A, bq[u][nb], acc[mb][nb]);
                    }
                }
                load_b(3 * g0 + u + kBRing, bq[u]);
                if (kd == 2) {   // end of a chunk: publish the next chunk's weights
                    publish_a(buf ^ 1, ast);
                    __syncthreads();
                }
            }
        }

        // ---- the step's Z tile is complete ----
        const int zr = zrow0 + step * 4 + zrw;   // this wave's Z row
        if constexpr (!FUSED) {
#pragma unroll
            for (int nb = 0; nb < kNBW; ++nb) {
                const int w = col0 + nb * 16 + (lane & 15);
                if (zr < h_end && w < a.W) {
                    u16 *dst = a.out + (((size_t)n * a.D + od) * HW + (size_t)zr * a.W + w) * kHeadPlaneChannels;
#pragma unroll
                    for (int mb = 0; mb < kMBW; ++mb) {
                        if (mb < mcnt) {
                            const int m0 = (mb0 + mb) * 16 + 4 * (lane >> 4);
                            const f32x4_t v = acc[mb][nb];
                            uint2 pk;
                            pk.x = (uint32_t)E::from_f32(v[0]) | ((uint32_t)E::from_f32(v[1]) << 16);
                            pk.y = (uint32_t)E::from_f32(v[2]) | ((uint32_t)E::from_f32(v[3]) << 16);
                            *reinterpret_cast<uint2 *>(dst + m0) = pk;
                        }
                    }
                }
            }
        } else {
            // Z rows -> ring slot ((zr - zrow0) mod 6), rounded once to the storage type
            uint8_t *zrow = Zr + ((step * 4 + zrw) % kZRing) * (kStripPos * kZPosBytes);
#pragma unroll
            for (int nb = 0; nb < kNBW; ++nb) {
                const int pos = nb * 16 + (lane & 15);
#pragma unroll
                for (int mb = 0; mb < kMBW; ++mb) {
                    const int m0 = (mb0 + mb) * 16 + 4 * (lane >> 4);
                    if (mb < mcnt && m0 < kZCh) {
                        const f32x4_t v = acc[mb][nb];
                        uint2 pk;
                        pk.x = (uint32_t)E::from_f32(v[0]) | ((uint32_t)E::from_f32(v[1]) << 16);
                        pk.y = (uint32_t)E::from_f32(v[2]) | ((uint32_t)E::from_f32(v[3]) << 16);
                        *reinterpret_cast<uint2 *>(zrow + pos * kZPosBytes + m0 * 2) = pk;
                    }
                }
            }
            __syncthreads();
            // output rows completed by this step: h in [h_begin+4*step-2, h_begin+4*step+1]
            const int hlo = max(h_begin, h_begin + 4 * step - 2);
            const int hhi = min(h_end, h_begin + 4 * step + 2);
            const int groups = (a.C_out + 3) / 4;
            const int per_row = a.strip_out * groups;
            const bool vec = (a.C_out & 3) == 0;
            for (int item = tid; item < (hhi - hlo) * per_row; item += kThreads) {
                const int hr = item / per_row;
                const int rem = item - hr * per_row;
                const int c = rem / groups, grp = rem - c * groups;
                const int h = hlo + hr;
                const int w = strip * a.strip_out + c;
                if (w >= a.W) continue;
                const int c0 = grp * 4;
                float s4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    s4[i] = (a.bias != nullptr && c0 + i < a.C_out) ? E::to_f32(a.bias[c0 + i]) : 0.f;
#pragma unroll
                for (int ky = 0; ky < 3; ++ky) {
                    const uint8_t *zrow2 = Zr + ((h - h_begin + ky) % kZRing) * (kStripPos * kZPosBytes);
#pragma unroll
                    for (int kx = 0; kx < 3; ++kx) {
                        const u16 *src = reinterpret_cast<const u16 *>(zrow2 + (c + kx) * kZPosBytes) +
                                         (ky * 3 + kx) * a.C_out + c0;
                        if (vec) {
                            const uint2 v = *reinterpret_cast<const uint2 *>(src);
                            s4[0] += E::to_f32((u16)(v.x & 0xffffu));
                            s4[1] += E::to_f32((u16)(v.x >> 16));
                            s4[2] += E::to_f32((u16)(v.y & 0xffffu));
                            s4[3] += E::to_f32((u16)(v.y >> 16));
                        } else {
                            for (int i = 0; i < 4; ++i)
                                if (c0 + i < a.C_out) s4[i] += E::to_f32(src[i]);
                        }
                    }
                }
                u16 o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = E::from_f32(epilogue<EPI>(s4[i]));
                u16 *dst = a.out + (((size_t)n * a.D + od) * HW + (size_t)h * a.W + w) * a.C_out + c0;
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
        }
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

namespace cx {

hipError_t launch_head_gemm(const HeadGemmParams &p, hipStream_t stream) {
    HeadGemmKArgs a{};
    a.x = static_cast<const u16 *>(p.x);
    a.wp = static_cast<const u16 *>(p.wp);
    a.bias = static_cast<const u16 *>(p.bias);
    a.out = static_cast<u16 *>(p.out);
    a.N = p.N, a.C_in = p.C_in, a.C_out = p.C_out, a.D = p.D, a.H = p.H, a.W = p.W;
    a.nchunks = (p.C_in + 31) / 32;
    a.nchunks = (a.nchunks + kChunksPerIter - 1) / kChunksPerIter * kChunksPerIter;
    a.strip_out = p.fused ? kStripPos - 2 : kStripPos;
    a.strips = (p.W + a.strip_out - 1) / a.strip_out;
    // one workgroup per CU is resident (LDS and registers); aim for about one full wave of
    // workgroups, each band long enough that its two halo rows are a small overhead
    const long long cols = (long long)p.N * p.D * a.strips;
    int bands = (int)((256 + cols - 1) / cols);
    if (bands < 1) bands = 1;
    if (bands > p.H) bands = p.H;
    a.rows_per_band = (p.H + bands - 1) / bands;
    a.bands = (p.H + a.rows_per_band - 1) / a.rows_per_band;
    a.sample_bytes = (uint32_t)((size_t)p.D * p.H * p.W * p.C_in * 2);
    a.wp_bytes = (uint32_t)((size_t)((p.C_in + 31) / 32) * kAChunkPieces * 16);
    const long long wgs = cols * a.bands;
    a.total_wg = (uint32_t)wgs;
    const dim3 grid((unsigned)wgs), block(kThreads);
#define CX_HG(BFV, FV, EPIV) head_gemm_kernel<BFV, FV, EPIV><<<grid, block, 0, stream>>>(a)
    if (!p.fused) {
        if (p.bf16) CX_HG(true, false, EPI_NONE);
        else CX_HG(false, false, EPI_NONE);
    } else if (p.bf16) {
        if (p.epilogue == EPI_RELU) CX_HG(true, true, EPI_RELU);
        else if (p.epilogue == EPI_CLAMP1) CX_HG(true, true, EPI_CLAMP1);
        else CX_HG(true, true, EPI_NONE);
    } else {
        if (p.epilogue == EPI_RELU) CX_HG(false, true, EPI_RELU);
        else if (p.epilogue == EPI_CLAMP1) CX_HG(false, true, EPI_CLAMP1);
        else CX_HG(false, true, EPI_NONE);
    }
#undef CX_HG
    return hipGetLastError();
}

}  // namespace cx
