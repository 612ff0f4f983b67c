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
// with m = (ky*3+kx)*C_out + co (108 rows used, padded to 128), K = 3 * C_in.  [head.cu, header
// comment: the 3x1x1 convolution whose output channels are the nine spatial taps.]
//
// Matrix cores: v_mfma_f32_32x32x16 -- on gfx950 a single wave keeps the matrix pipe full with
// this shape, while the 16x16x32 shape needs two waves per SIMD.  Operand layout used: lane l
// supplies row (A) / column (B) l%32 with the 8 consecutive k values 8*(l/32)..+7; it receives
// accumulator element i at row 8*(i/4) + 4*(l/32) + i%4, column l%32.  (A and B share the k
// assignment, so only the row/column assignment matters.)
//
// A workgroup (4 waves) owns a strip of 128 computed columns of one frame and walks a band of
// rows two rows per step: wave w computes row (w/2) of the step, columns 64*(w%2) .. +63, as a
// 128 x 64 tile (4 x 2 blocks of 32 x 32, 128 accumulators).  K runs as one pipeline over the
// whole band: 32-channel chunks, each with its three temporal taps as k-steps (2 MFMA k16 each).
//   * B (activations): raw buffer loads straight into registers -- rows, columns, frames and
//     channels outside the tensor read as zero without branches (the convolution's zero
//     padding) -- into a ring that runs three k-steps ahead of use.
//   * A (weights, 3 taps x 128 rows x 32 channels = 24 KiB per chunk): staged through registers
//     into LDS buffers (rows of 64 B, 16-byte slots XOR-swizzled so fragment reads spread over
//     the banks), NABUF-1 chunks ahead; the next k-step's fragments are read into registers
//     before the current k-step's MFMAs are issued.
//
// PLANE mode writes Z rounded to the storage type into the 112-channel plane of the split head.
// FUSED mode keeps the last four Z rows of the strip (rounded the same way, 108 channels) in an
// LDS ring and applies the nine-tap stencil + bias + epilogue itself: output row h needs Z rows
// h-1..h+1 and columns w-1..w+1, so a strip computes 128 columns for 126 outputs and a band two
// extra rows.  The split head's 787 MB plane never touches HBM.
// ---------------------------------------------------------------------------------------------
constexpr int kRows = 128;                 // A rows per temporal tap: 4 x 32 (108 used)
constexpr int kMB = 4;                     // 32-row blocks
constexpr int kNB = 2;                     // 32-column blocks per wave
constexpr int kWaveCols = kNB * 32;        // 64 positions per wave
constexpr int kStripPos = 2 * kWaveCols;   // 128 computed columns per strip (two waves)
constexpr int kStepRows = 2;               // Z rows per step (two waves each)
constexpr int kAChunkPieces = 3 * kRows * 4;                 // 1536 16-byte pieces per chunk
constexpr int kAPPT = kAChunkPieces / 256;                   // 6 per thread
constexpr int kPlaneCh = 112;              // rows stored into the split head's plane
constexpr int kZCh = 108;                  // Z channels kept for the stencil (9 taps x 12)
constexpr int kZPosBytes = kZCh * 2;
constexpr int kZRing = 4;                  // Z rows kept: two old + two new
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;  // a buffer offset past any resource range
constexpr int kBRing = 3;                  // B ring slots, one per k-step of a chunk

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
__global__ __launch_bounds__(256, 1) void head_gemm_kernel(HeadGemmKArgs a) {
    using E = Elem<BF>;
    typedef typename E::vec8 vec8;
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    // Weight chunks staged in LDS: three buffers let a chunk be staged two chunks ahead with one
    // barrier per chunk; the fused kernel's LDS also holds the Z ring, so it uses two.
    constexpr int NABUF = FUSED ? 2 : 3;
    __shared__ __attribute__((aligned(16))) uint4 As[NABUF][kAChunkPieces];
    __shared__ __attribute__((aligned(16))) uint8_t Zr[FUSED ? kZRing * kStripPos * kZPosBytes : 16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int zrw = wave >> 1;                // Z row of the step this wave computes
    const int half = wave & 1;                // which 64 columns of the strip

    uint32_t lin = xcd_remap(blockIdx.x, a.total_wg);
    const int od = lin % a.D;          // frames of one (strip, band) are consecutive: they share
    lin /= a.D;                        // input frames, so they run on one XCD's L2
    const int strip = lin % a.strips;
    lin /= a.strips;
    const int band = lin % a.bands;
    const int n = lin / a.bands;

    const int HW = a.H * a.W;
    const int col0 = (FUSED ? strip * a.strip_out - 1 : strip * kStripPos) + half * kWaveCols;
    const int h_begin = band * a.rows_per_band;
    const int h_end = min(a.H, h_begin + a.rows_per_band);
    const int zrow0 = FUSED ? h_begin - 1 : h_begin;
    const int zrows = FUSED ? h_end - h_begin + 2 : h_end - h_begin;
    const int nsteps = (zrows + kStepRows - 1) / kStepRows;
    const int kofs = (lane >> 5) * 8;         // channel offset of this lane's k slice

    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.x + (size_t)n * a.D * HW * a.C_in), (short)0, (int)a.sample_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)a.wp, (short)0, (int)a.wp_bytes, 0x00020000);

    // Byte offset of this lane's B slice = a per-lane column part (fixed for the whole band)
    // + a wave-uniform part for (row, frame, chunk).  Anything outside the tensor gets an offset
    // past the buffer range and reads as zero.
    uint32_t colpart[kNB];
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
        const int w = col0 + nb * 32 + (lane & 31);
        colpart[nb] = (unsigned)w < (unsigned)a.W ? (uint32_t)(w * a.C_in + kofs) * 2u : kOutOfRange;
    }
    // B slices of k-step s = 3 * (global chunk) + kd: [block][k16 half]
    auto load_b = [&](int s, vec8 (&dst)[kNB][2]) {
        const int g = s / 3, kd = s - 3 * g;
        const int st = g / a.nchunks, c = g - st * a.nchunks;
        const int h = zrow0 + st * kStepRows + zrw;
        const int f = od - 1 + kd;
        const uint32_t upart = (uint32_t)(((size_t)f * HW + (size_t)h * a.W) * a.C_in + c * 32) * 2u;
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const bool ok = (unsigned)h < (unsigned)a.H && (unsigned)f < (unsigned)a.D &&
                                c * 32 + k2 * 16 + kofs < a.C_in && colpart[nb] != kOutOfRange;
                const uint32_t off = ok ? upart + colpart[nb] + k2 * 32u : kOutOfRange;
                dst[nb][k2] = __builtin_bit_cast(vec8, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
            }
    };
    uint4 ast[kAPPT];
    auto stage_a = [&](int cc) {
#pragma unroll
        for (int j = 0; j < kAPPT; ++j) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(
                wr, (uint32_t)(cc * kAChunkPieces + tid + j * 256) * 16u, 0, 0);
            ast[j] = uint4{v.x, v.y, v.z, v.w};
        }
    };
    auto publish_a = [&](int buf) {
#pragma unroll
        for (int j = 0; j < kAPPT; ++j) {
            const int i = tid + j * 256, r = i >> 2;
            As[buf][r * 4 + ((i & 3) ^ aswz(r))] = ast[j];
        }
    };
    // A fragments of one k-step: [block][k16 half]
    auto read_a = [&](int buf, int kd, vec8 (&dst)[kMB][2]) {
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const int r = kd * kRows + mb * 32 + (lane & 31);
                const int q = k2 * 2 + (lane >> 5);
                dst[mb][k2] = __builtin_bit_cast(vec8, As[buf][r * 4 + (q ^ aswz(r))]);
            }
    };

    f32x16_t acc[kMB][kNB];
    vec8 bq[kBRing][kNB][2];
    vec8 af[2][kMB][2];

    // prologue: weights of chunks 0 .. NABUF-2 published, B of k-steps 0 .. 2 in flight, A
    // fragments of k-step 0 in registers
#pragma unroll
    for (int c = 0; c < NABUF - 1; ++c) {
        stage_a(c % a.nchunks);
        publish_a(c);
    }
#pragma unroll
    for (int u = 0; u < kBRing; ++u) load_b(u, bq[u]);
    __syncthreads();
    read_a(0, 0, af[0]);

#pragma unroll 1
    for (int step = 0; step < nsteps; ++step) {
#pragma unroll
        for (int i = 0; i < kMB; ++i)
#pragma unroll
            for (int j = 0; j < kNB; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
#pragma unroll 1
        for (int cc = 0; cc < a.nchunks; ++cc) {
            const int g = step * a.nchunks + cc;
            const int buf = g % NABUF;
#pragma unroll
            for (int kd = 0; kd < 3; ++kd) {
                if (kd == 0) stage_a((cc + NABUF - 1) % a.nchunks);
                // the next k-step's A fragments (for kd == 2 the next chunk's, when it is
                // already published) are read before this k-step's MFMAs
                if (kd < 2)
                    read_a(buf, kd + 1, af[(kd + 1) & 1]);
                else if (NABUF == 3)
                    read_a((g + 1) % NABUF, 0, af[1]);
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
                    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
                        for (int nb = 0; nb < kNB; ++nb)
                            acc[mb][nb] = E::mfma32x32x16(af[kd & 1][mb][k2], bq[kd][nb][k2], acc[mb][nb]);
                load_b(3 * g + kd + kBRing, bq[kd]);
                if (kd == 2) {   // end of a chunk: publish the chunk NABUF-1 ahead
                    publish_a((g + NABUF - 1) % NABUF);
                    __syncthreads();
                    if (NABUF == 2) read_a((g + 1) % NABUF, 0, af[0]);
                    else {
#pragma unroll
                        for (int mb = 0; mb < kMB; ++mb) {
                            af[0][mb][0] = af[1][mb][0];
                            af[0][mb][1] = af[1][mb][1];
                        }
                    }
                }
            }
        }

        // ---- the step's Z tile is complete: this wave holds rows 0..127 of 64 columns ----
        const int zr = zrow0 + step * kStepRows + zrw;   // this wave's Z row
        if constexpr (!FUSED) {
            if (zr < h_end) {
#pragma unroll
                for (int nb = 0; nb < kNB; ++nb) {
                    const int w = col0 + nb * 32 + (lane & 31);
                    if (w < a.W) {
                        u16 *dst = a.out + (((size_t)n * a.D + od) * HW + (size_t)zr * a.W + w) * kPlaneCh;
#pragma unroll
                        for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                const int m0 = mb * 32 + 8 * j + 4 * (lane >> 5);
                                if (m0 < kPlaneCh) {
                                    const f32x16_t v = acc[mb][nb];
                                    uint2 pk;
                                    pk.x = (uint32_t)E::from_f32(v[4 * j]) | ((uint32_t)E::from_f32(v[4 * j + 1]) << 16);
                                    pk.y = (uint32_t)E::from_f32(v[4 * j + 2]) | ((uint32_t)E::from_f32(v[4 * j + 3]) << 16);
                                    *reinterpret_cast<uint2 *>(dst + m0) = pk;
                                }
                            }
                    }
                }
            }
        } else {
            // Z rows -> ring slot ((zr - zrow0) mod 4), rounded once to the storage type
            uint8_t *zrow = Zr + ((step * kStepRows + zrw) % kZRing) * (kStripPos * kZPosBytes);
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb) {
                const int pos = half * kWaveCols + nb * 32 + (lane & 31);
#pragma unroll
                for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int m0 = mb * 32 + 8 * j + 4 * (lane >> 5);
                        if (m0 < kZCh) {
                            const f32x16_t v = acc[mb][nb];
                            uint2 pk;
                            pk.x = (uint32_t)E::from_f32(v[4 * j]) | ((uint32_t)E::from_f32(v[4 * j + 1]) << 16);
                            pk.y = (uint32_t)E::from_f32(v[4 * j + 2]) | ((uint32_t)E::from_f32(v[4 * j + 3]) << 16);
                            *reinterpret_cast<uint2 *>(zrow + pos * kZPosBytes + m0 * 2) = pk;
                        }
                    }
            }
            __syncthreads();
            // output rows completed by this step: h in [h_begin+2*step-2, h_begin+2*step-1]
            const int hlo = max(h_begin, h_begin + kStepRows * step - 2);
            const int hhi = min(h_end, h_begin + kStepRows * step);
            const int groups = (a.C_out + 3) / 4;
            const int per_row = a.strip_out * groups;
            const bool vec = (a.C_out & 3) == 0;
            for (int item = tid; item < (hhi - hlo) * per_row; item += 256) {
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
    a.strip_out = p.fused ? kStripPos - 2 : kStripPos;
    a.strips = (p.W + a.strip_out - 1) / a.strip_out;
    // One workgroup per CU is resident (LDS and registers).  Pick the band count that minimises
    // (rounds of 256 workgroups) x (rows a workgroup computes, halo included).
    const long long cols = (long long)p.N * p.D * a.strips;
    const int halo = p.fused ? 2 : 0;
    long long best = -1;
    int best_bands = 1;
    for (int bands = 1; bands <= p.H && bands <= 64; ++bands) {
        const int rpb = (p.H + bands - 1) / bands;
        const int real_bands = (p.H + rpb - 1) / rpb;
        const long long rounds = (cols * real_bands + 255) / 256;
        const long long cost = rounds * (((rpb + halo) + kStepRows - 1) / kStepRows);
        if (best < 0 || cost < best) best = cost, best_bands = real_bands;
    }
    a.rows_per_band = (p.H + best_bands - 1) / best_bands;
    a.bands = (p.H + a.rows_per_band - 1) / a.rows_per_band;
    a.sample_bytes = (uint32_t)((size_t)p.D * p.H * p.W * p.C_in * 2);
    a.wp_bytes = (uint32_t)((size_t)a.nchunks * kAChunkPieces * 16);
    const long long wgs = cols * a.bands;
    a.total_wg = (uint32_t)wgs;
    const dim3 grid((unsigned)wgs), block(256);
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
