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
// where GEMM row m stands for one spatial tap (ky, kx) of one output channel co (108 of 128 rows
// used), K = 3 * C_in.  [head.cu, header comment: the 3x1x1 convolution whose output channels
// are the nine spatial taps.]
//
// Matrix cores: v_mfma_f32_32x32x16 (one wave per SIMD keeps the pipe full with this shape).
// Lane l supplies row (A) / column (B) l%32 with 8 k values (the k half l/32) of a 16-wide k
// slice, and receives accumulator element i at row 8*(i/4) + 4*(l/32) + i%4, column l%32.
//
// Work split: a workgroup is four waves on four consecutive output frames of one (band, strip);
// each wave walks its band one row at a time.  Per row a wave computes a 128 x 128 tile (GEMM rows
// x 128 columns of the row): 4 x 4 blocks of 32 x 32, all 256 accumulators.  Column block nb,
// lane column j holds position p = 4*j + nb of the wave's strip, so the horizontal neighbours of
// a position sit in the same lane (blocks nb-1, nb+1) except at nb = 0 / 3, where they are one
// lane away (a DPP wavefront shift).
//
// Row roles (set by the weight packing): accumulator register i of block mb in lane half h is
// slot t = 16*mb + i of that half; slot t < 54 holds spatial tap t/6 of output channel 6*h + t%6.
// So every lane owns six output channels of its four positions, with all nine taps in registers.
//
// K order: 64-channel chunks (one 128-byte cache line of a position), and in a chunk the three
// temporal taps one after the other, each as four k16 slices.  Slice s takes channels
// 32*h + 8*s .. +7 from lane half h, so for one tap the four slices of a position are the four
// consecutive 16-byte pieces of the lane's half line.  A tap runs as two half-taps (column blocks
// 0-1, then 2-3), each four slices of 4 x 2 MFMAs.
//   * B (activations): raw buffer loads straight into registers; the four pieces of a lane's
//     half line are loaded back to back, so every cache line is fetched whole, once.  Rows,
//     columns, frames and channels outside the tensor read as zero without branches (the
//     convolution's zero padding).  A ring of four half-taps: each half-tap starts by loading
//     the half-tap three ahead.
//   * A (weights, 3 taps x 128 rows x 64 channels = 48 KiB per chunk): copied global -> LDS by
//     the buffer unit itself (LDS DMA, no registers), two buffers, each chunk issued a whole
//     chunk before it is needed.  The packing stores every 128-byte row with its eight 16-byte
//     pieces already XOR-permuted, so the fragment reads spread over the LDS banks.
//
// PLANE mode stores Z, rounded to the storage type, as the 112-channel plane of the split head.
// FUSED mode applies the nine-tap stencil in registers: the horizontal taps combine neighbouring
// positions, the vertical taps are carried from row to row (two fp32 partial sums per output),
// and bias + epilogue are applied once per output.  Output row h needs Z rows h-1 .. h+1 and
// columns w-1 .. w+1, so a strip computes 128 columns for 126 outputs and a band two extra rows.
// Nothing of Z is rounded or stored: the fused head keeps fp32 from the GEMM to the epilogue.
// ---------------------------------------------------------------------------------------------
constexpr int kMB = 4;                  // 32-row blocks: 128 GEMM rows per temporal tap
constexpr int kNB = 4;                  // 32-column blocks per wave
constexpr int kWavePos = 32 * kNB;      // 128 positions per wave and row
constexpr int kSlices = 4;              // k16 slices per tap of a 64-channel chunk
constexpr int kHalves = 6;              // half-taps per chunk
constexpr int kRing = 4;                // B ring depth in half-taps
constexpr int kLoadsPerHalf = 2 * kSlices;   // B loads per half-tap
constexpr int kDmaPerWave = kHeadChunkPieces / 256;  // 12 LDS-DMA copies of 1 KiB per wave
constexpr int kHalfCo = 6;              // output channels per lane half
constexpr int kPlaneCh = kHeadPlaneChannels;
constexpr uint32_t kOff = 0xFFFFFFFFu;  // an offset past any buffer range; saturating adds keep it

// s_waitcnt immediates: vmcnt is split over bits 3:0 and 15:14; expcnt / lgkmcnt left open.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);
// Every half-tap starts with its B loads.  The copy of chunk g+1 is issued at the barrier before
// the last slice of chunk g-1 and must be complete at the same point of chunk g: the operations
// a wave issues in between are the B loads of the six half-taps of chunk g.
constexpr int kVmAfterCopy = kLoadsPerHalf * kHalves;
static_assert(kVmAfterCopy < 64, "vmcnt holds 6 bits");

struct HeadGemmKArgs {
    const u16 *x;
    const u16 *wp;
    const u16 *bias;
    u16 *out;          // the plane (PLANE) or y (FUSED)
    int N, C_in, C_out, D, H, W;
    int nchunks;       // 64-channel chunks per Z row, even (the padding reads zeros)
    int rows_per_band, bands, strips, strip_out, fgroups;
    uint32_t sample_bytes;  // bytes of one sample of x (buffer-resource range)
    uint32_t wp_bytes;
    uint32_t total_wg;
};

// Workgroup barrier without a memory fence (the waits before it are explicit), kept in place
// by the compiler.
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }
// Marks an accumulator block as redefined here (no code): values of the block are unpacked into
// VGPRs only after this point, so an epilogue that walks the blocks in order keeps one or a few
// blocks unpacked at a time instead of all 256 accumulators.
__device__ __forceinline__ void touch(f32x16_t &v) { asm volatile("" : "+a"(v)::"memory"); }

// CO12: C_out == 12, every lane stores its six channels as one 12-byte vector.
template <bool BF, bool FUSED, int EPI, bool CO12>
__global__ __launch_bounds__(256, 1) void head_gemm_kernel(HeadGemmKArgs a) {
    using E = Elem<BF>;
    typedef typename E::vec8 vec8;
    typedef __attribute__((address_space(3))) void lds_void;
    // Two weight buffers (even / odd chunks), separate objects so the compiler can tell that the
    // copy into one never overlaps the fragment reads from the other.
    __shared__ __attribute__((aligned(16))) uint4 As0[kHeadChunkPieces];
    __shared__ __attribute__((aligned(16))) uint4 As1[kHeadChunkPieces];
    // FUSED: the two carried partial sums of every lane's 6 channels x 4 positions, per wave
    // (cA: the output row before the next Z row, cB: the output row of the next Z row), as
    // float4 {cA0..3}, {cA4, cA5, cB0, cB1}, {cB2..5}.  Private to each wave.
    __shared__ float4 carry[FUSED ? 4 : 1][kNB][3][64];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane & 31, hh = lane >> 5;

    uint32_t lin = xcd_remap(blockIdx.x, a.total_wg);
    const int fg = lin % a.fgroups;    // frame groups of one (strip, band) are consecutive: they
    lin /= a.fgroups;                  // share input frames, so they run on one XCD's L2
    const int strip = lin % a.strips;
    lin /= a.strips;
    const int band = lin % a.bands;
    const int n = lin / a.bands;
    const int od = fg * 4 + wave;      // this wave's output frame (>= D: computes, stores nothing)

    const int HW = a.H * a.W;
    const int w0 = FUSED ? strip * a.strip_out - 1 : strip * kWavePos;   // column of position 0
    const int h_begin = band * a.rows_per_band;
    const int h_end = min(a.H, h_begin + a.rows_per_band);
    const int zrow0 = FUSED ? h_begin - 1 : h_begin;
    const int nsteps = (h_end - h_begin) + (FUSED ? 2 : 0);   // Z rows, the same in every wave
    const int nch = a.nchunks;

    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.x + (size_t)n * a.D * HW * a.C_in), (short)0, (int)a.sample_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)a.wp, (short)0, (int)a.wp_bytes, 0x00020000);

    // Byte offset of a B piece = a per-lane column part (fixed for the whole band) + a part for
    // (row, frame, chunk, lane half, slice), added with saturation so that either part out of
    // range makes the load read zero.
    uint32_t colpart[kNB];
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
        const int w = w0 + 4 * j + nb;
        colpart[nb] = (unsigned)w < (unsigned)a.W ? (uint32_t)(w * a.C_in) * 2u : kOff;
    }
    // per-slice offsets of one tap (Z row st, chunk c, tap kd) for this lane
    auto tap_offsets = [&](int st, int c, int kd, uint32_t (&up)[kSlices]) {
        const int row = zrow0 + st, f = od - 1 + kd;
        const bool ok = (unsigned)row < (unsigned)a.H && (unsigned)f < (unsigned)a.D;
        const uint32_t base = (uint32_t)((((size_t)f * HW + (size_t)row * a.W) * a.C_in + c * 64 + 32 * hh) * 2u);
#pragma unroll
        for (int sl = 0; sl < kSlices; ++sl)
            up[sl] = ok && c * 64 + 32 * hh + 8 * sl < a.C_in ? base + 16u * sl : kOff;
    };
    // B of a half-tap: blocks 2*hp and 2*hp+1, each the four slices of the lane's half line
    // back to back
    auto load_half = [&](int st, int c, int kd, int hp, vec8 (&dst)[2][kSlices]) {
        uint32_t up[kSlices];
        tap_offsets(st, c, kd, up);
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int sl = 0; sl < kSlices; ++sl)
                dst[b][sl] = __builtin_bit_cast(vec8, __builtin_amdgcn_raw_buffer_load_b128(
                    xr, __builtin_elementwise_add_sat(up[sl], colpart[2 * hp + b]), 0, 0));
    };
    // LDS DMA of packed weight chunk cc into buffer dstbuf: each wave copies 12 KiB.  Chunks past
    // the packed ones (the even padding) lie past the resource range and copy zeros.
    auto copy_a = [&](int cc, uint4 *dstbuf) {
#pragma unroll
        for (int q = 0; q < kDmaPerWave; ++q) {
            const int piece = wave * (kDmaPerWave * 64) + q * 64;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                wr, (lds_void *)&dstbuf[piece], 16,
                (uint32_t)((cc * kHeadChunkPieces + piece + lane) * 16), 0, 0, 0);
        }
    };
    const int swz = head_lds_swizzle(j);   // the swizzle of rows kd*128 + mb*32 + j
    // A fragments of tap kd, slice sl: piece 4*hh + sl of each row
    auto read_a = [&](const uint4 *srcbuf, int kd, int sl, vec8 (&dst)[kMB]) {
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) {
            const int r = kd * 128 + mb * 32 + j;
            dst[mb] = __builtin_bit_cast(vec8, srcbuf[r * 8 + ((4 * hh + sl) ^ swz)]);
        }
    };

    f32x16_t acc[kMB][kNB];
    vec8 bq[kRing][2][kSlices];   // [half-tap slot][block of the pair][slice]
    vec8 af[2][kMB];
    const f32x16_t zero = {};

    // FUSED: the bias of the lane's six output channels; carried sums start at zero
    float b6[kHalfCo];
#pragma unroll
    for (int c = 0; c < kHalfCo; ++c) {
        const int co = kHalfCo * hh + c;
        b6[c] = (FUSED && a.bias != nullptr && co < a.C_out) ? E::to_f32(a.bias[co]) : 0.f;
    }
    if constexpr (FUSED) {
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
            for (int k = 0; k < 3; ++k) carry[wave][nb][k][lane] = float4{0.f, 0.f, 0.f, 0.f};
    }

    // (row, chunk, tap) of the tap `ahead` taps after tap kd of chunk c of Z row st
    auto tap_after = [&](int st, int c, int kd, int ahead, int &ost, int &oc, int &okd) {
        okd = kd + ahead;
        oc = c;
        ost = st;
        while (okd >= 3) {
            okd -= 3;
            if (++oc == nch) oc = 0, ++ost;
        }
    };

    // ---- prologue: weight chunks 0 and 1 copied (0 complete), B of half-taps 0..2 loading ----
    copy_a(0, As0);
    copy_a(1, As1);
    load_half(0, 0, 0, 0, bq[0]);
    load_half(0, 0, 0, 1, bq[1]);
    load_half(0, 0, 1, 0, bq[2]);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(kDmaPerWave + (kRing - 1) * kLoadsPerHalf));
    wg_barrier();
    read_a(As0, 0, 0, af[0]);

    // Chunk g of the band is channel chunk g % nch of Z row g / nch.  Each pass of the loop body
    // runs one even chunk (buffer As0) and the following odd chunk (As1): twelve half-taps; the
    // ring slot of half-tap i of the pass is i % 4.
#pragma unroll 1
    for (int st = 0; st < nsteps; ++st) {
#pragma unroll 1
        for (int c2 = 0; c2 < nch; c2 += 2) {
#pragma unroll
          for (int i = 0; i < 2 * kHalves; ++i) {
            const int half = i / kHalves;                 // even / odd chunk of the pass
            const int kd = (i % kHalves) / 2, hp = i % 2;
            uint4 *const cbuf = half == 0 ? As0 : As1;   // this chunk's weights
            uint4 *const nbuf = half == 0 ? As1 : As0;   // the next chunk's
            {   // half-tap i+3 into the slot half-tap i-1 has finished with
                const int ahead_hp = (hp + kRing - 1) % 2;
                const int ahead_taps = (hp + kRing - 1) / 2;
                int lst, lc, lkd;
                tap_after(st, c2 + half, kd, ahead_taps, lst, lc, lkd);
                load_half(lst, lc, lkd, ahead_hp, bq[(i + kRing - 1) % kRing]);
            }
#pragma unroll
            for (int sl = 0; sl < kSlices; ++sl) {
                const int u = 2 * kSlices * kd + kSlices * hp + sl;   // 0 .. 23 within the chunk
                const bool last = u == 2 * kSlices * 3 - 1;
                const int cur = sl & 1;
                if (last) {
                    // Publish chunk g+1: its copy (issued one chunk ago, here) is complete once at
                    // most kVmAfterCopy younger operations are outstanding.  This wave's reads of
                    // chunk g are done (the last ones were issued in the previous slice), so
                    // after the barrier chunk g's buffer takes chunk g+2.
                    __builtin_amdgcn_s_waitcnt(waitcnt_vm(kVmAfterCopy));
                    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
                    wg_barrier();
                    const int wc = c2 + half + 2;    // weight chunk of chunk g+2
                    copy_a(wc < nch ? wc : wc - nch, cbuf);
                }
                // the next slice's A fragments: of this half-tap, the next half-tap (same tap:
                // the same fragments again for blocks 2-3; next tap), or the next chunk's
                if (!last) {
                    const int nsl = (sl + 1) % kSlices;
                    const int nkd = sl + 1 < kSlices ? kd : (hp == 1 ? kd + 1 : kd);
                    read_a(cbuf, nkd, nsl, af[cur ^ 1]);
                } else {
                    read_a(nbuf, 0, 0, af[cur ^ 1]);
                }
                if (i == 0 && sl == 0 && c2 == 0) {
#pragma unroll
                    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
                        for (int b = 0; b < 2; ++b)
                            acc[mb][2 * hp + b] = E::mfma32x32x16(af[cur][mb], bq[i % kRing][b][sl], zero);
                } else if (i == 1 && sl == 0 && c2 == 0) {
#pragma unroll
                    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
                        for (int b = 0; b < 2; ++b)
                            acc[mb][2 * hp + b] = E::mfma32x32x16(af[cur][mb], bq[i % kRing][b][sl], zero);
                } else {
#pragma unroll
                    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
                        for (int b = 0; b < 2; ++b)
                            acc[mb][2 * hp + b] = E::mfma32x32x16(af[cur][mb], bq[i % kRing][b][sl], acc[mb][2 * hp + b]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
          }
        }

        // ---- row zr of Z is complete in this wave's accumulators ----
        // The epilogues walk the accumulator blocks in order and read each value once, so only
        // one or two blocks are unpacked into registers at a time.
        const int zr = zrow0 + st;
        const size_t frame = (size_t)n * a.D + od;
        if constexpr (!FUSED) {
            if (zr < h_end && od < a.D) {
#pragma unroll
                for (int nb = 0; nb < kNB; ++nb) {
                    const int w = w0 + 4 * j + nb;
                    u16 *dst = a.out + (frame * HW + (size_t)zr * a.W + w) * kPlaneCh;
#pragma unroll
                    for (int mb = 0; mb < kMB; ++mb) touch(acc[mb][nb]);
#pragma unroll
                    for (int tap = 0; tap < 9; ++tap) {
                        u16 r6[kHalfCo];
#pragma unroll
                        for (int c = 0; c < kHalfCo; ++c) {
                            const int t = tap * kHalfCo + c;
                            r6[c] = E::from_f32(acc[t >> 4][nb][t & 15]);
                        }
                        if (w < a.W) {
                            if constexpr (CO12) {
                                uint3 v;
                                v.x = (uint32_t)r6[0] | ((uint32_t)r6[1] << 16);
                                v.y = (uint32_t)r6[2] | ((uint32_t)r6[3] << 16);
                                v.z = (uint32_t)r6[4] | ((uint32_t)r6[5] << 16);
                                *reinterpret_cast<uint3 *>(dst + tap * 12 + kHalfCo * hh) = v;
                            } else {
#pragma unroll
                                for (int c = 0; c < kHalfCo; ++c) {
                                    const int co = kHalfCo * hh + c;
                                    if (co < a.C_out) dst[tap * a.C_out + co] = r6[c];
                                }
                            }
                        }
                    }
                    if (CO12 && w < a.W && hh == 0) *reinterpret_cast<uint2 *>(dst + 108) = uint2{0u, 0u};
                }
            }
        } else {
            // Output row zr-1 = cA + taps ky=2 of row zr; the next cA = cB + taps ky=1; the next
            // cB = taps ky=0.  Position p takes tap (ky, kx) from position p + kx - 1: block
            // nb + kx - 1 of the same lane, or across a lane (wavefront shift) from block 3 for
            // kx = 0 at block 0, and from block 0 for kx = 2 at block 3.  The lanes that cross a
            // lane half or the wave hold halo columns, which are not stored.
            const int ho = zr - 1;   // the output row this Z row completes
            const bool emit = ho >= h_begin && ho < h_end && od < a.D;
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb) {
                float sum[3][kHalfCo];   // [ky]: this row's taps ky for this block's positions
#pragma unroll
                for (int ky = 0; ky < 3; ++ky)
#pragma unroll
                    for (int c = 0; c < kHalfCo; ++c) sum[ky][c] = 0.f;
#pragma unroll
                for (int kx = 0; kx < 3; ++kx) {
                    const int src = nb + kx - 1;
                    const int sb = src < 0 ? kNB - 1 : (src >= kNB ? 0 : src);
#pragma unroll
                    for (int mb = 0; mb < kMB; ++mb) {
                        bool used = false;   // does block (mb, sb) hold a slot with this kx?
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int t = 16 * mb + i;
                            if (t < 9 * kHalfCo && (t / kHalfCo) % 3 == kx) used = true;
                        }
                        if (!used) continue;
                        touch(acc[mb][sb]);
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int t = 16 * mb + i;
                            if (t >= 9 * kHalfCo || (t / kHalfCo) % 3 != kx) continue;
                            const int ky = t / kHalfCo / 3, c = t % kHalfCo;
                            float v = acc[mb][sb][i];
                            if (src < 0)   // left neighbour: lane l-1
                                v = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                    0, __builtin_bit_cast(int, v), 0x138, 0xF, 0xF, false));
                            else if (src >= kNB)   // right neighbour: lane l+1
                                v = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                    0, __builtin_bit_cast(int, v), 0x130, 0xF, 0xF, false));
                            sum[ky][c] += v;
                        }
                    }
                }
                const float4 k0 = carry[wave][nb][0][lane], k1 = carry[wave][nb][1][lane],
                             k2 = carry[wave][nb][2][lane];
                const float cA[kHalfCo] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y};
                const float cB[kHalfCo] = {k1.z, k1.w, k2.x, k2.y, k2.z, k2.w};
                float o[kHalfCo], nA[kHalfCo];
#pragma unroll
                for (int c = 0; c < kHalfCo; ++c) {
                    o[c] = cA[c] + sum[2][c];
                    nA[c] = cB[c] + sum[1][c];
                }
                carry[wave][nb][0][lane] = float4{nA[0], nA[1], nA[2], nA[3]};
                carry[wave][nb][1][lane] = float4{nA[4], nA[5], sum[0][0], sum[0][1]};
                carry[wave][nb][2][lane] = float4{sum[0][2], sum[0][3], sum[0][4], sum[0][5]};
                const int p = 4 * j + nb;
                const int w = w0 + p;
                if (emit && p >= 1 && p <= a.strip_out && w < a.W) {
                    u16 r6[kHalfCo];
#pragma unroll
                    for (int c = 0; c < kHalfCo; ++c) r6[c] = E::from_f32(epilogue<EPI>(o[c] + b6[c]));
                    u16 *dst = a.out + (frame * HW + (size_t)ho * a.W + w) * a.C_out;
                    if constexpr (CO12) {
                        uint3 v;
                        v.x = (uint32_t)r6[0] | ((uint32_t)r6[1] << 16);
                        v.y = (uint32_t)r6[2] | ((uint32_t)r6[3] << 16);
                        v.z = (uint32_t)r6[4] | ((uint32_t)r6[5] << 16);
                        *reinterpret_cast<uint3 *>(dst + kHalfCo * hh) = v;
                    } else {
#pragma unroll
                        for (int c = 0; c < kHalfCo; ++c)
                            if (kHalfCo * hh + c < a.C_out) dst[kHalfCo * hh + c] = r6[c];
                    }
                }
            }
        }
    }
    // no LDS copy may still be in flight when the workgroup's LDS is released
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
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
    const int packed_chunks = (p.C_in + 63) / 64;
    a.nchunks = (packed_chunks + 1) & ~1;   // the kernel runs chunks in pairs
    a.strip_out = p.fused ? kWavePos - 2 : kWavePos;
    a.strips = (p.W + a.strip_out - 1) / a.strip_out;
    a.fgroups = (p.D + 3) / 4;
    // One workgroup per CU is resident (accumulators fill the register file).  Pick the band count
    // that minimises (rounds of 256 workgroups) x (rows a wave computes, halo included).
    const long long cols = (long long)p.N * a.fgroups * a.strips;
    const int halo = p.fused ? 2 : 0;
    long long best = -1;
    int best_bands = 1;
    for (int bands = 1; bands <= p.H && bands <= 256; ++bands) {
        const int rpb = (p.H + bands - 1) / bands;
        const int real_bands = (p.H + rpb - 1) / rpb;
        const long long rounds = (cols * real_bands + 255) / 256;
        const long long cost = rounds * (rpb + halo);
        if (best < 0 || cost < best) best = cost, best_bands = real_bands;
    }
    a.rows_per_band = (p.H + best_bands - 1) / best_bands;
    a.bands = (p.H + a.rows_per_band - 1) / a.rows_per_band;
    a.sample_bytes = (uint32_t)((size_t)p.D * p.H * p.W * p.C_in * 2);
    a.wp_bytes = (uint32_t)((size_t)packed_chunks * kHeadChunkPieces * 16);
    const long long wgs = cols * a.bands;
    a.total_wg = (uint32_t)wgs;
    const dim3 grid((unsigned)wgs), block(256);
#define CX_HG(BFV, FV, EPIV)                                                          \
    do {                                                                              \
        if (p.C_out == 12) head_gemm_kernel<BFV, FV, EPIV, true><<<grid, block, 0, stream>>>(a);  \
        else head_gemm_kernel<BFV, FV, EPIV, false><<<grid, block, 0, stream>>>(a);    \
    } while (0)
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
