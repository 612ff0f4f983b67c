// The head's temporal GEMM on the matrix cores, in two modes: PLANE writes the split head's
// 112-channel intermediate plane (the split's stage 1; stage 2, the stencil, is stencil.hip), and
// FUSED applies the nine-tap stencil, bias and epilogue in registers so that only y (or the RGB
// frames) reaches HBM.
// (FastVideo head.cu: header comment -- the 27-tap output convolution as a 3x1x1 temporal
// convolution whose output channels are the nine spatial taps, then a stencil sum.)
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace cx {

namespace {

// ---------------------------------------------------------------------------------------------
// The head's temporal GEMM: Z[p, m] = sum_{kd, ci} Wt[m, (kd, ci)] * X[frame(p)-1+kd, h(p), w(p), ci]
// where GEMM row m stands for one spatial tap (ky, kx) of one output channel co (108 rows: 96 on
// 32-row blocks, 12 in a 16-row tile), K = 3 * C_in.  [head.cu, header comment: the 3x1x1 convolution whose output channels
// are the nine spatial taps.]
//
// Matrix cores: v_mfma_f32_32x32x16 (one wave per SIMD keeps the pipe full with this shape).
// Lane l supplies row (A) / column (B) l%32 with 8 k values (the k half l/32) of a 16-wide k
// slice, and receives accumulator element i at row 8*(i/4) + 4*(l/32) + i%4, column l%32.
// The ninth spatial tap (12 rows) runs on v_mfma_f32_16x16x32 instead of a fourth 32-row block
// (of which it would use 12 rows): lane l supplies row / column l%16 with k values 8*(l/16) ..
// +7 of a 32-wide k range and receives element i at row 4*(l/16) + i, column l%16.
//
// Work split: a workgroup is four waves on four consecutive output frames and one row range of
// the strips (a band of rows of one strip, or the end of one strip and the start of the next --
// the ranges are cut to near-equal cost so that every CU takes one); each wave walks its band one
// row at a time.  Per row a wave computes GEMM rows x 128 columns of
// the row: 3 x 4 blocks of 32 x 32 (192 accumulators) and 8 tiles of 16 x 16 (32).  Column block nb,
// lane column j holds position p = 4*j + nb of the wave's strip, so the horizontal neighbours of
// a position sit in the same lane (blocks nb-1, nb+1) except at nb = 0 / 3, where they are one
// lane away (a DPP wavefront shift).
//
// Row roles (set by the weight packing): accumulator register i of block mb < 3 in lane half h
// is slot t = 16*mb + i of that half, spatial tap t/6 of output channel 6*h + t%6 (taps 0..7).
// Tap 8 is a 16-row tile per 16 columns: row 8*h + c (c < 6) is output channel 6*h + c.  The two
// tiles of a 32-column block take their B operands from the block's two k16 fragments of one
// temporal tap, rearranged by one lane swap (v_permlane16_swap: columns 0..15 of both slices in
// one register, 16..31 in the other, k pieces in the order 0, 2, 1, 3); one more swap of their
// results puts rows 8*h .. 8*h+7 of column j into lane j + 32*h.  So every lane owns six output channels of
// its four positions, with all nine taps in registers.
//
// K runs in stages of 32 channels; a stage holds the three temporal taps, each as two k16 slices
// (six steps of 3 x 4 32-row MFMAs, plus the tap-8 tiles' 2 x 4 after each odd step).  Both operands of a stage are copied global -> LDS by the buffer
// unit itself (LDS DMA: no registers, 1 KiB per instruction) into one of two buffer pairs:
//   * A (weights): 3 taps x 128 rows x 32 channels = 24 KiB, contiguous in the packing, which
//     already holds the LDS order.
//   * B (activations): the 128 positions of the row in the six input frames the four output
//     frames read (frames f0-1 .. f0+4), 32 channels each = 48 KiB.  Output frame f0+w reads
//     input frames w, w+1, w+2 of the window, so the three waves that share an input frame
//     share one copy of it.  Rows, columns, frames and channels outside the tensor copy zeros
//     (the convolution's zero padding); the copies need no branches.
// An A or B row is 64 bytes = four 16-byte pieces, stored XOR-permuted by (row/4) % 4 (A) or
// (column j/4) % 4 (B): the 32 rows / columns a fragment read takes fall on distinct LDS banks.
// A fragment read is a per-lane part (row or column, piece) plus a compile-time offset.
//
// A wave never waits for a copy it just issued: the copies of stage g+1 are issued one stage
// ahead, and a single barrier per stage, placed before the stage's last step, publishes them to
// every wave (each wave first waits for its own copies) and frees the buffers of stage g (every
// wave has its last fragments of stage g in registers): the copies of stage g+2 go out right after
// it, interleaved one by one with the last step's MFMAs, and the first fragments of stage g+1 are
// read while those MFMAs run.  The copy offsets are formed without branches.
//
// PLANE mode stores Z, rounded to the storage type, as the 112-channel plane of the split head.
// FUSED mode applies the nine-tap stencil in registers.  The vertical taps are summed by the
// matrix cores themselves: the weights come in three row versions, and Z row zr takes version
// zr mod 3, in which the accumulator slot of (kx, channel) in one of three rotating accumulator
// sets holds the vertical tap that output row zr - 1, zr or zr + 1 needs -- so the three Z rows
// an output row reads all add into the same registers.  When an output row is complete its set
// is read out: the horizontal taps combine neighbouring positions, bias + epilogue are applied
// once per output, and the set is cleared for the row three further on.  Output row h needs Z
// rows h-1 .. h+1 and columns w-1 .. w+1, so a strip computes 128 columns for 126 outputs and a
// band two extra rows.  Nothing of Z is rounded or stored: the fused head keeps fp32 from the
// GEMM to the epilogue.
// ---------------------------------------------------------------------------------------------
constexpr int kMB32 = 3;                // blocks on the 32x32 matrix cores (taps 0..7)
constexpr int kRow8 = 32 * kMB32;       // first LDS row of the tap-8 tile (16 rows)
constexpr int kNB = 4;                  // 32-column blocks per wave
constexpr int kWavePos = 32 * kNB;      // 128 positions per wave and row
constexpr int kSteps = 6;               // k16 steps per stage: 3 temporal taps x 2 slices
constexpr int kInFrames = 6;            // input frames of a workgroup's four output frames
constexpr int kBPieces = kInFrames * kWavePos * 4;   // 16-byte pieces of a stage's B window
constexpr int kCopyA = kHeadChunkPieces / 256;       // LDS-DMA copies of 1 KiB per wave: 6
constexpr int kCopyB = kBPieces / 256;               // 12
constexpr int kHalfCo = 6;              // output channels per lane half
constexpr int kPlaneCh = kHeadPlaneChannels;
constexpr uint32_t kOff = 0xFFFFFFFFu;  // an offset past any buffer range; saturating adds keep it
constexpr int kMaxRanges = kHeadMaxRanges;   // row ranges per (sample, frame group)

// s_waitcnt immediates: vmcnt is split over bits 3:0 and 15:14; expcnt / lgkmcnt left open.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);
static_assert(kCopyA + kCopyB < 64, "vmcnt holds 6 bits");

struct HeadGemmKArgs {
    const u16 *x;
    const u16 *wp;
    const u16 *bias;
    u16 *out;          // the plane (PLANE) or y (FUSED)
    int N, C_in, C_out, D, H, W;   // D, H: output extent
    int D_in, H_in, d_org, h_org;  // input region (see ConvRegion)
    int d_lo, d_hi, h_lo, h_hi;
    int nchunks;       // 32-channel stages per Z row, even (the padding reads zeros)
    int strips, strip_out, fgroups;
    int ranges;        // row ranges per (sample, frame group)
    uint32_t window_bytes;  // bytes of the six input frames of a workgroup (buffer-resource range)
    uint32_t wp_bytes;
    uint32_t total_wg;
    // Row range g covers positions [bound[g], bound[g+1]) of the strip-major (strip, output row)
    // order of one frame group: output row h of strip s is position s*H + h.
    int bound[kMaxRanges + 1];
};

// 0.f through an asm the compiler cannot look into
__device__ __forceinline__ float opaque_zero() {
    float z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
    return z;
}
// v_permlane16_swap of one register pair: rows (16 lanes) 1 and 3 of a trade places with rows 0
// and 2 of b.  Written out, since the compiler has merged separate swaps of different registers
// into one; the waits cover the reads of values the preceding instructions just wrote.
__device__ __forceinline__ void lane_swap16(float &a, float &b) {
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
// v_permlane32_swap of one register pair: lanes 32..63 of a trade places with lanes 0..31 of b
// (so with a = b = v, lane l of b (l < 32) and of a (l >= 32) holds v of lane l ^ 32).  Written
// out like lane_swap16.
__device__ __forceinline__ void lane_swap32(uint32_t &a, uint32_t &b) {
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
// n mod 3 in 0..2 for any int n
__device__ __forceinline__ int mod3(int n) { return ((n % 3) + 3) % 3; }
// a + b saturated at 2^32 - 1 (one VALU instruction: the add's clamp bit); b uniform.  An
// all-ones operand (an invalid part of a copy offset) stays past every buffer range.
__device__ __forceinline__ uint32_t add_sat(uint32_t a, uint32_t b) {
    uint32_t r;
    asm("v_add_u32_e64 %0, %1, %2 clamp" : "=v"(r) : "v"(a), "s"(b));
    return r;
}
// Workgroup barrier without a memory fence (the waits before it are explicit), kept in place
// by the compiler.
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }
// Marks an accumulator block as redefined here (no code): values of the block are unpacked into
// VGPRs only after this point, so an epilogue that walks the blocks in order keeps one or a few
// blocks unpacked at a time instead of all 256 accumulators.
__device__ __forceinline__ void touch(f32x16_t &v) { asm volatile("" : "+a"(v)::"memory"); }
__device__ __forceinline__ void touch(f32x4_t &v) { asm volatile("" : "+a"(v)::"memory"); }

// Swaps rows (16 lanes) 1 and 3 of a with rows 0 and 2 of b, in every register of a tile.
__device__ __forceinline__ void swap_rows16(f32x4_t &a, f32x4_t &b) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 p = __builtin_bit_cast(u32x4, a), q = __builtin_bit_cast(u32x4, b);
    u32x4 x, y;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const auto r = __builtin_amdgcn_permlane16_swap(p[i], q[i], false, false);
        x[i] = r[0];
        y[i] = r[1];
    }
    a = __builtin_bit_cast(f32x4_t, x);
    b = __builtin_bit_cast(f32x4_t, y);
}
// The tap-8 tiles' B operands from the two k16 fragments s0, s1 of a 32-column block (rows of
// 16 lanes: s0 = [c0-15 k0-7 | c16-31 k0-7 | c0-15 k8-15 | c16-31 k8-15], s1 likewise for k16-31):
// one row swap gives lo = columns 0..15 as [k0-7 | k16-23 | k8-15 | k24-31] and hi = columns
// 16..31 in the same k order (the tile's A operand takes its k pieces in that order too).
template <typename vec8>
__device__ __forceinline__ void tile_operands(vec8 s0, vec8 s1, vec8 &lo, vec8 &hi) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 p = __builtin_bit_cast(u32x4, s0), q = __builtin_bit_cast(u32x4, s1);
    u32x4 x, y;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const auto t = __builtin_amdgcn_permlane16_swap(p[d], q[d], false, false);
        x[d] = t[0];
        y[d] = t[1];
    }
    lo = __builtin_bit_cast(vec8, x);
    hi = __builtin_bit_cast(vec8, y);
}

// CO12: C_out == 12, every lane stores its six channels as one 12-byte vector.  RGB (FUSED and
// CO12 only): instead of y, the 8-bit RGB pixels of the video step -- each value rounded to the
// storage type first, then coded (rgb_code); position (h, w) gives pixels (2h+dy, 2w+dx), colour
// c from channel 4c + 2dy + dx.  Lane half 0 (channels 0..5) writes pixel row 2h, half 1
// (channels 6..11) row 2h+1; each takes the two codes it lacks from the other half.
template <bool BF, bool FUSED, int EPI, bool CO12, bool RGB = false>
__global__ __launch_bounds__(256, 1) void head_gemm_kernel(HeadGemmKArgs a) {
    using E = Elem<BF>;
    typedef typename E::vec8 vec8;
    typedef __attribute__((address_space(3))) void lds_void;
    // Two buffer pairs (even / odd stages), separate objects so the compiler can tell that the
    // copies into one never overlap the fragment reads from the other.
    __shared__ __attribute__((aligned(16))) uint4 As0[kHeadChunkPieces];
    __shared__ __attribute__((aligned(16))) uint4 As1[kHeadChunkPieces];
    __shared__ __attribute__((aligned(16))) uint4 Bs0[kBPieces];
    __shared__ __attribute__((aligned(16))) uint4 Bs1[kBPieces];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane & 31, hh = lane >> 5;

    uint32_t lin = xcd_remap(blockIdx.x, a.total_wg);
    const int fg = lin % a.fgroups;    // frame groups of one row range are consecutive: they
    lin /= a.fgroups;                  // share input frames, so they run on one XCD's L2
    const int range = lin % a.ranges;
    const int n = lin / a.ranges;
    const int f0 = fg * 4;             // the group's first output frame
    const int od = f0 + wave;          // this wave's output frame (>= D: computes, stores nothing)

    const int HW = a.H * a.W;
    const int nch = a.nchunks;
    // x through the six input frames the group's window covers: window frame i is input frame
    // fw0 + i.  fw0 may lie before the first frame (or the window past the last one); those frames
    // are never addressed (their copies take an offset past the range), so only the address
    // arithmetic of the base reaches outside x.  Any number of frames works: only the window must
    // fit the 32-bit range.
    const int fw0 = f0 - 1 + a.d_org;
    const long long frame_elems = (long long)a.H_in * a.W * a.C_in;
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)((uintptr_t)a.x + (uintptr_t)((((long long)n * a.D_in + fw0) * frame_elems) * 2)),
        (short)0, (int)a.window_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)a.wp, (short)0, (int)a.wp_bytes, 0x00020000);
    // FUSED: y (or the RGB frames) through the group's four output frames f0 .. f0+3 (frames past
    // the last one are never stored to)
    const size_t frame0 = (size_t)n * a.D + f0;
    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
        RGB ? (void *)(reinterpret_cast<uint8_t *>(a.out) + frame0 * HW * 12)
            : (void *)(a.out + frame0 * HW * a.C_out),
        (short)0, RGB ? (int)(4 * HW * 12) : (int)(4 * HW * a.C_out * 2), 0x00020000);

    const int bpiece = (lane & 3) ^ ((lane >> 4) & 3);
    const uint32_t frame_bytes = (uint32_t)a.H_in * (uint32_t)a.W * (uint32_t)a.C_in * 2u;
    const uint32_t row_bytes = (uint32_t)a.W * (uint32_t)a.C_in * 2u;
    // Fragment reads of step u (temporal tap u/2, k16 slice u%2): the per-lane part of the slot
    // (row / column j, piece 2*slice + hh, permuted) plus a compile-time offset; B adds this
    // wave's first window frame.
    int lbase[2], lbaseB[2];
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
        lbase[sl] = j * 4 + ((2 * sl + hh) ^ ((j >> 2) & 3));
        lbaseB[sl] = lbase[sl] + wave * (kNB * 32 * 4);
    }
    // The tap-8 tile's A operand of temporal tap kd (16 rows x 32 channels): lane l reads row
    // kRow8 + l%16, piece 0, 2, 1, 3 for l/16 = 0..3 (the B operands' k order); it is read with
    // the odd step's fragments.
    const int q8 = ((lane >> 4) & 1) * 2 + (lane >> 5);
    const int lbase8 = (kRow8 + (lane & 15)) * 4 + (q8 ^ head_lds_swizzle(kRow8 + (lane & 15)));
    auto read_frags = [&](const uint4 *abuf, const uint4 *bbuf, int u, vec8 (&fa)[kMB32],
                          vec8 (&fb)[kNB], vec8 &fa8) {
        const int kd = u >> 1, sl = u & 1;
#pragma unroll
        for (int mb = 0; mb < kMB32; ++mb)
            fa[mb] = __builtin_bit_cast(vec8, abuf[lbase[sl] + (kd * 128 + mb * 32) * 4]);
        if (sl == 1) fa8 = __builtin_bit_cast(vec8, abuf[lbase8 + kd * 128 * 4]);
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
            fb[nb] = __builtin_bit_cast(vec8, bbuf[lbaseB[sl] + (kd * kNB + nb) * 128]);
    };

    // B fragments rotate through three sets (set u % 3 for step u), so that at an odd step the
    // even step's fragments are still there for the tap-8 tiles.
    f32x16_t acc[kMB32][kNB];
    f32x4_t t8[kNB][2];
    vec8 af[2][kMB32], bf[3][kNB], a8;
    const f32x16_t zero = {};
    const f32x4_t zero4 = {};

    // FUSED: the bias of the lane's six output channels
    float b6[kHalfCo];
#pragma unroll
    for (int c = 0; c < kHalfCo; ++c) {
        const int co = kHalfCo * hh + c;
        b6[c] = (FUSED && a.bias != nullptr && co < a.C_out) ? E::to_f32(a.bias[co]) : 0.f;
    }

    // The workgroup's row range, one segment per strip it touches (one or two): each segment is
    // a band of output rows [h_begin, h_end) of one strip, run as its own pipeline.
    const int r_end = a.bound[range + 1];
#pragma unroll 1
    for (int rpos = a.bound[range]; rpos < r_end;) {
        const int strip = rpos / a.H;
        const int h_begin = rpos - strip * a.H;
        const int h_end = min(a.H, h_begin + (r_end - rpos));
        rpos += h_end - h_begin;
        const int w0 = FUSED ? strip * a.strip_out - 1 : strip * kWavePos;   // column of position 0
        const int zrow0 = FUSED ? h_begin - 1 : h_begin;
        const int nsteps = (h_end - h_begin) + (FUSED ? 2 : 0);   // Z rows, the same in every wave
        const int nstages = nsteps * nch;

        // B window copies: this wave issues copies k = wave + 4*t; lane i of copy k fills slot
        // 64*k + i = ((frame*4 + nb)*32 + column j)*4 + piece', with frame = k/8, nb = (k/2) % 4,
        // j = 16*(k%2) + i/4 and piece' = piece ^ ((j/4) % 4) -- the piece of lane i is therefore
        // (i%4) ^ ((i/16) % 4) in every copy.  With k = wave + 4*t, copy t fills window frame t/2
        // from column w0 + 4*(i/4) + dw, dw = 64*(wave%2) + wave/2 + 2*(t%2): the wave's twelve
        // copies are six frames at two column offsets, and a lane's part of the source offset is one
        // of two values fixed for the whole kernel (kOff where the column is outside the tensor).
        uint32_t bcol[2];
#pragma unroll
        for (int par = 0; par < 2; ++par) {
            const int col = w0 + 4 * (lane >> 2) + 64 * (wave & 1) + (wave >> 1) + 2 * par;
            bcol[par] = (unsigned)col < (unsigned)a.W ? (uint32_t)((col * a.C_in + 8 * bpiece) * 2) : kOff;
        }
        // Copies of stage (Z row st, channel chunk c) into one buffer pair.  Weight chunks past the
        // packed ones (the even padding) lie past the resource range and copy zeros.  Every offset
        // is formed without branches: an invalid part is all ones, which the saturating add keeps.
        auto copy_stage = [&](int st, int c, uint4 *abuf, uint4 *bbuf) __attribute__((always_inline)) {
            // FUSED: the weight version of the stage's Z row (head_fused_role).  Chunks past the
            // packed ones (the even padding) lie past the resource range and copy zeros.
            const int cbase = FUSED ? (c * 3 + mod3(st)) * kHeadChunkPieces : c * kHeadChunkPieces;
#pragma unroll
            for (int q = 0; q < kCopyA; ++q) {
                // copy k fills LDS rows 16k .. 16k+15; rows 112 .. 127 of each temporal tap (k = 7
                // mod 8) are never read, so their copy takes an offset past the range: no traffic
                const int k = wave * kCopyA + q;
                const int piece = k * 64;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    wr, (lds_void *)&abuf[piece], 16,
                    (k & 7) == 7 ? kOff : (uint32_t)((cbase + piece + lane) * 16), 0, 0, 0);
            }
            // Z row zr reads input row zr + h_org; window frame i is input frame fw0 + i.  The
            // frame / row / chunk part of an offset is uniform (scalar registers); the column part
            // is the lane's; one saturating add joins them.
            const int row = __builtin_amdgcn_readfirstlane(zrow0 + st + a.h_org);
            const bool rok = row >= a.h_lo && row < a.h_hi;
            const uint32_t rbase = (uint32_t)row * row_bytes + (uint32_t)(64 * c);
            const uint32_t cmask = 0u - (uint32_t)(32 * c + 8 * bpiece >= a.C_in);   // ~0: no channels
            const uint32_t colv[2] = {bcol[0] | cmask, bcol[1] | cmask};
#pragma unroll
            for (int t = 0; t < kCopyB; ++t) {
                const int k = wave + 4 * t;
                const int f = fw0 + (t >> 1);
                const bool fok = rok && f >= a.d_lo && f < a.d_hi;
                const uint32_t up = fok ? (uint32_t)(t >> 1) * frame_bytes + rbase : kOff;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void *)&bbuf[k * 64], 16,
                                                         add_sat(colv[t & 1], up), 0, 0, 0);
            }
        };
        if constexpr (FUSED) {
            // the three sets start empty; each is cleared again as its output row is read out
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb) {
#pragma unroll
                for (int mb = 0; mb < kMB32; ++mb) {
                    acc[mb][nb] = zero;
                    touch(acc[mb][nb]);
                }
                t8[nb][0] = t8[nb][1] = zero4;
                touch(t8[nb][0]), touch(t8[nb][1]);
            }
        }

        // ---- prologue: stages 0 and 1 copied, stage 0 complete and published ----
        copy_stage(0, 0, As0, Bs0);
        if (nstages > 1) {
            copy_stage(0, 1, As1, Bs1);   // (nch is even, so stage 1 is chunk 1 of Z row 0)
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(kCopyA + kCopyB));
        } else {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        }
        wg_barrier();
        read_frags(As0, Bs0, 0, af[0], bf[0], a8);

        // Stage g = st*nch + c uses buffer pair g % 2; each pass of the chunk loop runs an even and
        // the following odd stage.
        // One Z row (band-local index st): every channel chunk, two stages per pass.
        auto row_body = [&](auto K, int st) __attribute__((always_inline)) {
            (void)K;
#pragma unroll 1
            for (int c2 = 0; c2 < nch; c2 += 2) {
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    // the stage two ahead: chunk c2 + half + 2 of this Z row, or of the next one
                    const int wrap = c2 + half + 2 >= nch;
                    const int st2 = st + wrap, c_2 = c2 + half + 2 - (wrap ? nch : 0);
                    uint4 *const ca = half == 0 ? As0 : As1;
                    uint4 *const cbb = half == 0 ? Bs0 : Bs1;
                    uint4 *const na = half == 0 ? As1 : As0;
                    uint4 *const nbb = half == 0 ? Bs1 : Bs0;
#pragma unroll
                    for (int u = 0; u < kSteps; ++u) {
                        const int cur = u & 1, bs = u % 3;
                        if (u + 1 < kSteps) {
                            read_frags(ca, cbb, u + 1, af[cur ^ 1], bf[(u + 1) % 3], a8);
                        } else {
                            // Publish the next stage (its copies were issued one stage ago) and
                            // release this one: this wave's last fragments of it are in registers
                            // once its reads are complete.  (Past the last stage the reads below are
                            // of a stale buffer and never used; they keep every path's waits the
                            // same.)
                            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
                            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
                            wg_barrier();
                            read_frags(na, nbb, 0, af[cur ^ 1], bf[0], a8);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                        if (!FUSED && half == 0 && u == 0 && c2 == 0) {
                            // PLANE, first step of a Z row: every accumulator starts from zero
#pragma unroll
                            for (int mb = 0; mb < kMB32; ++mb)
#pragma unroll
                                for (int nb = 0; nb < kNB; ++nb)
                                    acc[mb][nb] = E::mfma32x32x16(af[cur][mb], bf[bs][nb],
                                                                  FUSED ? acc[mb][nb] : zero);
                        } else {
#pragma unroll
                            for (int mb = 0; mb < kMB32; ++mb)
#pragma unroll
                                for (int nb = 0; nb < kNB; ++nb)
                                    acc[mb][nb] = E::mfma32x32x16(af[cur][mb], bf[bs][nb], acc[mb][nb]);
                        }
                        if (u & 1) {
                            // tap 8 of temporal tap u/2: both k16 fragments are in registers
                            const bool first8 = !FUSED && half == 0 && u == 1 && c2 == 0;   // PLANE
#pragma unroll
                            for (int nb = 0; nb < kNB; ++nb) {
                                vec8 lo, hi;
                                tile_operands(bf[(u + 2) % 3][nb], bf[bs][nb], lo, hi);
                                t8[nb][0] = E::mfma16x16x32(a8, lo, first8 ? zero4 : t8[nb][0]);
                                t8[nb][1] = E::mfma16x16x32(a8, hi, first8 ? zero4 : t8[nb][1]);
                            }
                        }
                        if (u + 1 == kSteps) {
                            // The copies of the stage two ahead go into this stage's buffers, one
                            // between each two of this step's MFMAs, so they issue while the matrix
                            // pipe runs.  Past the last stage they still run (in bounds: rows and
                            // chunks that do not exist copy zeros) and nothing reads them.
                            copy_stage(st2, c_2, ca, cbb);
#pragma unroll
                            for (int i = 0; i < kCopyA + kCopyB; ++i) {
                                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one buffer load
                            }
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }

        };

        // ---- row zr of Z is complete in this wave's accumulators ----
        // PLANE: the epilogue walks the accumulator blocks in order and reads each value once, so
        // only one or two blocks are unpacked into registers at a time.
        auto plane_epilogue = [&](int st) __attribute__((always_inline)) {
            const int zr = zrow0 + st;
            const size_t frame = (size_t)n * a.D + od;
            {
                // tap 8, channel c < 6 of lane half h: t8[nb][c / 4][c % 4] after this swap
#pragma unroll
                for (int nb = 0; nb < kNB; ++nb) swap_rows16(t8[nb][0], t8[nb][1]);
                if (zr < h_end && od < a.D) {
#pragma unroll
                    for (int nb = 0; nb < kNB; ++nb) {
                        const int w = w0 + 4 * j + nb;
                        u16 *dst = a.out + (frame * HW + (size_t)zr * a.W + w) * kPlaneCh;
#pragma unroll
                        for (int mb = 0; mb < kMB32; ++mb) touch(acc[mb][nb]);
                        touch(t8[nb][0]), touch(t8[nb][1]);
#pragma unroll
                        for (int tap = 0; tap < 9; ++tap) {
                            u16 r6[kHalfCo];
#pragma unroll
                            for (int c = 0; c < kHalfCo; ++c) {
                                const int t = tap * kHalfCo + c;
                                const float v = tap < 8 ? acc[tap < 8 ? t >> 4 : 0][nb][t & 15]
                                                        : t8[nb][c >> 2][c & 3];
                                r6[c] = E::from_f32(v);
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
                        if (!CO12 && w < a.W) {
                            // channels past the 9*C_out tap channels are zero (the two lane halves
                            // take alternate ones)
                            for (int ch = 9 * a.C_out + hh; ch < kPlaneCh; ch += 2) dst[ch] = 0;
                        }
                    }
                }
            }
        };
        // FUSED, at the end of Z row st (band-local), whose output row st - 1 has set SD: see below.
        auto fused_epilogue = [&](auto SD, int st) __attribute__((always_inline)) {
            constexpr int sd = decltype(SD)::value;
            const int zr = zrow0 + st;
            {
                // Output row zr - 1 is complete in set sd (head_fused_role): each of its
                // 18 slots per position block holds one horizontal tap kx of one output channel,
                // summed over the three vertical taps.  Position p takes tap kx from position
                // p + kx - 1, so a slot of block sb feeds the output of block sb + 1 - kx of the same
                // lane, or across a lane (wavefront shift): block 3 with kx = 0 feeds block 0 of the
                // next lane, block 0 with kx = 2 block 3 of the previous lane.  The lanes that cross a
                // lane half or the wave hold halo columns, which are not stored.  The set is cleared
                // as it is read, for the output row three further on.
                const int ho = zr - 1;   // the output row this Z row completes
                const bool emit = ho >= h_begin && ho < h_end && od < a.D;
                float osum[kNB][kHalfCo];
#pragma unroll
                for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
                    for (int c = 0; c < kHalfCo; ++c) osum[nb][c] = b6[c];
                // a zero the compiler cannot see through, for the tap-8 tiles' register of the set
                const float z = opaque_zero();
                {
#pragma unroll
                    for (int sb = 0; sb < kNB; ++sb) {
                        // register sd of the two tap-8 tiles: one lane swap gives this lane channels
                        // 4 and 5 of its half (horizontal tap 2)
                        float r[2] = {t8[sb][0][sd], t8[sb][1][sd]};
                        lane_swap16(r[0], r[1]);
#pragma unroll
                        for (int q = 0; q < 18; ++q) {
                            const int kx = q / kHalfCo, c = q % kHalfCo;
                            int nb = sb + 1 - kx;
                            float v = q < 16 ? acc[sd][sb][q < 16 ? q : 0] : r[q - 16 > 0 ? 1 : 0];
                            if (nb >= kNB) {   // to the next lane (it takes lane l-1)
                                nb = 0;
                                v = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                    0, __builtin_bit_cast(int, v), 0x138, 0xF, 0xF, false));
                            } else if (nb < 0) {   // to the previous lane (it takes lane l+1)
                                nb = kNB - 1;
                                v = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                    0, __builtin_bit_cast(int, v), 0x130, 0xF, 0xF, false));
                            }
                            osum[nb][c] += v;
                        }
                        // cleared for the output row three further on: the 32x32 block by a matrix
                        // instruction of zeros (an ordinary accumulator result, so it stays in place),
                        // the tiles' register directly
                        vec8 za;   // zeros the compiler cannot see: one instruction per block
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            reinterpret_cast<float *>(&za)[e] = opaque_zero();
                        acc[sd][sb] = E::mfma32x32x16(za, za, zero);
                        t8[sb][0][sd] = z;
                        t8[sb][1][sd] = z;
                    }
                }
#pragma unroll
                for (int nb = 0; nb < kNB; ++nb) {
                    const float *o = osum[nb];
                    const int p = 4 * j + nb;
                    const int w = w0 + p;
                    const bool st_ok = emit && p >= 1 && p <= a.strip_out && w < a.W;
                    u16 r6[kHalfCo];
#pragma unroll
                    for (int c = 0; c < kHalfCo; ++c) r6[c] = E::from_f32(epilogue<EPI>(o[c]));
                    // 32-bit offsets into the group's four output frames, no branches: a store that
                    // must not happen goes to an offset past the buffer range, where it is dropped
                    const uint32_t yoff =
                        (uint32_t)(((wave * a.H + ho) * a.W + w) * a.C_out + kHalfCo * hh) * 2u;
                    if constexpr (RGB) {
                        uint32_t q[kHalfCo];
#pragma unroll
                        for (int c = 0; c < kHalfCo; ++c) q[c] = rgb_code(E::to_f32(r6[c]));
                        // half 0 lacks blue of row 2h (channels 8, 9), half 1 red of row 2h+1
                        // (channels 2, 3): local channels 2 and 3 of the other half, taken from
                        // lane l ^ 32 by one lane swap (a VALU instruction, no LDS round trip)
                        uint32_t sa = q[2] | (q[3] << 8), sb = sa;
                        lane_swap32(sa, sb);
                        const uint32_t recv = hh ? sa : sb;
                        const uint32_t r0 = recv & 0xFFu, r1 = (recv >> 8) & 0xFFu;
                        // bytes R G B R G B of pixels (2h + hh, 2w) and (2h + hh, 2w + 1)
                        const uint32_t p01 = hh == 0 ? (q[0] | (q[4] << 8)) : (r0 | (q[0] << 8));
                        const uint32_t p23 = hh == 0 ? (r0 | (q[1] << 8)) : (q[4] | (r1 << 8));
                        const uint32_t p45 = hh == 0 ? (q[5] | (r1 << 8)) : (q[1] | (q[5] << 8));
                        const uint32_t roff =
                            st_ok ? (uint32_t)(((wave * 2 * a.H + 2 * ho + hh) * 2 * a.W + 2 * w) * 3) : kOff;
                        // the six bytes as one 4-byte and one 2-byte store: 4 + 2 where the run
                        // starts 4-byte aligned, else 2 + 4 (a store that must not happen keeps
                        // an offset past the range)
                        const bool al = (roff & 3u) == 0;
                        __builtin_amdgcn_raw_buffer_store_b32(al ? (p01 | (p23 << 16)) : (p23 | (p45 << 16)), yr,
                                                              al ? roff : __builtin_elementwise_add_sat(roff, 2u), 0, 0);
                        __builtin_amdgcn_raw_buffer_store_b16((u16)(al ? p45 : p01), yr,
                                                              al ? __builtin_elementwise_add_sat(roff, 4u) : roff, 0, 0);
                    } else if constexpr (CO12) {
                        typedef uint32_t v3u __attribute__((ext_vector_type(3)));
                        const v3u v = {(uint32_t)r6[0] | ((uint32_t)r6[1] << 16),
                                       (uint32_t)r6[2] | ((uint32_t)r6[3] << 16),
                                       (uint32_t)r6[4] | ((uint32_t)r6[5] << 16)};
                        __builtin_amdgcn_raw_buffer_store_b96(v, yr, st_ok ? yoff : kOff, 0, 0);
                    } else {
#pragma unroll
                        for (int c = 0; c < kHalfCo; ++c)
                            __builtin_amdgcn_raw_buffer_store_b16(
                                r6[c], yr, st_ok && kHalfCo * hh + c < a.C_out ? yoff + 2u * c : kOff, 0, 0);
                    }
                }
            }
        };

        if constexpr (FUSED) {
            // Sets are numbered from the band's first Z row: Z row st takes weight version st mod 3
            // and completes output row st - 1 (band-local), whose set is (st - 1) mod 3.  Unrolled by
            // three so that the set is a compile-time index.
#pragma unroll 1
            for (int st = 0; st < nsteps; st += 3) {
                row_body(std::integral_constant<int, 0>{}, st);
                fused_epilogue(std::integral_constant<int, 2>{}, st);
                if (st + 1 < nsteps) {
                    row_body(std::integral_constant<int, 1>{}, st + 1);
                    fused_epilogue(std::integral_constant<int, 0>{}, st + 1);
                }
                if (st + 2 < nsteps) {
                    row_body(std::integral_constant<int, 2>{}, st + 2);
                    fused_epilogue(std::integral_constant<int, 1>{}, st + 2);
                }
            }
        } else {
#pragma unroll 1
            for (int st = 0; st < nsteps; ++st) {
                row_body(std::integral_constant<int, 0>{}, st);
                plane_epilogue(st);
            }
        }
        // Before the next segment's first copies: every copy of this one has landed (the last
        // stages issue copies that nothing reads) and every wave is done with its buffers.
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        wg_barrier();
    }
}

}  // namespace

// Row ranges.  One workgroup per CU is resident (the accumulators fill the register file), and
// a workgroup's time is the number of Z rows it computes: its output rows plus, in FUSED mode, two
// halo rows for every strip its range touches.  The strip-major (strip, row) order of a frame
// group is cut into `ranges` contiguous pieces of near-equal cost, the same cut for every
// (sample, frame group), with the range count that minimises rounds of 256 workgroups x the
// largest piece.  A piece may run from the end of one strip into the next, so every CU can take
// one without the bands of a strip having to divide the rows evenly.
HeadRangePlan plan_head_ranges(int N, int D, int H, int W, bool fused) {
    HeadRangePlan rp{};
    rp.strip_out = fused ? kWavePos - 2 : kWavePos;
    rp.strips = (W + rp.strip_out - 1) / rp.strip_out;
    rp.fgroups = (D + 3) / 4;
    const int halo = fused ? 2 : 0;
    const long long groups = (long long)N * rp.fgroups;   // (sample, frame group) pairs
    const long long SH = (long long)rp.strips * H;
    if (groups <= 0 || SH <= 0) return rp;
    // fills one piece from position pos with cost at most K (greedy), returning its cost
    auto fill = [&](long long &pos, long long K) {
        long long cost = 0;
        while (pos < SH) {
            const long long left = H - pos % H, room = K - cost - halo;
            if (room <= 0) break;
            const long long take = room < left ? room : left;
            cost += take + halo;
            pos += take;
            if (take < left) break;
        }
        return cost;
    };
    // pieces needed when no piece costs more than K
    auto pieces_for = [&](long long K) {
        long long count = 0, pos = 0;
        while (pos < SH) fill(pos, K), ++count;
        return count;
    };
    // the smallest largest-piece cost with at most R pieces
    auto cost_for = [&](long long R) {
        long long lo = halo + 1, hi = SH + (long long)rp.strips * halo;
        while (lo < hi) {
            const long long mid = (lo + hi) / 2;
            if (pieces_for(mid) <= R) hi = mid;
            else lo = mid + 1;
        }
        return lo;
    };
    long long best = -1, ranges = 1;
    const long long rmax = SH < kMaxRanges ? SH : kMaxRanges;
    for (long long rounds = 1; rounds <= 4; ++rounds) {
        long long R = 256 * rounds / groups;
        if (R > rmax) R = rmax;
        if (R < 1) R = 1;
        const long long cost = (groups * R + 255) / 256 * cost_for(R);
        if (best < 0 || cost < best) best = cost, ranges = R;
        if (R == rmax) break;
    }
    const long long K = cost_for(ranges);
    long long pos = 0, worst = 0;
    int g = 0;
    rp.bound[0] = 0;
    while (pos < SH && g < kMaxRanges) {
        const long long c = fill(pos, K);
        if (c > worst) worst = c;
        rp.bound[++g] = (int)pos;
    }
    for (int r = g + 1; r <= ranges; ++r) rp.bound[r] = (int)SH;   // empty ranges
    rp.ranges = (int)ranges;
    rp.max_z_rows = (int)worst;
    rp.workgroups = groups * ranges;
    return rp;
}

hipError_t launch_head_gemm(const HeadGemmParams &p, hipStream_t stream) {
    HeadGemmKArgs a{};
    a.x = static_cast<const u16 *>(p.x);
    a.wp = static_cast<const u16 *>(p.wp);
    a.bias = static_cast<const u16 *>(p.bias);
    a.out = static_cast<u16 *>(p.out);
    a.N = p.N, a.C_in = p.C_in, a.C_out = p.C_out, a.D = p.D, a.H = p.H, a.W = p.W;
    a.D_in = p.rg.D_in, a.H_in = p.rg.H_in, a.d_org = p.rg.d_org, a.h_org = p.rg.h_org;
    a.d_lo = p.rg.d_lo, a.d_hi = p.rg.d_hi, a.h_lo = p.rg.h_lo, a.h_hi = p.rg.h_hi;
    const int packed_chunks = (p.C_in + 31) / 32;
    a.nchunks = (packed_chunks + 1) & ~1;   // the kernel runs stages in pairs
    const HeadRangePlan rp = plan_head_ranges(p.N, p.D, p.H, p.W, p.fused);
    a.strip_out = rp.strip_out, a.strips = rp.strips, a.fgroups = rp.fgroups, a.ranges = rp.ranges;
    for (int r = 0; r <= rp.ranges; ++r) a.bound[r] = rp.bound[r];
    a.window_bytes = (uint32_t)((size_t)kInFrames * p.rg.H_in * p.W * p.C_in * 2);
    a.wp_bytes = (uint32_t)((size_t)packed_chunks * (p.fused ? 3 : 1) * kHeadChunkPieces * 16);
    const long long wgs = rp.workgroups;
    a.total_wg = (uint32_t)wgs;
    const dim3 grid((unsigned)wgs), block(256);
#define CX_HG(BFV, FV, EPIV)                                                          \
    do {                                                                              \
        if (p.C_out == 12) head_gemm_kernel<BFV, FV, EPIV, true><<<grid, block, 0, stream>>>(a);  \
        else head_gemm_kernel<BFV, FV, EPIV, false><<<grid, block, 0, stream>>>(a);    \
    } while (0)
    if (p.rgb) {   // fused, C_out == 12
        if (p.bf16) {
            if (p.epilogue == EPI_RELU) head_gemm_kernel<true, true, EPI_RELU, true, true><<<grid, block, 0, stream>>>(a);
            else if (p.epilogue == EPI_CLAMP1) head_gemm_kernel<true, true, EPI_CLAMP1, true, true><<<grid, block, 0, stream>>>(a);
            else head_gemm_kernel<true, true, EPI_NONE, true, true><<<grid, block, 0, stream>>>(a);
        } else {
            if (p.epilogue == EPI_RELU) head_gemm_kernel<false, true, EPI_RELU, true, true><<<grid, block, 0, stream>>>(a);
            else if (p.epilogue == EPI_CLAMP1) head_gemm_kernel<false, true, EPI_CLAMP1, true, true><<<grid, block, 0, stream>>>(a);
            else head_gemm_kernel<false, true, EPI_NONE, true, true><<<grid, block, 0, stream>>>(a);
        }
    } else if (!p.fused) {
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
