// MFMA implicit-GEMM 3x3x3 (and 3x1x1) convolution for channels-last bf16/fp16 video tensors on
// gfx950.
//
// GEMM view: D[m, p] = sum_k Wt[m, k] * X[k, p] with m = output row (output channel, or for the
// split head one of the 9*12 tap-channels of its intermediate plane), p = output position, and
// k = (tap, input channel).  The weights are the A operand (rows = m), so one lane of the
// 16x16 accumulator holds four consecutive output channels of one position: an 8-byte store into
// the channels-last output.  (FastVideo head.cu, header comment: the 27-tap form of the output
// convolution and its split into a temporal conv whose output channels are the spatial taps.)
//
// Per workgroup (256 threads, 4 waves): a TH x TW block of output positions of one frame times
// BM output rows.  The K loop runs over (input-channel chunk of 32, live temporal tap) stages;
// each stage stages one input frame's window -- (TH+2) x (TW+2) positions x 32 channels, zero
// outside the tensor -- in LDS with coalesced 16-byte loads, and its nine spatial taps read their
// B fragments from it by address offset (the reuse the per-position form lacks).  A fragments
// (weights) come from global memory, where they are L2-resident, in an order packed so that one
// 16-row fragment is 1 KiB contiguous.  Stages whose frame lies in the temporal padding are
// skipped (they only ever multiply zeros).  Small problems split K over channel chunks and
// reduce fp32 partials in a second kernel.
//
// Matrix-core operand layout used (v_mfma_f32_16x16x32_{bf16,f16}): lane l supplies row l%16 of A
// and column l%16 of B, each with the 8 consecutive k values 8*(l/16)..8*(l/16)+7; it receives
// rows 4*(l/16)..4*(l/16)+3 of column l%16 of D.  Only the row/column assignment matters for
// correctness -- A and B share the same k assignment, so any permutation of k inside a 32-chunk
// cancels in the dot product.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace cx {

namespace {


struct IgemmKArgs {
    const u16 *x;
    const u16 *wp;
    const u16 *bias;
    u16 *y;
    float *partial;
    int N, C_in, D, H, W;          // D, H, W: output extent
    int W_in;                      // input width (W at stride 1)
    int D_in, H_in, d_org, h_org;  // input region (see ConvRegion)
    int d_lo, d_hi, h_lo, h_hi;
    int Mrows, Mpad, Cy;
    int nchunks, chunks_per_split, splits;
    int tiles_h, tiles_w, mtiles;
    uint32_t total_wg;
    uint32_t wp_bytes;   // packed weights (buffer-resource range of the 32x32 kernel)
    // stream-K (igemm32 with SK): partial slots in `partial`, one arrival counter per tile
    unsigned *sk_count;
    int sk_groups;       // workgroups (a multiple of 8)
    uint32_t sk_total;   // stages in the stream-K order
    int sk_unit_stages;  // stages of one (output-row tile, sample, spatial tile) over all frames
};

// Stores four rows m0..m0+3 of one accumulator column (bias already added): fp32 partials for
// split-K, else epilogue + one rounding to the storage type.
template <bool BF, int EPI, bool SPLITK>
__device__ __forceinline__ void store_rows(const IgemmKArgs &a, f32x4_t v, size_t pos, int split,
                                          size_t P, int m0) {
    using E = Elem<BF>;
    if (m0 >= a.Mrows) return;
    if constexpr (SPLITK) {
        float *dst = a.partial + ((size_t)split * P + pos) * a.Cy + m0;
        if (m0 + 3 < a.Mrows && (a.Cy & 3) == 0) {
            *reinterpret_cast<f32x4_t *>(dst) = v;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (m0 + i < a.Mrows) dst[i] = v[i];
        }
    } else {
        u16 o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = E::from_f32(epilogue<EPI>(v[i]));
        u16 *dst = a.y + pos * a.Cy + m0;
        if (m0 + 3 < a.Mrows && (a.Cy & 3) == 0) {
            uint2 pk;
            pk.x = (uint32_t)o[0] | ((uint32_t)o[1] << 16);
            pk.y = (uint32_t)o[2] | ((uint32_t)o[3] << 16);
            *reinterpret_cast<uint2 *>(dst) = pk;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (m0 + i < a.Mrows) dst[i] = o[i];
        }
    }
}

// The 27-tap convolution.  K is walked in stages s = (input-channel chunk cc, live temporal tap
// kd): each stage stages ONE input frame's window -- (TH+2) x (TW+2) positions x 32 channels --
// in LDS and runs its nine spatial taps from it.  The window is double-buffered: the next
// stage's 16-byte global loads are issued into registers before the current stage's MFMAs and
// written to the other LDS buffer after them, so one barrier per stage suffices.  Weight
// fragments stream from global memory (L2-resident) through a 3-tap-deep register ring.
template <bool BF, int MB, int NBW, int WM, int WN, int TH, int TW, int EPI, bool SPLITK>
__global__ __launch_bounds__(256, 2) void igemm3d_kernel(IgemmKArgs a) {
    using E = Elem<BF>;
    typedef typename E::vec8 vec8;
    constexpr int BM = WM * MB * 16;
    constexpr int NBLK_ROW = TW / 16;
    static_assert(TW % 16 == 0, "tile width must be a multiple of 16");
    static_assert(TH * NBLK_ROW == WN * NBW, "each wave owns NBW of the tile's 16-position blocks");
    static_assert(WM * WN == 4, "four waves per workgroup");
    constexpr int WH = TH + 2, WW = TW + 2;
    constexpr int FPOS = WH * WW;          // window positions of one frame
    constexpr int PIECES = FPOS * 4;       // 16-byte pieces of one staged window
    constexpr int PPT = (PIECES + 255) / 256;
    constexpr int PD = 3;                  // weight-fragment prefetch distance (taps)
    // A window position is 64 bytes (32 channels) in four 16-byte pieces, stored XOR-permuted by
    // (column / 4) % 4, and window rows are RowPos positions apart (a multiple of 4): any 16
    // consecutive columns of a row -- what one fragment read takes -- fall on distinct bank
    // groups.
    constexpr int RowPos = (WW + 3) / 4 * 4;
    __shared__ __attribute__((aligned(16))) uint4 win[2][WH * RowPos * 4];
    __shared__ float bias_s[BM];   // this workgroup's output rows (0 past C_out / no bias)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM, wn = wave / WM;

    // Each XCD takes a contiguous run of workgroups (xcd_remap), frame innermost: the frames of
    // one tile run together on one XCD, so each input frame window, read by three output frames,
    // comes from HBM about once and from that XCD's L2 after.
    uint32_t lin = xcd_remap(blockIdx.x, a.total_wg);
    const int mt = lin % a.mtiles;
    lin /= a.mtiles;
    const int od = lin % a.D;
    lin /= a.D;
    const int tw = lin % a.tiles_w;
    lin /= a.tiles_w;
    const int th = lin % a.tiles_h;
    lin /= a.tiles_h;
    const int n = lin % a.N;
    const int split = lin / a.N;

    const int oh0 = th * TH, ow0 = tw * TW;
    const int c_begin = split * a.chunks_per_split;
    const int c_end = min(a.nchunks, c_begin + a.chunks_per_split);
    // live temporal taps: input frame fi0 + kd inside [d_lo, d_hi)
    const int fi0 = od + a.d_org - 1;
    const int kd_lo = max(0, a.d_lo - fi0);
    const int kd_hi = min(2, a.d_hi - 1 - fi0);
    const int nkd = max(0, kd_hi - kd_lo + 1);
    const int nst = (c_end - c_begin) * nkd;

    f32x4_t acc[MB][NBW];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NBW; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int mrow_lane = mt * BM + wm * MB * 16 + (lane & 15);
    const int kofs = (lane >> 4) * 8;
    const size_t frame_elems = (size_t)a.H_in * a.W * a.C_in;

    uint4 stg[PPT];
    auto fetch = [&](int s) {
        const int cc = c_begin + s / nkd, kd = kd_lo + s % nkd;
        const u16 *base = a.x + ((size_t)n * a.D_in + (fi0 + kd)) * frame_elems + cc * 32;
#pragma unroll
        for (int j = 0; j < PPT; ++j) {
            const int i = tid + j * 256;
            uint4 v = {0u, 0u, 0u, 0u};
            if (PIECES % 256 == 0 || i < PIECES) {
                const int q = i & 3, pos = i >> 2;
                const int wh = pos / WW, ww = pos - wh * WW;
                const int h = oh0 - 1 + wh + a.h_org, w = ow0 - 1 + ww;
                if (h >= a.h_lo && h < a.h_hi && (unsigned)w < (unsigned)a.W &&
                    cc * 32 + q * 8 < a.C_in)
                    v = *reinterpret_cast<const uint4 *>(base + ((size_t)h * a.W + w) * a.C_in + q * 8);
            }
            stg[j] = v;
        }
    };
    // the LDS slot of this thread's pieces (the same in every stage)
    int cslot[PPT];
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        const int i = tid + j * 256, q = i & 3, pos = i >> 2;
        const int wh = pos / WW, ww = pos - wh * WW;
        cslot[j] = (wh * RowPos + ww) * 4 + (q ^ ((ww >> 2) & 3));
    }
    auto commit = [&](int buf) {
#pragma unroll
        for (int j = 0; j < PPT; ++j) {
            const int i = tid + j * 256;
            if (PIECES % 256 == 0 || i < PIECES) win[buf][cslot[j]] = stg[j];
        }
    };
    auto load_a = [&](int s, int j, vec8 *dst) {
        const int cc = c_begin + s / nkd, kd = kd_lo + s % nkd;
        const u16 *wb = a.wp + ((size_t)(cc * 27 + kd * 9 + j) * a.Mpad + mrow_lane) * 32 + kofs;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) dst[mb] = *reinterpret_cast<const vec8 *>(wb + mb * 16 * 32);
    };

    for (int i = tid; i < BM; i += 256) {
        const int m = mt * BM + i;
        bias_s[i] = (!SPLITK && a.bias != nullptr && m < a.Mrows) ? E::to_f32(a.bias[m]) : 0.f;
    }
    vec8 aq[PD][MB];
    if (nst > 0) {
        fetch(0);
        commit(0);
#pragma unroll
        for (int p = 0; p < PD; ++p) load_a(0, p, aq[p]);
    }
    __syncthreads();

    // B fragment slot of lane column (lane & 15) + kx, piece lane / 16, in window row 0 and block
    // column 0; block columns are multiples of 16, which keep the swizzle
    int bslot[3];
#pragma unroll
    for (int kx = 0; kx < 3; ++kx) {
        const int col = (lane & 15) + kx;
        bslot[kx] = col * 4 + ((lane >> 4) ^ ((col >> 2) & 3));
    }
    for (int s = 0; s < nst; ++s) {
        const int buf = s & 1;
        const bool more = s + 1 < nst;
        if (more) fetch(s + 1);
        const uint4 *wsrc = win[buf];
#pragma unroll
        for (int j = 0; j < 9; ++j) {
            const int ky = j / 3, kx = j % 3;
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const int blk = wn * NBW + nb;
                const int r = blk / NBLK_ROW, c0 = (blk % NBLK_ROW) * 16;
                const vec8 B = __builtin_bit_cast(vec8, wsrc[bslot[kx] + ((r + ky) * RowPos + c0) * 4]);
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[mb][nb] = E::mfma16x16x32(aq[j % PD][mb], B, acc[mb][nb]);
            }
            // refill this slot with the tap PD ahead (possibly in the next stage)
            if (j + PD < 9)
                load_a(s, j + PD, aq[j % PD]);
            else if (more)
                load_a(s + 1, j + PD - 9, aq[j % PD]);
        }
        if (more) commit(buf ^ 1);
        __syncthreads();
    }

    const size_t P = (size_t)a.N * a.D * a.H * a.W;
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
        const int blk = wn * NBW + nb;
        const int r = blk / NBLK_ROW, c0 = (blk % NBLK_ROW) * 16;
        const int oh = oh0 + r, ow = ow0 + c0 + (lane & 15);
        if (oh >= a.H || ow >= a.W) continue;
        const size_t pos = (((size_t)n * a.D + od) * a.H + oh) * a.W + ow;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int r0 = wm * MB * 16 + mb * 16 + 4 * (lane >> 4);
            const float4 bv = *reinterpret_cast<const float4 *>(&bias_s[r0]);
            const f32x4_t v = acc[mb][nb];
            store_rows<BF, EPI, SPLITK>(a, f32x4_t{v[0] + bv.x, v[1] + bv.y, v[2] + bv.z, v[3] + bv.w},
                                       pos, split, P, mt * BM + r0);
        }
    }
}

// ---------------------------------------------------------------------------------------------
// The 27-tap convolution for narrow outputs (C_out <= 16: the direct head) on 16x16x32 MFMA.
// What limits this form is the vector memory path's line requests (each costs about an L2
// latency divided by the requests a CU keeps in flight), so the kernel is built to request few
// lines per output:
//   * Channels run in stages of 64 (a pair of 32-channel chunks): a window position is then one
//     whole 128-byte line, and one LDS-DMA copy (buffer_load ... lds, 16 bytes per lane, 1 KiB of
//     LDS) moves 8 whole lines.  Window: (TH+2) x (TW+2) = 10 x 34 positions.
//   * A workgroup takes NF (4 or 8) consecutive output frames of an 8 x 32 tile and walks the
//     NF + 2 input frames they read: each input window is copied once and applied to every output
//     frame that reads it (temporal taps kd = 0, 1, 2 of frames i, i-1, i-2), instead of once per
//     output frame and tap.
//   * The weights of a pair (2 chunks x 27 taps x 16 rows x 32 channels) sit in three LDS slots,
//     one per temporal tap (18 KiB each), copied once per workgroup and pair by the same DMA.
//     Slot kd is last read at input frame NF-1+kd of a pair, so the next pair's taps 0 and 1
//     are copied during its last two input frames and tap 2 during the next pair's first one --
//     no stall between pairs.
//   * Windows are double-buffered (separate objects; input frames 0..NF+1 of a pair are fully
//     unrolled, so every buffer and slot is known at compile time): the copies of the next
//     window go out one by one between the MFMAs of the first steps of the current one and are
//     waited for at its end, one barrier per input frame.  ~140 KiB of LDS: one workgroup
//     (4 waves) per CU.
//   * Wave w owns 4 output rows x 16 columns of the tile (rows 4*(w/2).., columns 16*(w%2)..) in
//     each of the NF frames: a window fragment of row wr and column shift kx feeds the
//     vertical taps ky of up to three of its rows in up to three output frames.
// LDS layouts (16-byte pieces): window position (row, col) at (row * 34 + col) * 8, its piece p
// (channels 8p..8p+7 of the pair) in slot p ^ ((col >> 1) & 7) -- any 16 consecutive columns of
// one piece fall on distinct bank groups; weight fragment (chunk half h, spatial tap t) of a
// temporal-tap slot at (9h + t) * 64, row m's piece p in slot 4m + (p ^ ((m >> 2) & 3)).  The DMA
// fetches, for each LDS slot, the global piece that belongs there: the permutations stay inside
// one line, so copies remain whole lines.  Zero padding (rows, columns, frames, channels, the
// second chunk past the range) is an offset past the buffer range: the copy fetches nothing and
// writes zeros.
// Addressing: a window is one 32-bit buffer range from its first valid input row (at most ten
// rows of one frame), so frames of any size work.
// output frames per workgroup: 8 where that leaves few frame slots empty, else 4
__host__ __device__ constexpr int narrow_frames(int D) { return D >= 8 && (D % 8 == 0 || D % 8 > 4) ? 8 : 4; }
constexpr int kNarTH = 8, kNarTW = 32;                   // output tile
constexpr int kNarRowPos = kNarTW + 2;                   // window row length (even)
constexpr int kNarPos = (kNarTH + 2) * kNarRowPos;       // 340 window positions
constexpr int kNarWinCopies = (kNarPos + 7) / 8;         // 43 DMA copies of 8 positions
constexpr int kNarWinSlots = kNarWinCopies * 64;
constexpr int kNarACopies = 18;                          // 2 chunks x 9 spatial taps, 1 KiB each
constexpr int kNarWinPerWave = (kNarWinCopies + 3) / 4;  // 11
constexpr int kNarAPerWave = (kNarACopies + 3) / 4;      // 5
constexpr int kNarWaitVm0 = (7 << 4) | (15 << 8);        // s_waitcnt vmcnt(0), nothing else

// The uniform parts of one window copy and of one temporal tap's weight copies of
// igemm3d_narrow_kernel (at namespace scope: the host pass emits no launch stub for a kernel
// template with local struct types).
struct WinCopy {
    const u16 *xbase;  // the window's rows (its first valid one)
    int pmax;          // pieces holding input channels of the range's chunks (0: none)
    uint32_t cdelta;   // byte offset of the pair's first channel in a position
};
struct WCopy {
    uint32_t abase;    // byte offset of fragment (chunk cc0, tap kd*9) in the packing
    bool second;       // the pair's second chunk lies in the range
    bool live;         // there is such a copy
};

template <bool BF, int EPI, bool SPLITK, int NF>
__global__ __launch_bounds__(256, 1) void igemm3d_narrow_kernel(IgemmKArgs a) {
    using E = Elem<BF>;
    typedef typename E::vec8 vec8;
    typedef __attribute__((address_space(3))) void lds_void;
    static_assert(NF == 4 || NF == 8, "four or eight output frames per workgroup");
    constexpr int kStages = NF + 2;   // input frames per pair
    __shared__ __attribute__((aligned(16))) uint4 Win0[kNarWinSlots];
    __shared__ __attribute__((aligned(16))) uint4 Win1[kNarWinSlots];
    __shared__ __attribute__((aligned(16))) uint4 Wk0[kNarACopies * 64];
    __shared__ __attribute__((aligned(16))) uint4 Wk1[kNarACopies * 64];
    __shared__ __attribute__((aligned(16))) uint4 Wk2[kNarACopies * 64];
    __shared__ __attribute__((aligned(16))) float bias_s[16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // frame group innermost: consecutive groups of a tile share two input frames in L2
    uint32_t lin = xcd_remap(blockIdx.x, a.total_wg);
    const int fgroups = (a.D + NF - 1) / NF;
    const int fg = lin % fgroups;
    lin /= fgroups;
    const int tw = lin % a.tiles_w;
    lin /= a.tiles_w;
    const int th = lin % a.tiles_h;
    lin /= a.tiles_h;
    const int n = lin % a.N;
    const int split = lin / a.N;

    const int oh0 = th * kNarTH, ow0 = tw * kNarTW;
    const int od0 = fg * NF;
    const int c_begin = split * a.chunks_per_split;
    const int c_end = min(a.nchunks, c_begin + a.chunks_per_split);
    const int npairs = (c_end - c_begin + 1) / 2;
    const int fw0 = od0 - 1 + a.d_org;   // input frame of window i = fw0 + i

    // the window's input rows: oh0 - 1 + h_org + row, valid inside [h_lo, h_hi); the buffer range
    // starts at the first valid one
    const int wrow0 = oh0 - 1 + a.h_org;
    const int hbase = max(a.h_lo, wrow0);
    const int hlast = min(a.h_hi, wrow0 + kNarTH + 2);   // exclusive
    const uint32_t row_bytes = (uint32_t)a.W * (uint32_t)a.C_in * 2u;
    const uint32_t win_range = hlast > hbase ? (uint32_t)(hlast - hbase) * row_bytes : 0u;
    const size_t frame_elems = (size_t)a.H_in * a.W * a.C_in;

    // per-lane parts of this wave's window copies: copy k = wave + 4t, lane i -> position
    // 8k + i/8, LDS slot piece i%8 <- global piece (i%8) ^ ((col >> 1) & 7)
    uint32_t woff[kNarWinPerWave];
    int wpiece[kNarWinPerWave];
#pragma unroll
    for (int t = 0; t < kNarWinPerWave; ++t) {
        const int k = wave + 4 * t;
        const int P = 8 * k + (lane >> 3);
        const int row = P / kNarRowPos, col = P - row * kNarRowPos;
        const int p = (lane & 7) ^ ((col >> 1) & 7);
        const int h = wrow0 + row, w = ow0 - 1 + col;
        const bool ok = k < kNarWinCopies && P < kNarPos && h >= hbase && h < hlast &&
                        (unsigned)w < (unsigned)a.W;
        woff[t] = ok ? (uint32_t)(h - hbase) * row_bytes + ((uint32_t)w * a.C_in + 8u * p) * 2u : 0xFFFFFFFFu;
        wpiece[t] = p;
    }
    // per-lane part of the weight copies: row lane/4, slot lane%4 <- piece (lane%4) ^ ((row>>2)&3)
    const uint32_t alane = (uint32_t)((lane >> 2) * 64 + (((lane & 3) ^ ((lane >> 4) & 3)) * 16));
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)a.wp, (short)0, (int)(a.wp_bytes), 0x00020000);

    // The copies one input frame's stage issues, at most kNarWinPerWave + kNarAPerWave per wave:
    // the next window (pair jw, input frame iw) and, for some stages, one temporal tap's weights
    // (pair ja, tap kda).  window() / weights() fix their uniform parts, copy_one issues copy i.
    auto window = [&](int jw, int iw) {
        WinCopy c;
        const int cc0 = c_begin + 2 * jw;
        const int f = fw0 + iw;
        const bool fok = jw < npairs && f >= a.d_lo && f < a.d_hi;
        c.pmax = fok ? min(cc0 + 1 < c_end ? 8 : 4, (a.C_in - 32 * cc0 + 7) / 8) : 0;
        c.xbase = a.x + (((size_t)n * a.D_in + (fok ? f : 0)) * frame_elems + ((size_t)hbase * a.W) * a.C_in);
        c.cdelta = (uint32_t)cc0 * 64u;   // 32 channels x 2 bytes per chunk
        return c;
    };
    auto weights = [&](int ja, int kda) {
        WCopy c;
        const int cc0 = c_begin + 2 * ja;
        c.live = ja < npairs;
        c.second = cc0 + 1 < c_end;
        c.abase = (uint32_t)((cc0 * 27 + kda * 9) * a.Mpad) * 64u;
        return c;
    };
    auto copy_one = [&](int i, const WinCopy &cw, uint4 *win, const WCopy &ca, uint4 *wk) {
        if (i < kNarWinPerWave) {
            const int k = wave + 4 * i;
            if (kNarWinCopies % 4 != 0 && k >= kNarWinCopies) return;   // wave-uniform
            const uint32_t off = wpiece[i] < cw.pmax && woff[i] != 0xFFFFFFFFu ? woff[i] + cw.cdelta : 0xFFFFFFFFu;
            const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
                (void *)cw.xbase, (short)0, (int)win_range, 0x00020000);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void *)&win[k * 64], 16, off, 0, 0, 0);
        } else if (ca.live) {
            const int q = wave + 4 * (i - kNarWinPerWave);
            if (q >= kNarACopies) return;   // wave-uniform
            const int hq = q / 9, tq = q - 9 * hq;
            const uint32_t frag = ca.abase + (uint32_t)((hq * 27 + tq) * a.Mpad) * 64u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_void *)&wk[q * 64], 16,
                                                     hq == 0 || ca.second ? frag + alane : 0xFFFFFFFFu, 0, 0, 0);
        }
    };

    // fragment reads: weight (h, spatial tap) of row lane%16, piece lane/16; window (row, column
    // shift kx, chunk half h) of column c0 + kx + lane%16, piece 4h + lane/16
    const int cb = wave & 1, r0 = 4 * (wave >> 1);
    const int aslot = (lane & 15) * 4 + ((lane >> 4) ^ ((lane >> 2) & 3));
    int bslot[2][3];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int kx = 0; kx < 3; ++kx) {
            const int col = 16 * cb + kx + (lane & 15);
            const int p = 4 * h + (lane >> 4);
            bslot[h][kx] = (r0 * kNarRowPos + col) * 8 + (p ^ ((col >> 1) & 7));
        }

    f32x4_t acc[NF][4];
#pragma unroll
    for (int o = 0; o < NF; ++o)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[o][r] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Input frame I of a pair from window win: output frame o = I - kd takes temporal tap kd for
    // each kd with 0 <= o < NF.  36 steps (chunk half h, window row wrr, column shift kx), each
    // one window fragment -- read two steps ahead -- and the MFMAs it feeds; the weight fragments
    // of the live taps at the start of each half.  The stage's copies (ncopy of them) go out one
    // after each of the first steps.
    auto stage = [&](auto Ic, const uint4 *win, int ncopy, const WinCopy &cw, uint4 *nwin,
                     const WCopy &ca, uint4 *wk) {
        constexpr int I = decltype(Ic)::value;
        constexpr bool live0 = I < NF, live1 = I >= 1 && I - 1 < NF, live2 = I >= 2;
        const uint4 *wks[3] = {Wk0, Wk1, Wk2};
        constexpr int kSteps = 36;
        auto read_b = [&](int it) {
            const int h = it / 18, wrr = (it % 18) / 3, kx = it % 3;
            return __builtin_bit_cast(vec8, win[bslot[h][kx] + wrr * (kNarRowPos * 8)]);
        };
        vec8 A[3][9];
        vec8 Bq[3];
        Bq[0] = read_b(0);
        Bq[1] = read_b(1);
#pragma unroll
        for (int it = 0; it < kSteps; ++it) {
            const int h = it / 18, wrr = (it % 18) / 3, kx = it % 3;
            if (it % 18 == 0) {
#pragma unroll
                for (int kd = 0; kd < 3; ++kd) {
                    if (!(kd == 0 ? live0 : kd == 1 ? live1 : live2)) continue;
#pragma unroll
                    for (int t = 0; t < 9; ++t)
                        A[kd][t] = __builtin_bit_cast(vec8, wks[kd][(9 * h + t) * 64 + aslot]);
                }
            }
            if (it + 2 < kSteps) Bq[(it + 2) % 3] = read_b(it + 2);
#pragma unroll
            for (int kd = 0; kd < 3; ++kd) {
                if (!(kd == 0 ? live0 : kd == 1 ? live1 : live2)) continue;
                const int o = I - kd;
#pragma unroll
                for (int ky = 0; ky < 3; ++ky) {
                    const int r = wrr - ky;
                    if (r >= 0 && r < 4) acc[o][r] = E::mfma16x16x32(A[kd][ky * 3 + kx], Bq[it % 3], acc[o][r]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            if (it < ncopy) copy_one(it, cw, nwin, ca, wk);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    if (tid < 16) bias_s[tid] = (!SPLITK && a.bias != nullptr && tid < a.Mrows) ? E::to_f32(a.bias[tid]) : 0.f;
    constexpr int kAll = kNarWinPerWave + kNarAPerWave;
    if (npairs > 0) {
        // pair 0's first window and its temporal taps 0 and 1 (tap 2 follows with input frame 0)
        const WinCopy w0 = window(0, 0);
        const WCopy none{0u, false, false};
        const WCopy t0 = weights(0, 0), t1 = weights(0, 1);
#pragma unroll
        for (int i = 0; i < kNarWinPerWave; ++i) copy_one(i, w0, Win0, none, Wk0);
#pragma unroll
        for (int i = kNarWinPerWave; i < kAll; ++i) copy_one(i, w0, Win0, t0, Wk0);
#pragma unroll
        for (int i = kNarWinPerWave; i < kAll; ++i) copy_one(i, w0, Win0, t1, Wk1);
    }
    __builtin_amdgcn_s_waitcnt(kNarWaitVm0);
    __syncthreads();
    // the stage of input frame I of pair j: its window is in Win{I % 2}; it copies the next
    // window (frame I+1, or frame 0 of pair j+1) into the other buffer, and weights: tap 2 of pair
    // j with frame 0, taps 0 and 1 of pair j+1 with frames NF and NF+1.
    auto run = [&](auto Ic, int j) {
        constexpr int I = decltype(Ic)::value;
        const bool last = I + 1 == kStages;
        const WinCopy cw = window(last ? j + 1 : j, last ? 0 : I + 1);
        const int kda = I == 0 ? 2 : (I == NF ? 0 : (I == NF + 1 ? 1 : -1));
        const WCopy ca = kda < 0 ? WCopy{0u, false, false} : weights(kda == 2 ? j : j + 1, kda);
        uint4 *wk = kda == 0 ? Wk0 : (kda == 1 ? Wk1 : Wk2);
        const int ncopy = kda < 0 ? kNarWinPerWave : kAll;
        if constexpr (I % 2 == 0) stage(Ic, Win0, ncopy, cw, Win1, ca, wk);
        else stage(Ic, Win1, ncopy, cw, Win0, ca, wk);
        __builtin_amdgcn_s_waitcnt(kNarWaitVm0);
        __syncthreads();
    };
    using std::integral_constant;
#pragma unroll 1
    for (int j = 0; j < npairs; ++j) {
        run(integral_constant<int, 0>{}, j);
        run(integral_constant<int, 1>{}, j);
        run(integral_constant<int, 2>{}, j);
        run(integral_constant<int, 3>{}, j);
        run(integral_constant<int, 4>{}, j);
        run(integral_constant<int, 5>{}, j);
        if constexpr (kStages > 6) {
            run(integral_constant<int, 6>{}, j);
            run(integral_constant<int, 7>{}, j);
            run(integral_constant<int, 8>{}, j);
            run(integral_constant<int, 9>{}, j);
        }
    }
    static_assert(kStages == 6 || kStages == 10, "the pair loop above runs input frames 0..kStages-1");

    const size_t P = (size_t)a.N * a.D * a.H * a.W;
    const int m0 = 4 * (lane >> 4);
    const float4 bv = *reinterpret_cast<const float4 *>(&bias_s[m0]);
#pragma unroll
    for (int o = 0; o < NF; ++o) {
        const int od = od0 + o;
        if (od >= a.D) break;   // (uniform)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int oh = oh0 + r0 + r, ow = ow0 + 16 * cb + (lane & 15);
            if (oh >= a.H || ow >= a.W) continue;
            const size_t pos = (((size_t)n * a.D + od) * a.H + oh) * a.W + ow;
            store_rows<BF, EPI, SPLITK>(a, f32x4_t{acc[o][r][0] + bv.x, acc[o][r][1] + bv.y,
                                                  acc[o][r][2] + bv.z, acc[o][r][3] + bv.w},
                                       pos, split, P, m0);
        }
    }
}

// ---------------------------------------------------------------------------------------------
// The 27-tap convolution for wide outputs (C_out > 16) on v_mfma_f32_32x32x16: one wave per SIMD
// keeps that pipe full.  Each wave owns a 64 x 256 tile (2 x 8 blocks, all 256 accumulators): per
// k16 slice it takes two weight fragments from L2 and eight input fragments from LDS, so the four
// waves of a workgroup fetch disjoint weight rows and every weight byte leaves L2 once per
// workgroup.  Operand layout: lane l supplies row (A) / column (B) l%32 with the 8 k values of
// half l/32 of a 16-wide k slice, and receives accumulator element i at row 8*(i/4) + 4*(l/32) +
// i%4, column l%32.
//
// Workgroup: 256 output rows (four waves along M) x an 8 x 32 block of positions of one frame.
// K runs in stages (32-channel chunk, live temporal tap); a stage's input window -- 10 x 34
// positions x 32 channels, zero outside the tensor -- is copied global -> LDS by the buffer unit
// (LDS DMA, 16 positions x 64 bytes per copy, no registers) into one of three buffers, two
// stages ahead, and its nine spatial taps read their B fragments from it by address offset.  Window rows are 36
// positions apart (34 used) and each 64-byte position holds its four 16-byte pieces XOR-permuted
// by (column/4) % 4: any 16 consecutive columns of a row then fall on distinct LDS bank groups,
// and a fragment address is a per-lane part (column, piece) plus a row part that fits the
// instruction's offset field.  Weight fragments (1 KiB contiguous each in the packing) stream
// from L2 into a register ring half a stage deep.  The compiler cannot see that a DMA copy into
// one window buffer never overlaps reads from another, so the three buffers are separate objects
// and the stage loop is unrolled by three.
// ---------------------------------------------------------------------------------------------
// Tile geometry by LW, the columns one 32-lane block spans, and NB, the 32-position blocks of a
// tile: LW = 32 gives NB x 32 positions per workgroup (one row per block), LW = 16 gives
// 2NB x 16 (two rows per block) for narrow frames.  NB = 8 (256 positions, all 256 accumulators
// of a wave) is the default; NB = 4 halves the tile for convolutions with few positions, which
// then fill the chip without splitting K.
template <int LW, int NB_, int S = 1>
struct W32Geom {
    static constexpr int R = 32 / LW;                    // rows per 32-position block
    static constexpr int NB = NB_;                       // 32-position blocks per tile
    static constexpr int TH = NB * R, TW = LW;           // workgroup tile = every wave's tile
    // Window: stride 1 reads TH+2 input rows x TW+2 columns; stride 2 (spatial) reads 2TH+1 rows
    // x 2TW+1 columns and stores a row's even window columns (taps kx = 0, 2) at LDS columns
    // 0..TW and its odd ones (kx = 1) from column OddBase, so every tap reads unit-stride.
    static constexpr int WH = S == 1 ? TH + 2 : 2 * TH + 1;            // window rows
    static constexpr int WW = S == 1 ? TW + 2 : TW + 1;                // (even) columns used
    static constexpr int OddBase = S == 1 ? 0 : (TW + 1 + 3) / 4 * 4;  // first odd column slot
    static constexpr int RowPos = S == 1 ? (WW + 3) / 4 * 4 : OddBase + (TW + 3) / 4 * 4;
    static constexpr int Pos = WH * RowPos;              // window positions
    static constexpr int Copies = (Pos * 4 + 63) / 64;   // DMA copies of 16 positions
    static constexpr int CopiesPerWave = (Copies + 3) / 4;
    static constexpr int Slots = Copies * 64;            // 16-byte pieces per window buffer
};
constexpr int kW32Slices = 18;                          // k16 slices per stage: 9 taps x 2 halves
constexpr int kW32PD = 9;                               // weight prefetch distance in slices

// slot of (window row r, column c, piece); with RowPos a multiple of 4 the row part is a
// multiple of 16 slots
template <int RowPos>
__device__ __forceinline__ int w32_slot(int r, int c, int piece) {
    return (r * RowPos + c) * 4 + (piece ^ ((c >> 2) & 3));
}
__device__ __forceinline__ void w32_barrier() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ void w32_touch(f32x16_t &v) { asm volatile("" : "+a"(v)::"memory"); }
__device__ constexpr int w32_waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kW32WaitLgkm0 = 15 | (3 << 14) | (7 << 4);
// cache-policy operand of the buffer intrinsics: sc1 (device scope)
constexpr int kCpolSc1 = 16;
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// Block order.  Workgroups dispatch round-robin over the 8 XCDs (block b to XCD b % 8), each XCD
// with its own L2.  XCD x takes a contiguous share of the tiles whose frame has all three temporal
// taps, in tile-major order with the frame innermost (neighbouring frames share two of their
// three input frames), and after them a share of the first / last frames, which have two taps:
// the short workgroups run last and fill the final round.  Returns the tile index (all
// coordinates but the frame) and sets the frame od.
__device__ __forceinline__ uint32_t w32_block_order(uint32_t b, uint32_t total, int D, int &od) {
    const uint32_t xcd = b % 8u, k = b / 8u;
    const uint32_t q8 = total / 8u, r8 = total % 8u;
    const uint32_t s0 = xcd * q8 + min(xcd, r8), cnt = q8 + (xcd < r8 ? 1u : 0u);
    const uint32_t inner = D >= 3 ? (uint32_t)(D - 2) : 0u;
    const uint64_t interior = (uint64_t)(total / (uint32_t)D) * inner;
    // this XCD's interior share: [c0, c1) of the interior list, proportional to its block count
    const uint32_t c0 = (uint32_t)((uint64_t)s0 * interior / total);
    const uint32_t c1 = (uint32_t)((uint64_t)(s0 + cnt) * interior / total);
    if (k < c1 - c0) {
        const uint32_t li = c0 + k;
        od = 1 + (int)(li % inner);
        return li / inner;
    }
    const uint32_t le = (s0 - c0) + (k - (c1 - c0));
    if (D >= 3) {
        od = (le & 1u) ? D - 1 : 0;
        return le >> 1;
    }
    od = (int)(le % (uint32_t)D);
    return le / (uint32_t)D;
}

// Stream-K order (SK): the stages of all tiles form one list -- output-row tile outermost, then
// sample and spatial tile, then frame, then the tile's own stages (chunk, live temporal tap) --
// and logical workgroup g of G takes the stages [g*S/G, (g+1)*S/G) of the S in the list.  Logical
// workgroups g of one XCD are consecutive (block b runs on XCD b % 8).  Within a spatial tile the
// frames run in the order 1, 0, 2, 3, ..., D-1 (D >= 3): a three-tap frame, then a two-tap one,
// so that with G about the number of tiles a range is most of one tile and the end or the start
// of its neighbour, and the workgroups of an XCD walk K nearly together (their weight stream
// stays in its L2).
__device__ __forceinline__ uint32_t sk_bound(uint32_t h, uint32_t total, uint32_t G) {
    return (uint32_t)((uint64_t)h * total / G);
}
// the logical workgroup whose range holds stage xs
__device__ __forceinline__ uint32_t sk_owner(uint32_t xs, uint32_t total, uint32_t G) {
    return (uint32_t)(((uint64_t)(xs + 1) * G - 1) / total);
}
__host__ __device__ __forceinline__ int sk_frame(int i, int D) { return D >= 3 && i < 2 ? 1 - i : i; }

// SK = false: one workgroup per (tile, K split), as w32_block_order assigns.  SK = true
// (stream-K): a.sk_groups workgroups, each walking its range of the stream-K order as segments
// (a tile's stages inside the range); a segment that is a whole tile is stored directly, the
// pieces of a split tile meet through fp32 partials (see the end of the segment loop).
template <bool BF, int EPI, bool SPLITK, int LW, int NB, int S, bool SK = false>
__global__ __launch_bounds__(256, 1) void igemm32_kernel(IgemmKArgs a) {
    using E = Elem<BF>;
    using G = W32Geom<LW, NB, S>;
    typedef typename E::vec8 vec8;
    typedef __attribute__((address_space(3))) void lds_void;
    static_assert(!(SK && SPLITK), "stream-K sums its own pieces");
    __shared__ __attribute__((aligned(16))) uint4 Win0[G::Slots];
    __shared__ __attribute__((aligned(16))) uint4 Win1[G::Slots];
    __shared__ __attribute__((aligned(16))) uint4 Win2[G::Slots];
    __shared__ float bias_s[256];   // this workgroup's 256 output rows (0 past C_out / no bias)
    __shared__ int sk_last;         // (SK) this workgroup's piece was the last of its tile to end

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane & 31, hh = lane >> 5;
    const int pr = j / LW, pc = j % LW;      // row / column of lane column j in its block

    const size_t frame_elems = (size_t)a.H_in * a.W_in * a.C_in;
    const uint32_t frame_bytes = (uint32_t)(frame_elems * 2);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)a.wp, (short)0, (int)(a.wp_bytes), 0x00020000);

    // (SK) logical workgroup g and its range [x, x_end) of the stream-K order
    uint32_t g = 0, x = 0, x_end = 0;
    if constexpr (SK) {
        const uint32_t G = (uint32_t)a.sk_groups;   // a multiple of 8
        g = (blockIdx.x % 8u) * (G / 8u) + blockIdx.x / 8u;
        x = sk_bound(g, a.sk_total, G);
        x_end = sk_bound(g + 1, a.sk_total, G);
    }
#pragma unroll 1
    for (;;) {
        int od, mt, n, th, tw, split = 0, kd_lo, nkd, sbase, nst;
        uint32_t t0 = 0, tile_len = 0, seg_hi = 0, tile_id = 0;   // (SK) the segment's tile
        if constexpr (SK) {
            if (x >= x_end) break;
            const uint32_t u = x / (uint32_t)a.sk_unit_stages;
            const uint32_t rem = x - u * (uint32_t)a.sk_unit_stages;
            // the frame whose stages hold rem (every frame has at least one live tap)
            uint32_t cum = 0;
            od = -1, kd_lo = 0, nkd = 0;
            for (int i = 0; i < a.D; ++i) {
                const int f = sk_frame(i, a.D);
                const int fi = f + a.d_org - 1;
                const int lo = max(0, a.d_lo - fi), hi = min(2, a.d_hi - 1 - fi);
                const uint32_t st = (uint32_t)(a.nchunks * max(0, hi - lo + 1));
                if (rem < cum + st) {
                    od = f, kd_lo = lo, nkd = hi - lo + 1, tile_len = st;
                    break;
                }
                cum += st;
            }
            if (od < 0) break;   // (not reached: the host sizes the order from the same taps)
            sbase = (int)(rem - cum);
            t0 = x - (uint32_t)sbase;
            seg_hi = min(tile_len, x_end - t0);
            nst = (int)seg_hi - sbase;
            const uint32_t nsp = (uint32_t)a.N * a.tiles_h * a.tiles_w;
            mt = (int)(u / nsp);
            uint32_t sp = u - (uint32_t)mt * nsp;
            tw = (int)(sp % (uint32_t)a.tiles_w);
            sp /= (uint32_t)a.tiles_w;
            th = (int)(sp % (uint32_t)a.tiles_h);
            n = (int)(sp / (uint32_t)a.tiles_h);
            tile_id = u * (uint32_t)a.D + (uint32_t)od;
        } else {
            uint32_t lin = w32_block_order(blockIdx.x, a.total_wg, a.D, od);
            mt = lin % a.mtiles;
            lin /= a.mtiles;
            tw = lin % a.tiles_w;
            lin /= a.tiles_w;
            th = lin % a.tiles_h;
            lin /= a.tiles_h;
            n = lin % a.N;
            split = lin / a.N;
            const int c_begin = split * a.chunks_per_split;
            const int c_end = min(a.nchunks, c_begin + a.chunks_per_split);
            // live temporal taps: input frame fi0 + kd inside [d_lo, d_hi)
            const int fi = od + a.d_org - 1;
            kd_lo = max(0, a.d_lo - fi);
            const int kd_hi = min(2, a.d_hi - 1 - fi);
            nkd = max(0, kd_hi - kd_lo + 1);
            sbase = c_begin * nkd;
            nst = max(0, (c_end - c_begin) * nkd);
        }

        const int oh0 = th * G::TH, ow0 = tw * G::TW;
        const int fi0 = od + a.d_org - 1;
        const int mbase = mt * 256 + wave * 64;       // this wave's first GEMM row
        const bool mlive = mbase < a.Mrows;           // (all-padding waves compute zeros, store none)

        // stage s of this segment is stage sbase + s of its tile: chunk t / nkd, temporal tap
        // kd_lo + t % nkd
        auto stage_coords = [&](int s, int &cc, int &kd) {
            const int t = sbase + s;
            cc = t / nkd;
            kd = kd_lo + t % nkd;
        };
        // Window copies: this wave issues copies k = wave + 4*t; lane i of copy k fills slot 64k + i
        // = position 16k + i/4 (row, column = position / RowPos, % RowPos), piece (i%4) ^
        // ((column/4) % 4).
        // The source offsets are recomputed per stage (a few ALU operations) rather than kept live.
        auto copy_window = [&](int s, uint4 *dst) {
            int cc, kd;
            stage_coords(s, cc, kd);
            const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(a.x + ((size_t)n * a.D_in + (fi0 + kd)) * frame_elems), (short)0,
                (int)frame_bytes, 0x00020000);
#pragma unroll
            for (int t = 0; t < G::CopiesPerWave; ++t) {
                const int k = wave + 4 * t;
                if (G::Copies % 4 != 0 && k >= G::Copies) break;   // wave-uniform
                const int pos = 16 * k + (lane >> 2);
                const int wh = pos / G::RowPos, ww = pos - wh * G::RowPos;
                const int piece = (lane & 3) ^ ((ww >> 2) & 3);
                // LDS column ww holds window column cw (input column S*ow0 - 1 + cw)
                const bool odd = S == 2 && ww >= G::OddBase;
                const int cw = S == 1 ? ww : (odd ? 2 * (ww - G::OddBase) + 1 : 2 * ww);
                const bool col_used = S == 1 ? ww < G::WW : (odd ? ww - G::OddBase < G::TW : ww < G::WW);
                const int h = S * oh0 - 1 + wh + a.h_org, w = S * ow0 - 1 + cw;
                const bool ok = col_used && pos < G::Pos && h >= a.h_lo && h < a.h_hi &&
                                (unsigned)w < (unsigned)a.W_in && cc * 32 + 8 * piece < a.C_in;
                const uint32_t off = ok ? (uint32_t)(((h * a.W_in + w) * a.C_in + cc * 32 + 8 * piece) * 2) : 0xFFFFFFFFu;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void *)&dst[k * 64], 16, off, 0, 0, 0);
            }
        };
        // weight fragments of slice q (tap q/2, k half q%2) of the stage whose first slice starts at
        // scalar offset sb: 2 blocks of 32 rows; the per-lane part of the offset is fixed
        const uint32_t alane = (uint32_t)((mbase + j) * 32 + 16 * hh);
        auto stage_abase = [&](int s) {
            int cc, kd;
            stage_coords(s, cc, kd);
            return (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(cc * 27 + kd * 9) * 2u * a.Mpad * 32u));
        };
        const uint32_t slice_bytes = (uint32_t)a.Mpad * 32u;   // one k16 slice of all rows
        auto load_a = [&](uint32_t sb, int q, vec8 (&dst)[2]) {
            const uint32_t sbase = sb + (uint32_t)q * slice_bytes;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
                dst[mb] = __builtin_bit_cast(vec8, __builtin_amdgcn_raw_buffer_load_b128(
                    wr, alane + mb * 1024u, sbase, 0));
        };
        // B fragment of slice q, block nb (rows R*nb .. +R-1 of the tile) from a window
        // buffer: a per-lane slot for (kx, k half) -- six values -- plus a compile-time row offset
        int lslot[3][2];
#pragma unroll
        for (int kx = 0; kx < 3; ++kx)
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const int col = S == 1 ? pc + kx : (kx == 1 ? G::OddBase + pc : pc + kx / 2);
                lslot[kx][k2] = w32_slot<G::RowPos>(S * pr, col, 2 * k2 + hh);
            }
        auto read_b = [&](const uint4 *win, int q, int nb) {
            const int tap = q / 2, ky = tap / 3, kx = tap % 3;
            return __builtin_bit_cast(vec8, win[lslot[kx][q % 2] + (S * G::R * nb + ky) * (G::RowPos * 4)]);
        };

        // (every launched workgroup has at least one stage: splits are never empty and every
        // output frame has a live temporal tap)
        f32x16_t acc[2][G::NB];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < G::NB; ++nb) {
                acc[mb][nb] = f32x16_t{};
                w32_touch(acc[mb][nb]);   // keeps the accumulators in AGPRs from the start
            }
        vec8 aq[kW32PD][2];
        vec8 bq[2][G::NB];

        {
            const int m = mt * 256 + threadIdx.x;
            bias_s[threadIdx.x] = (!SPLITK && a.bias != nullptr && m < a.Mrows) ? E::to_f32(a.bias[m]) : 0.f;
        }
        copy_window(0, Win0);
        if (nst > 1) copy_window(1, Win1);
        if (nst > 2) copy_window(2, Win2);
        uint32_t sb_cur = stage_abase(0);
#pragma unroll
        for (int q = 0; q < kW32PD; ++q) load_a(sb_cur, q, aq[q]);
        // windows 0..2 complete: younger than them are only the weight loads
        __builtin_amdgcn_s_waitcnt(w32_waitcnt_vm(kW32PD * 2));
        w32_barrier();
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb) bq[0][nb] = read_b(Win0, 0, nb);

        // Stage s computes from window buffer s % 3.  Window s+1 is complete for every wave from the
        // barrier that ends stage s-1 on, so the last slice of stage s already reads the first
        // fragments of stage s+1 and the MFMA pipe runs through the stage boundary.  The barrier that
        // ends stage s says every wave is done with window s (its buffer then takes window s+3) and
        // has its own copies of window s+2 complete.
#pragma unroll 1
        for (int s0 = 0; s0 < nst; s0 += 3) {
#pragma unroll
            for (int third = 0; third < 3; ++third) {
                const int s = s0 + third;
                if (third > 0 && s >= nst) break;              // uniform
                uint4 *const cur = third == 0 ? Win0 : third == 1 ? Win1 : Win2;
                uint4 *const nxt = third == 0 ? Win1 : third == 1 ? Win2 : Win0;
                const bool more = s + 1 < nst;
                // weights of the next stage (a stage past the last re-reads this one's, never used)
                const uint32_t sb_next = more ? stage_abase(s + 1) : sb_cur;
#pragma unroll
                for (int q = 0; q < kW32Slices; ++q) {
                    const int cb = q & 1;
                    if (q + 1 < kW32Slices) {
#pragma unroll
                        for (int nb = 0; nb < G::NB; ++nb) bq[cb ^ 1][nb] = read_b(cur, q + 1, nb);
                    } else {
                        // (after the last stage these reads are of a stale buffer and never used;
                        // issuing them anyway keeps the wait counts the same on every path)
#pragma unroll
                        for (int nb = 0; nb < G::NB; ++nb) bq[cb ^ 1][nb] = read_b(nxt, 0, nb);
                    }
                    // the next slice's reads go out before this slice's MFMAs (left to itself the
                    // scheduler sinks them behind the MFMAs and single-buffers the fragments)
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                        for (int nb = 0; nb < G::NB; ++nb)
                            acc[mb][nb] = E::mfma32x32x16(aq[q % kW32PD][mb], bq[cb][nb], acc[mb][nb]);
                    // refill the ring slot with the slice kW32PD ahead (in the next stage when past
                    // this one)
                    if (q + kW32PD < kW32Slices) load_a(sb_cur, q + kW32PD, aq[q % kW32PD]);
                    else load_a(sb_next, q + kW32PD - kW32Slices, aq[q % kW32PD]);
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (more) {
                    // own copies of window s+2 complete: they were issued after the previous
                    // barrier, and only this stage's weight loads (2 per slice) came after them
                    __builtin_amdgcn_s_waitcnt(w32_waitcnt_vm(2 * kW32Slices));
                    __builtin_amdgcn_s_waitcnt(kW32WaitLgkm0);
                    w32_barrier();
                    if (s + 3 < nst) copy_window(s + 3, cur);
                }
                sb_cur = sb_next;
            }
        }
        __builtin_amdgcn_s_waitcnt(w32_waitcnt_vm(0));

        const size_t P = (size_t)a.N * a.D * a.H * a.W;
        if (!SK || (sbase == 0 && seg_hi == tile_len)) {   // a whole tile: store it
#pragma unroll
            for (int nb = 0; nb < G::NB; ++nb) {
                const int oh = oh0 + G::R * nb + pr, ow = ow0 + pc;
                const bool inside = oh < a.H && ow < a.W;
                const size_t pos = (((size_t)n * a.D + od) * a.H + oh) * a.W + ow;
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) {
                    w32_touch(acc[mb][nb]);
                    if (inside && mlive) {
#pragma unroll
                        for (int gq = 0; gq < 4; ++gq) {
                            const f32x16_t v = acc[mb][nb];
                            const int m0 = mbase + mb * 32 + 8 * gq + 4 * hh;
                            const float4 bv = *reinterpret_cast<const float4 *>(&bias_s[m0 - mt * 256]);
                            store_rows<BF, EPI, SPLITK>(a, f32x4_t{v[4 * gq] + bv.x, v[4 * gq + 1] + bv.y,
                                                                  v[4 * gq + 2] + bv.z, v[4 * gq + 3] + bv.w},
                                                       pos, split, P, m0);
                        }
                    }
                }
            }
        } else if constexpr (SK) {
            // A piece of a split tile.  The tile's pieces are held by logical workgroups gf .. gl in
            // K order; each writes its fp32 partial tile to a slot of its own (slot 1 of gf -- the
            // piece that starts the tile is the last segment of its workgroup -- and slot 0 of every
            // later one, for which it is the first segment), then takes a ticket from the tile's
            // arrival counter.  The piece that draws the last ticket sums the np pieces in K order
            // -- its own from registers, the others from their slots -- so the sum does not depend
            // on which piece ends last, adds the bias, applies the epilogue and stores.  The
            // counters are cleared before the launch.
            // Coherence across XCDs (each has its own L2) without flushing or invalidating the L2s
            // (their weight and window lines are what the other workgroups run on): the partial
            // tiles are written and read with device-scope accesses (sc1, write-through /
            // coherent read, as relaxed device-scope atomics are), a piece's stores are complete
            // (vmcnt 0) before its ticket is taken, and the ticket is a device-scope atomic.
            constexpr int kChunks = 2 * G::NB * 4;   // 16-byte parts of a lane's accumulators
            constexpr uint32_t kSlotBytes = kChunks * 256 * 16;
            const uint32_t ng = (uint32_t)a.sk_groups;
            const uint32_t gf = sk_owner(t0, a.sk_total, ng), gl = sk_owner(t0 + tile_len - 1, a.sk_total, ng);
            const int np = (int)(gl - gf) + 1, me = (int)(g - gf);
            const __amdgpu_buffer_rsrc_t pr_rs = __builtin_amdgcn_make_buffer_rsrc(
                (void *)a.partial, (short)0, (int)(2 * ng * kSlotBytes), 0x00020000);
            // byte offset of this thread's part c of piece p's slot
            auto slot_off = [&](int p, int c) {
                return ((gf + (uint32_t)p) * 2u + (p == 0 ? 1u : 0u)) * kSlotBytes +
                       (uint32_t)(c * 256 + (int)threadIdx.x) * 16u;
            };
            if (mlive) {
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int nb = 0; nb < G::NB; ++nb) {
                        w32_touch(acc[mb][nb]);
                        const f32x16_t v = acc[mb][nb];
#pragma unroll
                        for (int gq = 0; gq < 4; ++gq)
                            __builtin_amdgcn_raw_buffer_store_b128(
                                __builtin_bit_cast(u32x4_t, f32x4_t{v[4 * gq], v[4 * gq + 1], v[4 * gq + 2], v[4 * gq + 3]}),
                                pr_rs, slot_off(me, (mb * G::NB + nb) * 4 + gq), 0, kCpolSc1);
                    }
            }
            __builtin_amdgcn_s_waitcnt(w32_waitcnt_vm(0));
            __syncthreads();
            if (threadIdx.x == 0)
                sk_last = __hip_atomic_fetch_add(a.sk_count + tile_id, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(np - 1);
            __syncthreads();
            if (__builtin_amdgcn_readfirstlane(sk_last) && mlive && np == 2) {
                // Two pieces (the usual split): the other piece's whole slot in one burst of loads
                // -- one round trip instead of one per 32-row block -- then own + other, which
                // (addition commuting) are the same bits as the K-order sum, whichever piece
                // ended last.
                f32x4_t ld[2][G::NB][4];
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
                        for (int gq = 0; gq < 4; ++gq)
                            ld[mb][nb][gq] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                pr_rs, slot_off(1 - me, (mb * G::NB + nb) * 4 + gq), 0, kCpolSc1));
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int nb = 0; nb < G::NB; ++nb) {
                        w32_touch(acc[mb][nb]);
                        const f32x16_t v = acc[mb][nb];
                        const int oh = oh0 + G::R * nb + pr, ow = ow0 + pc;
                        if (oh >= a.H || ow >= a.W) continue;
                        const size_t pos = (((size_t)n * a.D + od) * a.H + oh) * a.W + ow;
#pragma unroll
                        for (int gq = 0; gq < 4; ++gq) {
                            const f32x4_t o = ld[mb][nb][gq];
                            const int m0 = mbase + mb * 32 + 8 * gq + 4 * hh;
                            const float4 bv = *reinterpret_cast<const float4 *>(&bias_s[m0 - mt * 256]);
                            store_rows<BF, EPI, false>(a, f32x4_t{(v[4 * gq] + o[0]) + bv.x, (v[4 * gq + 1] + o[1]) + bv.y,
                                                                  (v[4 * gq + 2] + o[2]) + bv.z, (v[4 * gq + 3] + o[3]) + bv.w},
                                                       pos, 0, P, m0);
                        }
                    }
            } else if (__builtin_amdgcn_readfirstlane(sk_last)) {
                if (mlive) {
#pragma unroll
                    for (int mb = 0; mb < 2; ++mb) {
                        f32x4_t sum[G::NB][4] = {};
                        // pieces before this one, then this one, then the pieces after it
                        auto add_slot = [&](int p) {
                            f32x4_t ld[G::NB][4];
#pragma unroll
                            for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
                                for (int gq = 0; gq < 4; ++gq)
                                    ld[nb][gq] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                        pr_rs, slot_off(p, (mb * G::NB + nb) * 4 + gq), 0, kCpolSc1));
#pragma unroll
                            for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
                                for (int gq = 0; gq < 4; ++gq) sum[nb][gq] = p == 0 ? ld[nb][gq] : sum[nb][gq] + ld[nb][gq];
                        };
#pragma unroll 1
                        for (int p = 0; p < me; ++p) add_slot(p);
#pragma unroll
                        for (int nb = 0; nb < G::NB; ++nb) {
                            w32_touch(acc[mb][nb]);
                            const f32x16_t v = acc[mb][nb];
#pragma unroll
                            for (int gq = 0; gq < 4; ++gq) {
                                const f32x4_t own = f32x4_t{v[4 * gq], v[4 * gq + 1], v[4 * gq + 2], v[4 * gq + 3]};
                                sum[nb][gq] = me == 0 ? own : sum[nb][gq] + own;
                            }
                        }
#pragma unroll 1
                        for (int p = me + 1; p < np; ++p) add_slot(p);
#pragma unroll
                        for (int nb = 0; nb < G::NB; ++nb) {
                            const int oh = oh0 + G::R * nb + pr, ow = ow0 + pc;
                            if (oh >= a.H || ow >= a.W) continue;
                            const size_t pos = (((size_t)n * a.D + od) * a.H + oh) * a.W + ow;
#pragma unroll
                            for (int gq = 0; gq < 4; ++gq) {
                                const int m0 = mbase + mb * 32 + 8 * gq + 4 * hh;
                                const float4 bv = *reinterpret_cast<const float4 *>(&bias_s[m0 - mt * 256]);
                                const f32x4_t v = sum[nb][gq];
                                store_rows<BF, EPI, false>(a, f32x4_t{v[0] + bv.x, v[1] + bv.y, v[2] + bv.z, v[3] + bv.w},
                                                           pos, 0, P, m0);
                            }
                        }
                    }
                }
            }
        }
        if constexpr (!SK) {
            break;
        } else {
            x = t0 + seg_hi;
            __syncthreads();   // the next segment rewrites bias_s and the window buffers
        }
    }
}

// The 27-tap convolution when the output alone cannot fill the chip but K is long (few positions,
// many input channels): a workgroup computes one 64-row x 128-position tile, and its four waves
// split K four ways instead of the workgroups.  Wave q walks its own quarter of the 32-channel
// chunks with its own pair of window buffers in LDS and its own weight stream -- nothing is shared
// in the K loop, so it has no barrier: a wave waits only for its own copies -- and afterwards the
// four partial tiles are summed once through LDS, in the same order (wave 0, 1, 2, 3) for every
// output, and wave q stores 32-position block q of the tile.  No fp32 partials leave the CU and
// no second kernel runs.  Operand layout, window layout and weight packing are those of
// igemm32_kernel (a 64-row tile is two of its 32-row fragments).
template <bool BF, int EPI, int LW>
__global__ __launch_bounds__(256, 1) void igemm32_kq_kernel(IgemmKArgs a) {
    using E = Elem<BF>;
    using G = W32Geom<LW, 4, 1>;
    typedef typename E::vec8 vec8;
    typedef __attribute__((address_space(3))) void lds_void;
    // window buffer pair of each wave (even / odd stages); afterwards the partial tiles
    __shared__ __attribute__((aligned(16))) uint4 Win0[4][G::Slots];
    __shared__ __attribute__((aligned(16))) uint4 Win1[4][G::Slots];
    __shared__ __attribute__((aligned(16))) float bias_s[64];   // the tile's 64 rows (0 past C_out)
    static_assert(4 * G::Slots >= 2 * 6 * 256, "two waves' partial blocks fit one buffer set");

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane & 31, hh = lane >> 5;
    const int pr = j / LW, pc = j % LW;

    int od;
    uint32_t lin = w32_block_order(blockIdx.x, a.total_wg, a.D, od);
    const int mt = lin % a.mtiles;
    lin /= a.mtiles;
    const int tw = lin % a.tiles_w;
    lin /= a.tiles_w;
    const int th = lin % a.tiles_h;
    lin /= a.tiles_h;
    const int n = lin % a.N;

    const int oh0 = th * G::TH, ow0 = tw * G::TW;
    // this wave's quarter of the chunks (every wave has at least one: nchunks >= 4)
    const int c_begin = (a.nchunks * wave) >> 2;
    const int c_end = (a.nchunks * (wave + 1)) >> 2;
    const int fi0 = od + a.d_org - 1;
    const int kd_lo = max(0, a.d_lo - fi0);
    const int kd_hi = min(2, a.d_hi - 1 - fi0);
    const int nkd = max(0, kd_hi - kd_lo + 1);
    const int nst = max(0, (c_end - c_begin) * nkd);
    const int mbase = mt * 64;                    // the tile's first GEMM row

    const size_t frame_elems = (size_t)a.H_in * a.W_in * a.C_in;
    const uint32_t frame_bytes = (uint32_t)(frame_elems * 2);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)a.wp, (short)0, (int)(a.wp_bytes), 0x00020000);

    auto stage_coords = [&](int s, int &cc, int &kd) {
        cc = c_begin + s / nkd;
        kd = kd_lo + s % nkd;
    };
    // The whole window of stage s, copied by this wave alone: lane i of copy k fills slot
    // 64k + i = position 16k + i/4, piece (i%4) ^ ((column/4) % 4), as in igemm32_kernel.
    auto copy_window = [&](int s, uint4 *dst) {
        int cc, kd;
        stage_coords(s, cc, kd);
        const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(a.x + ((size_t)n * a.D_in + (fi0 + kd)) * frame_elems), (short)0,
            (int)frame_bytes, 0x00020000);
#pragma unroll
        for (int k = 0; k < G::Copies; ++k) {
            const int pos = 16 * k + (lane >> 2);
            const int wh = pos / G::RowPos, ww = pos - wh * G::RowPos;
            const int piece = (lane & 3) ^ ((ww >> 2) & 3);
            const int h = oh0 - 1 + wh + a.h_org, w = ow0 - 1 + ww;
            const bool ok = ww < G::WW && pos < G::Pos && h >= a.h_lo && h < a.h_hi &&
                            (unsigned)w < (unsigned)a.W_in && cc * 32 + 8 * piece < a.C_in;
            const uint32_t off = ok ? (uint32_t)(((h * a.W_in + w) * a.C_in + cc * 32 + 8 * piece) * 2) : 0xFFFFFFFFu;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void *)&dst[k * 64], 16, off, 0, 0, 0);
        }
    };
    const uint32_t alane = (uint32_t)((mbase + j) * 32 + 16 * hh);
    auto stage_abase = [&](int s) {
        int cc, kd;
        stage_coords(s, cc, kd);
        return (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(cc * 27 + kd * 9) * 2u * a.Mpad * 32u));
    };
    const uint32_t slice_bytes = (uint32_t)a.Mpad * 32u;
    auto load_a = [&](uint32_t sb, int q, vec8 (&dst)[2]) {
        const uint32_t sbase = sb + (uint32_t)q * slice_bytes;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
            dst[mb] = __builtin_bit_cast(vec8, __builtin_amdgcn_raw_buffer_load_b128(
                wr, alane + mb * 1024u, sbase, 0));
    };
    int lslot[3][2];
#pragma unroll
    for (int kx = 0; kx < 3; ++kx)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) lslot[kx][k2] = w32_slot<G::RowPos>(pr, pc + kx, 2 * k2 + hh);
    auto read_b = [&](const uint4 *win, int q, int nb) {
        const int tap = q / 2, ky = tap / 3, kx = tap % 3;
        return __builtin_bit_cast(vec8, win[lslot[kx][q % 2] + (G::R * nb + ky) * (G::RowPos * 4)]);
    };

    f32x16_t acc[2][4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            acc[mb][nb] = f32x16_t{};
            w32_touch(acc[mb][nb]);
        }
    vec8 aq[kW32PD][2];
    vec8 bq[2][4];
    // the bias now, into LDS (read after the barriers below), not as loads in the epilogue
    if (threadIdx.x < 64) {
        const int m = mbase + (int)threadIdx.x;
        bias_s[threadIdx.x] = (a.bias != nullptr && m < a.Mrows) ? E::to_f32(a.bias[m]) : 0.f;
    }

    if (nst > 0) {
        // window 0, the first weight slices, then window 1: the first MFMAs wait for neither
        // window 1 nor (loads complete in order) anything issued after what they read
        copy_window(0, Win0[wave]);
        uint32_t sb_cur = stage_abase(0);
#pragma unroll
        for (int q = 0; q < kW32PD; ++q) load_a(sb_cur, q, aq[q]);
        if (nst > 1) copy_window(1, Win1[wave]);
        // window 0 complete (younger: the weight loads and window 1)
        if (nst > 1) __builtin_amdgcn_s_waitcnt(w32_waitcnt_vm(G::Copies + 2 * kW32PD));
        else __builtin_amdgcn_s_waitcnt(w32_waitcnt_vm(2 * kW32PD));
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) bq[0][nb] = read_b(Win0[wave], 0, nb);

        // Stage s reads buffer s % 2.  From stage 1 on, a stage starts by copying window s+1
        // into the buffer stage s-1 read (its reads are complete); its last slice waits for
        // that window -- younger than its copies are only this stage's 17 weight refills so
        // far -- and reads the first fragments of stage s+1 from it.
#pragma unroll 1
        for (int s0 = 0; s0 < nst; s0 += 2) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int s = s0 + half;
                if (half > 0 && s >= nst) break;              // uniform
                uint4 *const cur = half == 0 ? Win0[wave] : Win1[wave];
                uint4 *const nxt = half == 0 ? Win1[wave] : Win0[wave];
                const bool more = s + 1 < nst;
                if (s > 0 && more) {
                    __builtin_amdgcn_s_waitcnt(kW32WaitLgkm0);
                    copy_window(s + 1, nxt);
                }
                const uint32_t sb_next = more ? stage_abase(s + 1) : sb_cur;
#pragma unroll
                for (int q = 0; q < kW32Slices; ++q) {
                    const int cb = q & 1;
                    if (q + 1 < kW32Slices) {
#pragma unroll
                        for (int nb = 0; nb < 4; ++nb) bq[cb ^ 1][nb] = read_b(cur, q + 1, nb);
                    } else {
                        // (after the last stage these reads are of a stale buffer and never used)
                        if (more) __builtin_amdgcn_s_waitcnt(w32_waitcnt_vm(2 * (kW32Slices - 1)));
#pragma unroll
                        for (int nb = 0; nb < 4; ++nb) bq[cb ^ 1][nb] = read_b(nxt, 0, nb);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                        for (int nb = 0; nb < 4; ++nb)
                            acc[mb][nb] = E::mfma32x32x16(aq[q % kW32PD][mb], bq[cb][nb], acc[mb][nb]);
                    if (q + kW32PD < kW32Slices) load_a(sb_cur, q + kW32PD, aq[q % kW32PD]);
                    else load_a(sb_next, q + kW32PD - kW32Slices, aq[q % kW32PD]);
                    __builtin_amdgcn_sched_barrier(0);
                }
                sb_cur = sb_next;
            }
        }
    }
    // every copy of this wave has landed and every wave is done with its windows
    __builtin_amdgcn_s_waitcnt(w32_waitcnt_vm(0));
    __builtin_amdgcn_s_waitcnt(kW32WaitLgkm0);
    w32_barrier();

    // Partial blocks: wave w leaves its blocks nb != w for their owner wave nb; block (w, nb, mb)
    // is 256 float4 (element group g of lane l at 64g + l), waves 0, 1 in the first buffer set
    // and 2, 3 in the second.
    auto pblock = [&](int w, int nb, int mb) {
        f32x4_t *base = reinterpret_cast<f32x4_t *>((w < 2) ? &Win0[0][0] : &Win1[0][0]);
        const int kk = nb - (nb > w ? 1 : 0);
        return base + (((w & 1) * 3 + kk) * 2 + mb) * 256;
    };
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        if (nb == wave) continue;   // uniform
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            w32_touch(acc[mb][nb]);
            f32x4_t *dst = pblock(wave, nb, mb);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x16_t v = acc[mb][nb];
                dst[64 * g + lane] = f32x4_t{v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]};
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(kW32WaitLgkm0);
    w32_barrier();

    // Wave `wave` owns block nb = wave: sum over the four waves in order, bias, epilogue, store.
    const size_t P = (size_t)a.N * a.D * a.H * a.W;
    const int oh = oh0 + G::R * wave + pr, ow = ow0 + pc;
    const bool inside = oh < a.H && ow < a.W;
    const size_t pos = (((size_t)n * a.D + od) * a.H + oh) * a.W + ow;
#pragma unroll
    for (int nbq = 0; nbq < 4; ++nbq) {
        if (nbq != wave) continue;   // uniform: the block index stays compile-time
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            w32_touch(acc[mb][nbq]);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x16_t own = acc[mb][nbq];
                f32x4_t sum = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const f32x4_t v = w == nbq ? f32x4_t{own[4 * g], own[4 * g + 1], own[4 * g + 2], own[4 * g + 3]}
                                               : pblock(w, nbq, mb)[64 * g + lane];
                    sum = w == 0 ? v : sum + v;
                }
                const int m0 = mbase + mb * 32 + 8 * g + 4 * hh;
                if (inside && m0 < a.Mrows) {
                    const float4 bv = *reinterpret_cast<const float4 *>(&bias_s[m0 - mbase]);
                    store_rows<BF, EPI, false>(a, f32x4_t{sum[0] + bv.x, sum[1] + bv.y,
                                                          sum[2] + bv.z, sum[3] + bv.w},
                                               pos, 0, P, m0);
                }
            }
        }
    }
}

// Sums the split-K partials, adds the bias, applies the epilogue and rounds once.  One thread
// per (position, 4 channels).
template <bool BF, int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *part, const u16 *bias,
                                                            u16 *y, long long P, int C,
                                                            int splits) {
    using E = Elem<BF>;
    const int groups = (C + 3) / 4;
    const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
    if (t >= P * groups) return;
    const long long pos = t / groups;
    const int c0 = (int)(t - pos * groups) * 4;
    float s[4] = {0.f, 0.f, 0.f, 0.f};
    const bool vec = (C & 3) == 0;
    for (int k = 0; k < splits; ++k) {
        const float *src = part + ((size_t)k * P + pos) * C + c0;
        if (vec) {
            const f32x4_t v = *reinterpret_cast<const f32x4_t *>(src);
#pragma unroll
            for (int i = 0; i < 4; ++i) s[i] += v[i];
        } else {
            for (int i = 0; i < 4; ++i)
                if (c0 + i < C) s[i] += src[i];
        }
    }
    u16 *dst = y + pos * C + c0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (c0 + i >= C) break;
        float v = s[i];
        if (bias != nullptr) v += E::to_f32(bias[c0 + i]);
        dst[i] = E::from_f32(epilogue<EPI>(v));
    }
}

// Direct (27 taps): wp[((cc*27 + tap)*Mpad + m)*32 + k] <- w[co = m, ci = 32*cc + k, tap].
// Direct for the 32x32 kernel: wp[(((cc*27 + tap)*2 + k2)*Mpad + m)*16 + k] <- w[m, 32*cc + 16*k2
// + k, tap]: one 32-row fragment of one k16 slice is 1 KiB contiguous.
// Temporal (head kernels): 32-channel chunk c holds 1536 16-byte pieces in LDS order -- slot
// s = r*4 + q' of row r = kd*128 + m holds channels 32*c + 8*q .. +7, q = q' ^ head_lds_swizzle(r),
// of the weight for temporal tap kd and the (spatial tap, output channel) head_row_role(m) names.
// Rows past the real ones and channels past C_in are zero.
__global__ __launch_bounds__(256) void pack3d_kernel(const u16 *w, u16 *wp, int C_in, int C_out,
                                                     int NT, int Mpad, int family,
                                                     long long total) {
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    u16 v = 0;
    if (family == IG_W32) {
        const int k = (int)(idx & 15);
        long long r = idx >> 4;
        const int m = (int)(r % Mpad);
        r /= Mpad;
        const int k2 = (int)(r & 1);
        r >>= 1;
        const int tap = (int)(r % 27);
        const int cc = (int)(r / 27);
        const int ci = cc * 32 + k2 * 16 + k;
        if (ci < C_in && m < C_out) v = w[((size_t)m * C_in + ci) * 27 + tap];
    } else if (family != IG_TEMPORAL && family != IG_FUSED) {
        const int k = (int)(idx & 31);
        long long r = idx >> 5;
        const int m = (int)(r % Mpad);
        r /= Mpad;
        const int tap = (int)(r % NT);
        const int cc = (int)(r / NT);
        const int ci = cc * 32 + k;
        if (ci < C_in && m < C_out) v = w[((size_t)m * C_in + ci) * 27 + tap];
    } else {
        // IG_TEMPORAL: one row layout per chunk; IG_FUSED: three versions, version after chunk
        const int nver = family == IG_FUSED ? 3 : 1;
        const int cv = (int)(idx / (kHeadChunkPieces * 8));
        const int cc = cv / nver, ver = cv - cc * nver;
        const int rem = (int)(idx - (long long)cv * (kHeadChunkPieces * 8));
        const int slot = rem >> 3, e = rem & 7;
        const int r = slot >> 2;
        const int q = (slot & 3) ^ head_lds_swizzle(r);
        const int kd = r >> 7, m = r & 127;
        const int ci = cc * 32 + 8 * q + e;
        int tap, co;
        if (family == IG_FUSED) head_fused_role(m, ver, tap, co);
        else head_row_role(m, tap, co);
        if (ci < C_in && tap >= 0 && co < C_out)
            v = w[((size_t)co * C_in + ci) * 27 + kd * 9 + tap];
    }
    wp[idx] = v;
}

template <bool BF, int MB, int NBW, int WM, int WN, int TH, int TW>
hipError_t launch_family(const IgemmPlan &pl, const IgemmKArgs &ka, int epi, bool splitk,
                         hipStream_t s) {
    const dim3 grid((unsigned)pl.workgroups), block(256);
#define CX_IG(EPIV, SK) igemm3d_kernel<BF, MB, NBW, WM, WN, TH, TW, EPIV, SK><<<grid, block, 0, s>>>(ka)
    if (splitk) {
        CX_IG(EPI_NONE, true);
    } else if (epi == EPI_RELU) {
        CX_IG(EPI_RELU, false);
    } else if (epi == EPI_CLAMP1) {
        CX_IG(EPI_CLAMP1, false);
    } else {
        CX_IG(EPI_NONE, false);
    }
#undef CX_IG
    return hipGetLastError();
}

template <bool BF, int F>
hipError_t launch_narrow(const IgemmPlan &pl, const IgemmKArgs &ka, int epi, bool splitk, hipStream_t s) {
    const dim3 grid((unsigned)pl.workgroups), block(256);
    if (splitk) igemm3d_narrow_kernel<BF, EPI_NONE, true, F><<<grid, block, 0, s>>>(ka);
    else if (epi == EPI_RELU) igemm3d_narrow_kernel<BF, EPI_RELU, false, F><<<grid, block, 0, s>>>(ka);
    else if (epi == EPI_CLAMP1) igemm3d_narrow_kernel<BF, EPI_CLAMP1, false, F><<<grid, block, 0, s>>>(ka);
    else igemm3d_narrow_kernel<BF, EPI_NONE, false, F><<<grid, block, 0, s>>>(ka);
    return hipGetLastError();
}

template <bool BF, int LW, int NB, int S = 1>
hipError_t launch_w32(const IgemmKArgs &ka, int epi, bool splitk, dim3 grid, hipStream_t s) {
    const dim3 block(256);
    if (splitk) igemm32_kernel<BF, EPI_NONE, true, LW, NB, S><<<grid, block, 0, s>>>(ka);
    else if (epi == EPI_RELU) igemm32_kernel<BF, EPI_RELU, false, LW, NB, S><<<grid, block, 0, s>>>(ka);
    else if (epi == EPI_CLAMP1) igemm32_kernel<BF, EPI_CLAMP1, false, LW, NB, S><<<grid, block, 0, s>>>(ka);
    else igemm32_kernel<BF, EPI_NONE, false, LW, NB, S><<<grid, block, 0, s>>>(ka);
    return hipGetLastError();
}

// Clears the stream-K arrival counters (a kernel, not a memset: the launch pair stays
// capturable in a graph).
__global__ __launch_bounds__(256) void sk_clear_kernel(unsigned *count, long long n) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i < n) count[i] = 0u;
}

template <bool BF, int LW>
hipError_t launch_sk_tile(const IgemmKArgs &ka, int epi, hipStream_t s) {
    const dim3 grid((unsigned)ka.sk_groups), block(256);
    if (epi == EPI_RELU) igemm32_kernel<BF, EPI_RELU, false, LW, 4, 1, true><<<grid, block, 0, s>>>(ka);
    else if (epi == EPI_CLAMP1) igemm32_kernel<BF, EPI_CLAMP1, false, LW, 4, 1, true><<<grid, block, 0, s>>>(ka);
    else igemm32_kernel<BF, EPI_NONE, false, LW, 4, 1, true><<<grid, block, 0, s>>>(ka);
    return hipGetLastError();
}

// stream-K: stride 1, the 4-block tiles (8 x 16 or 4 x 32)
template <bool BF>
hipError_t launch_sk(const IgemmPlan &pl, const IgemmKArgs &ka, int epi, hipStream_t s) {
    if (pl.splits != 1 || pl.stride != 1 || pl.kq) return hipErrorInvalidValue;
    if (pl.TW == 16 && pl.TH == 8) return launch_sk_tile<BF, 16>(ka, epi, s);
    if (pl.TW == 32 && pl.TH == 4) return launch_sk_tile<BF, 32>(ka, epi, s);
    return hipErrorInvalidValue;
}

template <bool BF, int LW>
hipError_t launch_kq(const IgemmKArgs &ka, int epi, dim3 grid, hipStream_t s) {
    const dim3 block(256);
    if (epi == EPI_RELU) igemm32_kq_kernel<BF, EPI_RELU, LW><<<grid, block, 0, s>>>(ka);
    else if (epi == EPI_CLAMP1) igemm32_kq_kernel<BF, EPI_CLAMP1, LW><<<grid, block, 0, s>>>(ka);
    else igemm32_kq_kernel<BF, EPI_NONE, LW><<<grid, block, 0, s>>>(ka);
    return hipGetLastError();
}

template <bool BF>
hipError_t launch_igemm_dtype(const IgemmPlan &pl, const IgemmKArgs &ka, int epi, bool splitk,
                              hipStream_t s) {
    switch (pl.family) {
        case IG_W32: {
            const dim3 grid((unsigned)pl.workgroups);
            if (pl.kq) {   // stride 1, 128-position tiles, no split-K
                if (splitk || pl.stride != 1) return hipErrorInvalidValue;
                if (pl.TW == 16 && pl.TH == 8) return launch_kq<BF, 16>(ka, epi, grid, s);
                if (pl.TW == 32 && pl.TH == 4) return launch_kq<BF, 32>(ka, epi, grid, s);
                return hipErrorInvalidValue;
            }
            if (pl.stride == 2) {   // 128-position tiles only (the stride-2 window is twice as big)
                if (pl.TW == 32 && pl.TH == 4) return launch_w32<BF, 32, 4, 2>(ka, epi, splitk, grid, s);
                if (pl.TW == 16 && pl.TH == 8) return launch_w32<BF, 16, 4, 2>(ka, epi, splitk, grid, s);
                return hipErrorInvalidValue;
            }
            if (pl.TW == 32) {
                if (pl.TH == 8) return launch_w32<BF, 32, 8>(ka, epi, splitk, grid, s);
                if (pl.TH == 4) return launch_w32<BF, 32, 4>(ka, epi, splitk, grid, s);
            } else if (pl.TW == 16) {
                if (pl.TH == 16) return launch_w32<BF, 16, 8>(ka, epi, splitk, grid, s);
                if (pl.TH == 8) return launch_w32<BF, 16, 4>(ka, epi, splitk, grid, s);
            }
            return hipErrorInvalidValue;
        }
        case IG_WIDE:
            return launch_family<BF, 4, 4, 2, 2, 8, 16>(pl, ka, epi, splitk, s);
        case IG_NARROW:
            return narrow_frames(ka.D) == 8 ? launch_narrow<BF, 8>(pl, ka, epi, splitk, s)
                                            : launch_narrow<BF, 4>(pl, ka, epi, splitk, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

IgemmPlan plan_igemm(int family, int N, int C_in, int C_out, int D, int H, int W, int stride) {
    IgemmPlan pl{};
    pl.family = family;
    pl.stride = stride;
    switch (family) {
        case IG_WIDE:
            pl.BM = 128, pl.TH = 8, pl.TW = 16, pl.ntaps = 27;
            pl.Mrows = C_out;
            break;
        case IG_NARROW:
            pl.BM = 16, pl.TH = 8, pl.TW = 32, pl.ntaps = 27;
            pl.Mrows = C_out;
            break;
        case IG_W32:   // tile geometry chosen with the split count below
            pl.BM = 256, pl.ntaps = 27;
            pl.Mrows = C_out;
            pl.TH = 8, pl.TW = 32;
            break;
        default:   // the head kernels: 3 temporal taps x 128 rows (9 * C_out used); the fused
                   // head's three row versions of them
            pl.BM = 128, pl.TH = 1, pl.TW = 256, pl.ntaps = family == IG_FUSED ? 9 : 3;
            pl.Mrows = 128;
            break;
    }
    pl.Mpad = (pl.Mrows + pl.BM - 1) / pl.BM * pl.BM;
    pl.mtiles = pl.Mpad / pl.BM;
    // 32-channel chunks
    pl.nchunks = (C_in + 31) / 32;
    if (family == IG_TEMPORAL || family == IG_FUSED) {
        // 256 consecutive positions of one frame per workgroup (no spatial structure needed)
        pl.tiles_h = 1;
        pl.tiles_w = (int)(((long long)H * W + 255) / 256);
    } else {
        pl.tiles_h = (H + pl.TH - 1) / pl.TH;
        pl.tiles_w = (W + pl.TW - 1) / pl.TW;
    }
    // (the narrow kernel takes narrow_frames(D) output frames per workgroup)
    const int dunits = family == IG_NARROW ? (D + narrow_frames(D) - 1) / narrow_frames(D) : D;
    const long long base = (long long)N * dunits * pl.tiles_h * pl.tiles_w * pl.mtiles;
    // Split K when the output alone cannot fill the 256 compute units a few times over.
    int splits = 1;
    if (family == IG_W32 && base > 0) {
        // One workgroup per CU: pick the tile geometry and split count minimising rounds of 256
        // workgroups x (stages per workgroup x the tile's cost per stage + about one stage of
        // prologue/epilogue) plus the fp32 partials' round trip (8 bytes per partial element at
        // HBM speed: about one stage per 3.75 M).  A 4-block tile does half the MFMAs of an
        // 8-block one per stage for the same weight stream: about 0.55 of its time.
        // (stride 2 takes the 4-block tiles only: its window is twice as big)
        static const struct { int TH, TW, NB; double cost; } geo[4] = {
            {8, 32, 8, 1.0}, {16, 16, 8, 1.0}, {4, 32, 4, 0.55}, {8, 16, 4, 0.55}};
        const double taps = D >= 3 ? (3.0 * D - 2.0) / D : (D == 2 ? 2.0 : 1.0);
        const int max_taps = D >= 3 ? 3 : D;
        const double part = (double)N * D * H * W * C_out / 3.75e6;
        double best = -1.0;
        // the chosen plan's rounds and per-round terms (for its one-round makespan below)
        long long best_rounds = 0;
        double best_units = 0.0, best_extra = 0.0;
        for (const auto &g : geo) {
            if (stride == 2 && g.NB != 4) continue;
            const long long th = (H + g.TH - 1) / g.TH, tw = (W + g.TW - 1) / g.TW;
            const long long gbase = (long long)N * D * th * tw * pl.mtiles;
            for (int sp = 1; sp <= pl.nchunks; ++sp) {
                const int cps = (pl.nchunks + sp - 1) / sp;
                const int se = (pl.nchunks + cps - 1) / cps;
                if (se != sp) continue;
                const long long rounds = (gbase * se + 255) / 256;
                const double extra = se > 1 ? se * part / rounds : 0.0;
                const double cost = rounds * (cps * taps * g.cost + 1.0 + extra);
                if (best < 0 || cost < best - 1e-9) {
                    best = cost, splits = se, pl.kq = 0;
                    pl.TH = g.TH, pl.TW = g.TW, pl.tiles_h = (int)th, pl.tiles_w = (int)tw;
                    best_rounds = rounds, best_units = cps * g.cost, best_extra = 1.0 + extra;
                }
            }
            // The same tile with 64 output rows per workgroup and K split over its four waves
            // (igemm32_kq_kernel): four times the workgroups of a 256-row tile, no partials;
            // about a fifth of a stage to sum the four partial tiles through LDS.  Stride 1,
            // and at least two chunks per wave.
            if (stride == 1 && g.NB == 4 && pl.nchunks >= 8) {
                const long long gq = (long long)N * D * th * tw * ((pl.Mrows + 63) / 64);
                const long long rounds = (gq + 255) / 256;
                const double cost = rounds * (((pl.nchunks + 3) / 4) * taps * g.cost + 1.2);
                if (cost < best - 1e-9) {
                    best = cost, splits = 1;
                    pl.TH = g.TH, pl.TW = g.TW, pl.tiles_h = (int)th, pl.tiles_w = (int)tw;
                    pl.kq = 1;
                    best_rounds = rounds, best_units = ((pl.nchunks + 3) / 4) * g.cost, best_extra = 1.2;
                }
            }
        }
        // Stream-K (igemm32_kernel<..., SK>) on the 4-block tiles, one workgroup per tile (the
        // count rounded up to a multiple of 8, at most one round): the workgroups take equal
        // shares of all tiles' stages, so the makespan is the average tile, where a plan that
        // runs in one round ends with its longest workgroups -- the interior frames' three
        // temporal taps, not the average the costs above use.  About 3.5 stages of overhead:
        // more prologues, the partials' round trip and the launch that clears the counters.
        // Stride 1.
        if (stride == 1 && best > 0) {
            double made = best_rounds == 1 ? best_units * max_taps + best_extra : best;
            const long long frame_taps = D >= 3 ? 3LL * D - 2 : (D == 2 ? 4 : 1);
            for (const auto &g : geo) {
                if (g.NB != 4) continue;
                const long long th = (H + g.TH - 1) / g.TH, tw = (W + g.TW - 1) / g.TW;
                const long long tiles = (long long)N * D * th * tw * pl.mtiles;
                const long long G = (tiles + 7) / 8 * 8;
                const long long total = (long long)N * th * tw * pl.mtiles * pl.nchunks * frame_taps;
                if (G > (long long)kSkMaxGroups || total >= (1LL << 31)) continue;
                const double cost = (double)((total + G - 1) / G) * g.cost + 3.5;
                if (cost < made - 1e-9) {
                    made = cost, splits = 1, pl.kq = 0, pl.sk = (int)G;
                    pl.TH = g.TH, pl.TW = g.TW, pl.tiles_h = (int)th, pl.tiles_w = (int)tw;
                }
            }
        }
        if (pl.kq) pl.mtiles = (pl.Mrows + 63) / 64;
    } else if (family != IG_TEMPORAL && family != IG_FUSED && base > 0 && base < 1024) {
        // (the 16x16 kernels run two workgroups per CU)
        splits = (int)((1024 + base - 1) / base);
        if (splits > pl.nchunks) splits = pl.nchunks;
    }
    pl.chunks_per_split = (pl.nchunks + splits - 1) / splits;
    pl.splits = (pl.nchunks + pl.chunks_per_split - 1) / pl.chunks_per_split;
    pl.workgroups = pl.sk ? (long long)pl.sk
                          : (long long)N * dunits * pl.tiles_h * pl.tiles_w * pl.mtiles * pl.splits;
    return pl;
}

size_t packed_bytes(const IgemmPlan &pl) {
    return (size_t)pl.nchunks * pl.ntaps * pl.Mpad * 32 * sizeof(u16);
}

// Stream-K: two partial slots per workgroup (the 4-block tile's 256 rows x 128 positions in
// fp32, 128 KiB each), then one arrival counter per tile.
static size_t sk_slots_bytes(const IgemmPlan &pl) { return (size_t)pl.sk * 2 * (2 * 4 * 4 * 256) * 16; }
static long long sk_tiles(const IgemmPlan &pl, int N, int D) {
    return (long long)N * pl.tiles_h * pl.tiles_w * pl.mtiles * D;
}

size_t splitk_workspace_bytes(const IgemmPlan &pl, int N, int D, int H, int W, int C_out) {
    if (pl.sk) return sk_slots_bytes(pl) + (size_t)sk_tiles(pl, N, D) * sizeof(unsigned);
    if (pl.splits <= 1) return 0;
    return (size_t)pl.splits * N * D * H * W * C_out * sizeof(float);
}

hipError_t launch_igemm3d(const IgemmPlan &pl, const IgemmParams &p, hipStream_t stream) {
    IgemmKArgs ka{};
    ka.x = static_cast<const u16 *>(p.x);
    ka.wp = static_cast<const u16 *>(p.wp);
    ka.bias = static_cast<const u16 *>(p.bias);
    ka.y = static_cast<u16 *>(p.y);
    ka.partial = p.partial;
    ka.N = p.N, ka.C_in = p.C_in, ka.D = p.D, ka.H = p.H, ka.W = p.W, ka.W_in = p.W_in;
    ka.D_in = p.rg.D_in, ka.H_in = p.rg.H_in, ka.d_org = p.rg.d_org, ka.h_org = p.rg.h_org;
    ka.d_lo = p.rg.d_lo, ka.d_hi = p.rg.d_hi, ka.h_lo = p.rg.h_lo, ka.h_hi = p.rg.h_hi;
    ka.Mrows = pl.Mrows, ka.Mpad = pl.Mpad, ka.Cy = p.Cy;
    ka.nchunks = pl.nchunks, ka.chunks_per_split = pl.chunks_per_split, ka.splits = pl.splits;
    ka.tiles_h = pl.tiles_h, ka.tiles_w = pl.tiles_w, ka.mtiles = pl.mtiles;
    ka.total_wg = (uint32_t)pl.workgroups;
    ka.wp_bytes = (uint32_t)packed_bytes(pl);
    if (pl.sk) {
        // the stream-K order's length: every (output-row tile, sample, spatial tile) has the
        // live temporal taps of each output frame times the chunks
        long long unit = 0;
        for (int od = 0; od < p.D; ++od) {
            const int fi = od + p.rg.d_org - 1;
            const int lo = fi < p.rg.d_lo ? p.rg.d_lo - fi : 0;
            const int hi = p.rg.d_hi - 1 - fi < 2 ? p.rg.d_hi - 1 - fi : 2;
            if (hi < lo) return hipErrorInvalidValue;   // (the region checks rule this out)
            unit += (long long)pl.nchunks * (hi - lo + 1);
        }
        const long long tiles = sk_tiles(pl, p.N, p.D);
        const long long total = unit * (tiles / p.D);
        if (p.partial == nullptr || total <= 0 || total >= (1LL << 31) || unit >= (1LL << 31))
            return hipErrorInvalidValue;
        ka.sk_count = reinterpret_cast<unsigned *>(reinterpret_cast<char *>(p.partial) + sk_slots_bytes(pl));
        ka.sk_groups = pl.sk;
        ka.sk_total = (uint32_t)total;
        ka.sk_unit_stages = (int)unit;
        sk_clear_kernel<<<dim3((unsigned)((tiles + 255) / 256)), dim3(256), 0, stream>>>(ka.sk_count, tiles);
        const hipError_t e = p.bf16 ? launch_sk<true>(pl, ka, p.epilogue, stream)
                                    : launch_sk<false>(pl, ka, p.epilogue, stream);
        return e;
    }
    const bool splitk = pl.splits > 1;
    hipError_t e = p.bf16 ? launch_igemm_dtype<true>(pl, ka, p.epilogue, splitk, stream)
                          : launch_igemm_dtype<false>(pl, ka, p.epilogue, splitk, stream);
    if (e != hipSuccess || !splitk) return e;
    const long long P = (long long)p.N * p.D * p.H * p.W;
    const long long threads = P * ((pl.Mrows + 3) / 4);
    const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
    const u16 *bias = static_cast<const u16 *>(p.bias);
    u16 *y = static_cast<u16 *>(p.y);
#define CX_RED(BFV, EPIV) \
    splitk_reduce_kernel<BFV, EPIV><<<grid, block, 0, stream>>>(p.partial, bias, y, P, pl.Mrows, pl.splits)
    if (p.bf16) {
        if (p.epilogue == EPI_RELU) CX_RED(true, EPI_RELU);
        else if (p.epilogue == EPI_CLAMP1) CX_RED(true, EPI_CLAMP1);
        else CX_RED(true, EPI_NONE);
    } else {
        if (p.epilogue == EPI_RELU) CX_RED(false, EPI_RELU);
        else if (p.epilogue == EPI_CLAMP1) CX_RED(false, EPI_CLAMP1);
        else CX_RED(false, EPI_NONE);
    }
#undef CX_RED
    return hipGetLastError();
}

hipError_t launch_pack3d(const IgemmPlan &pl, const void *w, void *wp, int C_in, int C_out,
                         hipStream_t stream) {
    const long long total = (long long)pl.nchunks * pl.ntaps * pl.Mpad * 32;
    if (total == 0) return hipSuccess;
    pack3d_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream>>>(
        static_cast<const u16 *>(w), static_cast<u16 *>(wp), C_in, C_out, pl.ntaps, pl.Mpad,
        pl.family, total);
    return hipGetLastError();
}

}  // namespace cx
