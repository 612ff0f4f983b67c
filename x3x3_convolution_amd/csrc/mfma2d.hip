// 2D pad-1 3x3 convolution of narrow layers (C_in, C_out <= 64) on the matrix cores, NCHW.
//
//   y[n,co,oh,ow] = E( b[co] + sum_{ci,ky,kx} w[co,ci,ky,kx] * X[n,ci, s*oh-1+ky, s*ow-1+kx] )
//
// [taesd_conv.cuh.new, header comment: the operator contract (NCHW, fp16 storage, fp32
// accumulation, pad 1, stride 1 or 2, optional bias and ReLU).]  The pages argue for a SIMT
// kernel at C <= 64 because matrix tiles would be under-filled on their hardware; on gfx950 a
// C = 64 layer at 256 x 256 has ~290 FLOP per compulsory byte, at the HBM / matrix-core ridge,
// so here the contraction runs on v_mfma_f32_32x32x16 (fp32 accumulation) and the kernel is a
// stream: input window in, output tile out.
//
// GEMM view per tile: rows = output channels (64, zero-padded), columns = output positions,
// K = 9 taps x 64 input channels (zero-padded), ordered (tap, channel).  Lane l supplies row (A)
// / column (B) l%32 with the 8 k values of half l/32 of a 16-wide k slice and receives
// accumulator element i at row 8*(i/4) + 4*(l/32) + i%4, column l%32.
//
// Persistent workgroups (one per CU: the LDS holds the whole weight set) walk the tiles; in
// each round the 256 workgroups take 256 consecutive tiles, each XCD a contiguous run of them
// (horizontally adjacent tiles share halo columns in that XCD's L2).
//   * Weights: read once per workgroup from OIHW and stored in LDS as 16-byte pieces of 8 input
//     channels, piece (tap, q, row) at ((tap*4 + q%4)*64 + row) of the array of channel half
//     q/4: a 32-row A fragment is 32 consecutive pieces.
//   * Input: a tile is 32 output columns x TH output rows (16 at stride 1, 4 at stride 2) and
//     runs as two 32-channel stages.  A stage's input window is loaded with 16-byte loads along
//     W (8 columns of one channel), transposed in registers (8 x 8 halves) and written to LDS
//     position-major: a position's 32 channels are four 16-byte pieces, stored XOR-permuted by
//     (column/4) % 4, so a fragment read of 32 consecutive columns hits distinct bank groups.
//     At stride 2 a window row holds its odd input columns first and its even ones after them
//     (the taps kx = 0, 2 read the odd ones, kx = 1 the even ones), so those reads are unit
//     stride too.  Two window buffers: the next stage's window is loaded while this one's
//     MFMAs run, one barrier per stage.
//   * Waves: eight per workgroup, two per SIMD, so one's vector work (window transposes,
//     stores) overlaps the other's MFMAs.  At stride 1 each owns all 64 rows and two output
//     rows (two 32-position blocks); at stride 2 each owns one output row and half the rows
//     (32 output channels), since a stride-2 tile is four output rows.
// Input columns are handled in aligned groups of 8, so W must be a multiple of 8 (checked by
// the host); rows, columns and channels outside the tensor load as zero (the zero padding).
#include "common.hpp"
#include "launch.hpp"

namespace cx {

namespace {

constexpr int kTW = 32;                  // output columns per tile
constexpr int kRows = 64;                // GEMM rows (output channels, zero-padded)
constexpr int kWPieces = 9 * 4 * kRows;  // weight pieces per 32-channel half (36 KiB)
constexpr int kWinSlots = 2592;          // 16-byte slots per window buffer (40.5 KiB)
constexpr uint32_t kOff = 0xFFFFFFFFu;   // past any buffer range; saturating adds keep it

template <int S>
struct M2Geom;
template <>
struct M2Geom<1> {
    static constexpr int NWaves = 8;     // two waves per SIMD
    static constexpr int TH = 16;        // output rows per tile
    static constexpr int NBW = 2;        // 32-position blocks per wave (output rows)
    static constexpr int MBW = 2;        // 32-row blocks per wave: all 64 output channels
    static constexpr int WRows = 18;     // window rows
    static constexpr int RowPos = 36;    // window row stride in positions (34 used)
    static constexpr int Groups = 6;     // 8-column load groups per window row (NCHW)
    static constexpr int WCols = 34;     // window columns (NHWC: one load per position piece)
    // the next window's columns are written after slices CommitFirst .. 17, (8 / (18 -
    // CommitFirst)) per slice: as late in the stage as possible (its loads were issued at the
    // stage's start), the transposes and LDS writes hidden between the MFMAs
    static constexpr int CommitFirst = 16;
};
template <>
struct M2Geom<2> {
    static constexpr int NWaves = 8;     // two waves per SIMD; wave w: output row w/2, channels
    static constexpr int TH = 4;         // 32*(w%2) .. +31
    static constexpr int NBW = 1;
    static constexpr int MBW = 1;
    static constexpr int WRows = 9;
    static constexpr int RowPos = 72;    // odd input columns at 0..32, even ones at 36..67
    static constexpr int Groups = 9;
    static constexpr int WCols = 65;
    static constexpr int CommitFirst = 16;
};
static_assert(M2Geom<1>::WRows * M2Geom<1>::RowPos * 4 == kWinSlots, "window size");
static_assert(M2Geom<2>::WRows * M2Geom<2>::RowPos * 4 == kWinSlots, "window size");
static_assert(8 % (18 - M2Geom<1>::CommitFirst) == 0 && 8 % (18 - M2Geom<2>::CommitFirst) == 0,
              "whole columns per slice");
static_assert(M2Geom<1>::NWaves * M2Geom<1>::MBW / 2 * M2Geom<1>::NBW == M2Geom<1>::TH,
              "waves cover the tile rows");
static_assert(M2Geom<2>::NWaves * M2Geom<2>::MBW / 2 * M2Geom<2>::NBW == M2Geom<2>::TH,
              "waves cover the tile rows");

struct Mfma2dKArgs {
    const u16 *x, *w, *bias;
    u16 *y;
    int N, C_in, C_out, H, W, Hout, Wout;
    int tiles_h, tiles_w, ntiles;
    uint32_t x_img_bytes, y_img_bytes, w_bytes;
};

__device__ __forceinline__ int m2_slot(int r, int c, int piece, int row_pos) {
    return (r * row_pos + c) * 4 + (piece ^ ((c >> 2) & 3));
}
__device__ __forceinline__ void m2_barrier() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ void m2_touch(f32x16_t &v) { asm volatile("" : "+a"(v)::"memory"); }
// dword i (a compile-time index) of a 16-byte vector
__device__ __forceinline__ uint32_t m2_dword(const uint4 &v, int i) {
    return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}
// waits for this thread's LDS writes only (the window stores); loads are consumed by then and
// global stores may still drain
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);
// halves h0 of a and h1 of b packed as (lo, hi)
__device__ __forceinline__ uint32_t m2_pack(uint32_t a, int h0, uint32_t b, int h1) {
    return ((a >> (16 * h0)) & 0xFFFFu) | (((b >> (16 * h1)) & 0xFFFFu) << 16);
}

// NHWC: channels-last x and y; C4 (NHWC only): C_out % 4 == 0, so a lane's four channels of a
// position are stored as one 8-byte piece.
template <bool BF, int S, int EPI, bool NHWC, bool C4>
__global__ __launch_bounds__(64 * M2Geom<S>::NWaves, 1) void mfma2d_kernel(Mfma2dKArgs a) {
    using E = Elem<BF>;
    using G = M2Geom<S>;
    constexpr int kThreads = 64 * G::NWaves;
    typedef typename E::vec8 vec8;
    __shared__ __attribute__((aligned(16))) uint4 Wc0[kWPieces];    // input channels 0..31
    __shared__ __attribute__((aligned(16))) uint4 Wc1[kWPieces];    // input channels 32..63
    __shared__ __attribute__((aligned(16))) uint4 Win0[kWinSlots];  // stage of channels 0..31
    __shared__ __attribute__((aligned(16))) uint4 Win1[kWinSlots];  // stage of channels 32..63
    __shared__ float bias_s[kRows];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // the wave's row group and first 32-row block: all 64 rows (MBW = 2) or half of them
    constexpr int MBW = G::MBW;
    const int wrow = MBW == 2 ? wave : wave >> 1;
    const int mb0 = MBW == 2 ? 0 : (wave & 1);
    const int j = lane & 31, hh = lane >> 5;
    const int HW = a.H * a.W;

    // ---- weights -> LDS, once per workgroup ----
    // Unit (row m, piece q of 8 input channels) reads the 8 x 9 contiguous halves
    // w[m][8q .. 8q+7][0..8] (144 bytes, 16-byte aligned since C_in % 8 == 0) and writes the
    // nine taps' pieces.
    {
        const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
            (void *)a.w, (short)0, (int)a.w_bytes, 0x00020000);
        for (int u = tid; u < kRows * 8; u += kThreads) {
            const int m = u & (kRows - 1), q = u >> 6;
            const bool ok = m < a.C_out && 8 * q < a.C_in;
            const uint32_t base = ok ? (uint32_t)((m * a.C_in + 8 * q) * 18) : kOff;
            uint32_t h[36];
#pragma unroll
            for (int i = 0; i < 9; ++i) {
                const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                    wr, __builtin_elementwise_add_sat(base, 16u * i), 0, 0));
                h[4 * i] = v.x, h[4 * i + 1] = v.y, h[4 * i + 2] = v.z, h[4 * i + 3] = v.w;
            }
            uint4 *dst = q < 4 ? Wc0 : Wc1;
#pragma unroll
            for (int t = 0; t < 9; ++t) {
                uint32_t d[4];
#pragma unroll
                for (int dd = 0; dd < 4; ++dd) {
                    const int e0 = (2 * dd) * 9 + t, e1 = (2 * dd + 1) * 9 + t;   // half indices
                    d[dd] = m2_pack(h[e0 >> 1], e0 & 1, h[e1 >> 1], e1 & 1);
                }
                dst[(t * 4 + (q & 3)) * kRows + m] = uint4{d[0], d[1], d[2], d[3]};
            }
        }
        if (tid < kRows)
            bias_s[tid] = (a.bias != nullptr && tid < a.C_out) ? E::to_f32(a.bias[tid]) : 0.f;
    }

    // ---- tiles of this workgroup ----
    const int nwg = gridDim.x;
    const int rank = (int)xcd_remap(blockIdx.x, (uint32_t)nwg);
    const int my_tiles = rank < a.ntiles ? (a.ntiles - 1 - rank) / nwg + 1 : 0;
    auto tile_coords = [&](int it, int &n, int &oh0, int &ow0) {
        int t = it * nwg + rank;
        const int tw = t % a.tiles_w;
        t /= a.tiles_w;
        const int th = t % a.tiles_h;
        n = t / a.tiles_h;
        oh0 = th * G::TH, ow0 = tw * kTW;
    };

    // ---- input window staging ----
    // NCHW: unit u = (window row, 8-column group, channel octet); a unit is eight 16-byte loads
    // along W (8 columns of one channel each), transposed in registers.  NHWC: unit u = (window
    // row, window column, 16-byte piece); a unit is one 16-byte load of 8 channels of one
    // position, already in the LDS order.
    // A thread owns units tid + k * kThreads.  The LDS slot a unit (column) goes to does not
    // depend on the tile, so it is computed once: columns outside the window (the unused part of
    // the NCHW edge groups) and units past the window go to a column no fragment read touches
    // (RowPos leaves spare columns in every row), which keeps the writes branch-free.
    constexpr int kUnits = NHWC ? G::WRows * G::WCols * 4 : G::WRows * G::Groups * 4;
    constexpr int kUPT = (kUnits + kThreads - 1) / kThreads;   // load units per thread
    constexpr int kLoads = NHWC ? 1 : 8;                       // 16-byte loads per unit
    constexpr int kTrash = S == 1 ? 34 : 33;
    uint4 sv[kUPT][kLoads];
    int wslot[kUPT][kLoads];
    // window column (input order, 0 = input column S*ow0 - 1) -> LDS column: at stride 2 the
    // even window columns (taps kx = 0, 2) come first and the odd ones (kx = 1) from column 36
    auto lds_col = [](int cw) { return S == 1 ? cw : ((cw & 1) ? 36 + (cw >> 1) : (cw >> 1)); };
#pragma unroll
    for (int k = 0; k < kUPT; ++k) {
        const int u = tid + kThreads * k;
        const bool uok = u < kUnits;
        if constexpr (NHWC) {
            const int o = u & 3, pos = uok ? u >> 2 : 0;
            const int r = pos / G::WCols, cw = pos - r * G::WCols;
            wslot[k][0] = m2_slot(r, uok ? lds_col(cw) : kTrash, o, G::RowPos);
        } else {
            const int o = u & 3, rg = u >> 2;
            const int g = rg % G::Groups;
            const int r = uok ? rg / G::Groups : 0;
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                int col;
                if constexpr (S == 1) {
                    col = g == 0 ? (x == 7 ? 0 : kTrash)
                                 : (g == G::Groups - 1 ? (x == 0 ? 33 : kTrash) : 1 + 8 * (g - 1) + x);
                } else {
                    col = g == 0 ? (x == 7 ? 0 : kTrash)
                                 : ((x & 1) ? 4 * (g - 1) + (x + 1) / 2 : 36 + 4 * (g - 1) + x / 2);
                }
                if (!uok) col = kTrash;
                wslot[k][x] = m2_slot(r, col, o, G::RowPos);
            }
        }
    }
    // loads of this thread's units for stage (tile it, channel half c)
    auto issue = [&](int it, int c) {
        int n, oh0, ow0;
        tile_coords(it, n, oh0, ow0);
        const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(a.x + (size_t)n * a.C_in * HW), (short)0, (int)a.x_img_bytes, 0x00020000);
#pragma unroll
        for (int k = 0; k < kUPT; ++k) {
            const int u = tid + kThreads * k;
            const int o = u & 3;
            const int ch0 = 32 * c + 8 * o;
            if constexpr (NHWC) {
                const int pos = u >> 2;
                const int r = pos / G::WCols, cw = pos - r * G::WCols;
                const int ih = S * oh0 - 1 + r, iw = S * ow0 - 1 + cw;
                const bool ok = u < kUnits && (unsigned)ih < (unsigned)a.H &&
                                (unsigned)iw < (unsigned)a.W && ch0 < a.C_in;
                const uint32_t off = ok ? (uint32_t)(((ih * a.W + iw) * a.C_in + ch0) * 2) : kOff;
                sv[k][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
            } else {
                const int rg = u >> 2;
                const int g = rg % G::Groups, r = rg / G::Groups;
                const int ih = S * oh0 - 1 + r;
                const int iw0 = S * ow0 - 8 + 8 * g;
                const bool ok = u < kUnits && (unsigned)ih < (unsigned)a.H &&
                                (unsigned)iw0 < (unsigned)a.W && ch0 < a.C_in;
                const uint32_t base = ok ? (uint32_t)(((ch0 * a.H + ih) * a.W + iw0) * 2) : kOff;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    sv[k][e] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                        xr, __builtin_elementwise_add_sat(base, (uint32_t)(e * HW * 2)), 0, 0));
            }
        }
    };
    // part x (0..7) of the loaded window into a window buffer.  NCHW: column x of every unit,
    // transposed to one position's 8 channels each (v_perm picks the two halves).  NHWC: units
    // [x*kUPT/8, (x+1)*kUPT/8) as they are.
    auto commit_col = [&](uint4 *win, int x) {
        if constexpr (NHWC) {
#pragma unroll
            for (int k = x * kUPT / 8; k < (x + 1) * kUPT / 8; ++k) win[wslot[k][0]] = sv[k][0];
        } else {
            const int dw = x >> 1;
            const uint32_t sel = (x & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
            for (int k = 0; k < kUPT; ++k) {
                uint32_t d[4];
#pragma unroll
                for (int dd = 0; dd < 4; ++dd)
                    d[dd] = __builtin_amdgcn_perm(m2_dword(sv[k][2 * dd + 1], dw),
                                                  m2_dword(sv[k][2 * dd], dw), sel);
                win[wslot[k][x]] = uint4{d[0], d[1], d[2], d[3]};
            }
        }
    };

    // ---- fragment addressing ----
    // B: window slot of (row, column) for tap column kx and k16 slice sl; the row part of this
    // wave and block is added as a compile-time offset plus the wave's base row.
    int lslot[3][2];
#pragma unroll
    for (int kx = 0; kx < 3; ++kx)
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
            const int col = S == 1 ? j + kx : (kx == 1 ? 36 + j : j + kx / 2);
            lslot[kx][sl] = m2_slot(S == 1 ? G::NBW * wrow : 2 * wrow, col, 2 * sl + hh, G::RowPos);
        }
    auto read_b = [&](const uint4 *win, int q, int nb) {
        const int tap = q >> 1, sl = q & 1, ky = tap / 3, kx = tap % 3;
        const int roff = S == 1 ? nb + ky : ky;
        return __builtin_bit_cast(vec8, win[lslot[kx][sl] + roff * (G::RowPos * 4)]);
    };
    const int abase = hh * kRows + j;
    auto read_a = [&](const uint4 *wc, int q, int mb) {
        const int tap = q >> 1, sl = q & 1;
        return __builtin_bit_cast(vec8, wc[abase + ((tap * 4 + 2 * sl) * kRows + mb * 32)]);
    };

    // Two accumulator sets: a tile's results are stored while the next tile's first stage runs
    // (its stores interleaved with the MFMAs), so the epilogue costs no matrix-core time.
    f32x16_t accA[MBW][G::NBW], accB[MBW][G::NBW];
    vec8 af[2][MBW], bq[2][G::NBW];
    const float4 *bias4 = reinterpret_cast<const float4 *>(bias_s);
    typedef f32x16_t AccSet[MBW][G::NBW];

    // ---- epilogue part: bias + E, one rounding, 4-byte stores along W (rows past C_out,
    // positions past the output go to an offset past the buffer range and are dropped).  Group
    // gi = (block nb, block mb, 4-row group g4) of a finished tile's accumulators. ----
    constexpr int kGroups = G::NBW * MBW * 4;
    constexpr int kGroupsPerSlice = (kGroups + 15) / 16;
    const bool odd = (j & 1) != 0;
    // per-lane constants of the stores: the lane's channel within a pair group (4*hh + odd) and
    // the v_perm selector that puts its own half low (even lane) or high (odd lane)
    const int HWo = a.Hout * a.Wout;
    const uint32_t psel = odd ? 0x01000504u : 0x05040100u;
    auto store_group = [&](AccSet &pacc, int gi, int oh0, int ow0,
                           const __amdgpu_buffer_rsrc_t &yr) __attribute__((always_inline)) {
        const int nb = gi / (4 * MBW), m = (gi / 4) % MBW, g4 = gi % 4;
        const int mb = mb0 + m;
        const int oh = oh0 + (S == 1 ? G::NBW * wrow + nb : wrow);
        if constexpr (NHWC) {
            // the lane's four consecutive channels m0 .. m0+3 of position (oh, ow0 + j): one
            // 8-byte store (channels past C_out and positions outside go to kOff)
            const int ow = ow0 + j;
            const int m0 = mb * 32 + 8 * g4 + 4 * hh;
            const uint32_t pb = oh < a.Hout && ow < a.Wout
                                    ? (uint32_t)(((oh * a.Wout + ow) * a.C_out + m0) * 2) : kOff;
            if (g4 == 0) m2_touch(pacc[m][nb]);
            uint32_t r[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) r[i] = E::from_f32(epilogue<EPI>(pacc[m][nb][4 * g4 + i]));
            if constexpr (C4) {
                typedef uint32_t v2u __attribute__((ext_vector_type(2)));
                const v2u v = {r[0] | (r[1] << 16), r[2] | (r[3] << 16)};
                __builtin_amdgcn_raw_buffer_store_b64(v, yr, m0 < a.C_out ? pb : kOff, 0, 0);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    __builtin_amdgcn_raw_buffer_store_b16(
                        (u16)r[i], yr, m0 + i < a.C_out ? __builtin_elementwise_add_sat(pb, 2u * i) : kOff, 0, 0);
            }
            return;
        }
        const int ow_even = ow0 + (j & ~1);   // Wout is even (W % 8 == 0): pairs never straddle
        // this lane's offset for channel 4*hh + odd of the group (rows past C_out fall past the
        // image and are dropped by the range check; positions outside go to kOff)
        const uint32_t lb = oh < a.Hout && ow_even < a.Wout
                                ? (uint32_t)(((4 * hh + (odd ? 1 : 0)) * HWo + oh * a.Wout + ow_even) * 2)
                                : kOff;
        if (g4 == 0) m2_touch(pacc[m][nb]);
        uint32_t r[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = E::from_f32(epilogue<EPI>(pacc[m][nb][4 * g4 + i]));
        // Lanes j, j^1 pair up: the even lane stores channels c, c+2 at columns (j, j+1), the
        // odd lane channels c+1, c+3 at (j-1, j): one 4-byte store per channel pair.
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
            const uint32_t A = r[2 * pr], B = r[2 * pr + 1];
            const uint32_t keep = odd ? B : A, send = odd ? A : B;
            const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0xB1, 0xF, 0xF, false);
            const uint32_t packed = __builtin_amdgcn_perm(recv, keep, psel);
            const uint32_t uo = (uint32_t)((mb * 32 + 8 * g4 + 2 * pr) * HWo * 2);
            __builtin_amdgcn_raw_buffer_store_b32(packed, yr, __builtin_elementwise_add_sat(lb, uo), 0, 0);
        }
    };
    auto y_rsrc = [&](int n) {
        return __builtin_amdgcn_make_buffer_rsrc(
            (void *)(a.y + (size_t)n * a.C_out * a.Hout * a.Wout), (short)0, (int)a.y_img_bytes,
            0x00020000);
    };

    // run one 32-channel stage into cacc: 18 k16 slices (9 taps x 2); the next stage's window
    // is written a few columns at a time after slices CommitFirst .. 17, and the previous tile's
    // results (pacc, tile pit) are stored over the first slices when has_prev
    auto run_stage = [&](AccSet &cacc, const uint4 *win, const uint4 *wc, uint4 *next_win,
                         bool has_next, AccSet &pacc, int pit, bool has_prev) __attribute__((always_inline)) {
        int pn = 0, poh0 = 0, pow0 = 0;
        tile_coords(pit, pn, poh0, pow0);
        const __amdgpu_buffer_rsrc_t yr = y_rsrc(pn);
#pragma unroll
        for (int m = 0; m < MBW; ++m) af[0][m] = read_a(wc, 0, mb0 + m);
#pragma unroll
        for (int nb = 0; nb < G::NBW; ++nb) bq[0][nb] = read_b(win, 0, nb);
#pragma unroll
        for (int q = 0; q < 18; ++q) {
            const int cb = q & 1;
            if (q + 1 < 18) {
#pragma unroll
                for (int m = 0; m < MBW; ++m) af[cb ^ 1][m] = read_a(wc, q + 1, mb0 + m);
#pragma unroll
                for (int nb = 0; nb < G::NBW; ++nb) bq[cb ^ 1][nb] = read_b(win, q + 1, nb);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int m = 0; m < MBW; ++m)
#pragma unroll
                for (int nb = 0; nb < G::NBW; ++nb)
                    cacc[m][nb] = E::mfma32x32x16(af[cb][m], bq[cb][nb], cacc[m][nb]);
            __builtin_amdgcn_sched_barrier(0);
            if (has_prev) {
#pragma unroll
                for (int k = 0; k < kGroupsPerSlice; ++k) {
                    const int gi = q * kGroupsPerSlice + k;
                    if (gi < kGroups) store_group(pacc, gi, poh0, pow0, yr);
                }
            }
            if (q >= G::CommitFirst && has_next) {
                constexpr int cps = 8 / (18 - G::CommitFirst);   // columns per slice
#pragma unroll
                for (int x = 0; x < cps; ++x) commit_col(next_win, (q - G::CommitFirst) * cps + x);
            }
        }
    };
    // one tile into cacc, storing the previous one's results (pacc) during its first stage
    auto tile_body = [&](AccSet &cacc, int it, AccSet &pacc, bool has_prev) __attribute__((always_inline)) {
        // the accumulators start at the bias of their channels (register i of block mb in
        // lane half hh: channel mb*32 + 8*(i/4) + 4*hh + i%4)
#pragma unroll
        for (int m = 0; m < MBW; ++m) {
            const int mb = mb0 + m;
            f32x16_t b16;
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const float4 bv = bias4[(mb * 32 + 8 * g4 + 4 * hh) >> 2];
                b16[4 * g4] = bv.x, b16[4 * g4 + 1] = bv.y, b16[4 * g4 + 2] = bv.z, b16[4 * g4 + 3] = bv.w;
            }
#pragma unroll
            for (int nb = 0; nb < G::NBW; ++nb) {
                cacc[m][nb] = b16;
                m2_touch(cacc[m][nb]);
            }
        }
        // stage 0 (channels 0..31, window buffer 0); the channels 32..63 window, loaded before
        // the previous tile's stores, goes to buffer 1
        run_stage(cacc, Win0, Wc0, Win1, true, pacc, it - 1, has_prev);
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        m2_barrier();
        // stage 1 (channels 32..63, buffer 1) while the next tile's first window loads
        const bool more = it + 1 < my_tiles;
        if (more) issue(it + 1, 0);
        run_stage(cacc, Win1, Wc1, Win0, more, pacc, it - 1, false);
        // The next tile's second window is loaded before the stores of this tile go out (in
        // the next tile's first stage), so waiting for those loads never waits for stores.
        if (more) issue(it + 1, 1);
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // this thread's window writes are done
        m2_barrier();
    };

    if (my_tiles > 0) {
        issue(0, 0);
#pragma unroll
        for (int x = 0; x < 8; ++x) commit_col(Win0, x);
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // the weight pieces, bias and first window are written
    m2_barrier();
    if (my_tiles > 0) issue(0, 1);

#pragma unroll 1
    for (int it = 0; it < my_tiles; it += 2) {
        tile_body(accA, it, accB, it > 0);
        if (it + 1 < my_tiles) tile_body(accB, it + 1, accA, true);
    }
    // the last tile's results
    if (my_tiles > 0) {
        const int last = my_tiles - 1;
        int n, oh0, ow0;
        tile_coords(last, n, oh0, ow0);
        const __amdgpu_buffer_rsrc_t yr = y_rsrc(n);
        if ((last & 1) == 0) {
#pragma unroll
            for (int gi = 0; gi < kGroups; ++gi) store_group(accA, gi, oh0, ow0, yr);
        } else {
#pragma unroll
            for (int gi = 0; gi < kGroups; ++gi) store_group(accB, gi, oh0, ow0, yr);
        }
    }
}

}  // namespace

bool mfma2d_supported(int C_in, int C_out, int H, int W, int stride, bool nhwc) {
    if (!(C_in >= 1 && C_in <= 64 && C_in % 8 == 0 && C_out >= 1 && C_out <= 64 &&
          (nhwc || W % 8 == 0) && (stride == 1 || stride == 2)))
        return false;
    // store offsets are formed for all 64 (padded) output channels of an image: 32-bit safe
    const long long hw_out = (long long)((H - 1) / stride + 1) * ((W - 1) / stride + 1);
    return H >= 1 && 64 * hw_out * 2 < (1ll << 31);
}

hipError_t launch_mfma2d(const Simt2dParams &p, hipStream_t stream) {
    Mfma2dKArgs a{};
    a.x = static_cast<const u16 *>(p.x);
    a.w = static_cast<const u16 *>(p.w);
    a.bias = static_cast<const u16 *>(p.bias);
    a.y = static_cast<u16 *>(p.y);
    a.N = p.N, a.C_in = p.C_in, a.C_out = p.C_out, a.H = p.H, a.W = p.W;
    a.Hout = p.Hout, a.Wout = p.Wout;
    const int TH = p.stride == 1 ? M2Geom<1>::TH : M2Geom<2>::TH;
    a.tiles_h = (p.Hout + TH - 1) / TH;
    a.tiles_w = (p.Wout + kTW - 1) / kTW;
    a.ntiles = p.N * a.tiles_h * a.tiles_w;
    a.x_img_bytes = (uint32_t)((size_t)p.C_in * p.H * p.W * 2);
    a.y_img_bytes = (uint32_t)((size_t)p.C_out * p.Hout * p.Wout * 2);
    a.w_bytes = (uint32_t)((size_t)p.C_out * p.C_in * 9 * 2);
    const int grid = a.ntiles < 256 ? a.ntiles : 256;
    if (grid == 0) return hipSuccess;
#define CX_M2(BFV, SV, EPIV)                                                                 \
    do {                                                                                     \
        const dim3 g_(grid), b_(64 * M2Geom<SV>::NWaves);                                    \
        if (!p.nhwc) mfma2d_kernel<BFV, SV, EPIV, false, false><<<g_, b_, 0, stream>>>(a);  \
        else if (p.C_out % 4 == 0) mfma2d_kernel<BFV, SV, EPIV, true, true><<<g_, b_, 0, stream>>>(a); \
        else mfma2d_kernel<BFV, SV, EPIV, true, false><<<g_, b_, 0, stream>>>(a);         \
    } while (0)
#define CX_M2E(BFV, SV)                                     \
    do {                                                    \
        if (p.epilogue == EPI_RELU) CX_M2(BFV, SV, EPI_RELU);   \
        else if (p.epilogue == EPI_CLAMP1) CX_M2(BFV, SV, EPI_CLAMP1); \
        else CX_M2(BFV, SV, EPI_NONE);                      \
    } while (0)
    if (p.bf16) {
        if (p.stride == 1) CX_M2E(true, 1);
        else CX_M2E(true, 2);
    } else {
        if (p.stride == 1) CX_M2E(false, 1);
        else CX_M2E(false, 2);
    }
#undef CX_M2E
#undef CX_M2
    return hipGetLastError();
}

}  // namespace cx
