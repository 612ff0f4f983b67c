// Host-side launchers of the gfx950 kernels.  Shapes are validated by the C ABI layer before any
// of these is called; each launcher only derives its grid and enqueues on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace cx {

// ---- 2D direct SIMT kernel (NCHW) ----------------------------------------------------------
struct Simt2dParams {
    const void *x, *w, *bias;
    void *y;
    int N, C_in, C_out, H, W, Hout, Wout, stride;
    bool bf16;
    bool nhwc;         // channels-last x and y (matrix-core kernel only)
    int epilogue;
};
hipError_t launch_simt2d(const Simt2dParams &p, hipStream_t stream);

// ---- 2D on the matrix cores (C_in and C_out <= 64, C_in % 8 == 0; NCHW also W % 8 == 0) ----
bool mfma2d_supported(int C_in, int C_out, int H, int W, int stride, bool nhwc);
hipError_t launch_mfma2d(const Simt2dParams &p, hipStream_t stream);

// ---- 3D input regions ------------------------------------------------------------------------
// Which input a 3D output reads: output frame od / row oh takes its temporal / vertical taps from
// input frames od + d_org - 1 + kd and rows oh + h_org - 1 + ky of x (stored extent D_in x H_in
// x W); only input frames [d_lo, d_hi) and rows [h_lo, h_hi) hold data, every other one reads as
// zero.  The plain convolution is the full region: D_in = D, H_in = H, origins 0, valid ranges
// the whole tensor.  Row bands with halo rows, frame chunks and causal temporal padding (with or
// without the previous chunk's frames) are other regions of the same sum.
struct ConvRegion {
    int D_in, H_in;
    int d_org, h_org;
    int d_lo, d_hi, h_lo, h_hi;
};
inline ConvRegion full_region(int D, int H) { return ConvRegion{D, H, 0, 0, 0, D, 0, H}; }

// ---- 3D MFMA implicit GEMM (NDHWC) ---------------------------------------------------------
// Tile families; the host picks one per request.
enum IgemmFamily {
    IG_WIDE = 0,   // 128 output rows x 128 positions per workgroup: C_out > 16
    IG_NARROW = 1, // 16 output rows x 256 positions: C_out <= 16 (the direct head), rows of x
                   // below 2 GiB / 10
    IG_TEMPORAL = 2, // packing only: 3 temporal taps x 128 rows (9 taps x 12 channels), head kernels
    IG_W32 = 3,     // 256 output rows x 8x32 positions on 32x32x16 MFMA: C_out > 16, one frame of
                    // x below 2 GiB (addressed through a 32-bit buffer range)
    IG_FUSED = 4    // packing only: the fused head's three row versions (head_fused_role) of
                    // 3 temporal taps x 128 rows per chunk
};

struct IgemmPlan {
    int family;
    int BM;            // output rows per workgroup
    int TH, TW;        // output positions per workgroup (rows x columns of one frame)
    int ntaps;         // 27 or 3
    int Mrows;         // rows that exist (C_out, or 112 for the split head's plane)
    int Mpad;          // packed rows = round_up(Mrows, BM)
    int nchunks;       // ceil(C_in / 32)
    int splits;        // split-K factor (1 = none)
    int chunks_per_split;
    int tiles_h, tiles_w, mtiles;
    long long workgroups;
    int stride;        // spatial stride (2: the 32x32 family's 128-position tiles only)
    int kq;            // 32x32 family: 1 = 64-row tiles whose four waves split K (no partials)
    int sk;            // 32x32 family: > 0 = stream-K with this many workgroups (they share the
                       // stages of all tiles evenly; split tiles meet through fp32 partials in the
                       // workspace), 0 = off
};

// Most workgroups of a stream-K launch: one round on the chip's 256 compute units.
constexpr int kSkMaxGroups = 256;

// Plans the MFMA launch (tile family, split-K) for a request over the output extent (D, H, W).
// Pure host arithmetic.
IgemmPlan plan_igemm(int family, int N, int C_in, int C_out, int D, int H, int W, int stride);

size_t packed_bytes(const IgemmPlan &pl);
// fp32 split-K partial sums, or 0 when splits == 1.
size_t splitk_workspace_bytes(const IgemmPlan &pl, int N, int D, int H, int W, int C_out);

struct IgemmParams {
    const void *x, *wp, *bias;
    void *y;           // output (C_out channels) or the split head's plane (112 channels)
    float *partial;    // split-K partials (splits > 1)
    int N, C_in, D, H, W;   // D, H, W: output extent
    int W_in;          // input width (W at stride 1)
    ConvRegion rg;     // input region (full_region(D, H_in) for the plain convolution)
    int Cy;            // channel stride of y
    bool bf16;
    int epilogue;
};
hipError_t launch_igemm3d(const IgemmPlan &pl, const IgemmParams &p, hipStream_t stream);

// Repack OIDHW weights for `pl` (family decides the row order).
hipError_t launch_pack3d(const IgemmPlan &pl, const void *w, void *wp, int C_in, int C_out,
                         hipStream_t stream);

// ---- split head, stage 2: nine-tap stencil over the 112-channel plane ----------------------
struct StencilParams {
    const void *g, *bias;
    void *y;
    int N, D, H, W, C_out;
    int g_off;         // plane rows carried above (and below) the H output rows: 0 or 1
    bool bf16;
    int epilogue;
};
hipError_t launch_head_stencil(const StencilParams &p, hipStream_t stream);

constexpr int kHeadPlaneChannels = 112;  // 9 taps x 12 channels = 108, padded to 7 x 16

// Packed weights of the head's temporal GEMM, per 32-channel chunk: 3 temporal taps x 128 GEMM
// rows x 32 channels = 1536 pieces of 16 bytes (8 channels), stored in the order the kernel's LDS
// holds them: piece slot s = r*4 + q' of row r = kd*128 + m holds channels 8*q .. 8*q+7 of the
// chunk with q = q' ^ head_lds_swizzle(r).
constexpr int kHeadChunkPieces = 3 * 128 * 4;
__host__ __device__ inline int head_lds_swizzle(int r) { return (r >> 2) & 3; }
// Role of GEMM row m (0..127).  Rows 0..95 (taps 0..7): the 32x32 matrix-core accumulator
// layout puts row m into register i = 4*((m%32)/8) + m%4 of 32-row block m/32 in lane half
// h = (m%8)/4; slot t = 16*(m/32) + i of half h carries spatial tap t/6 (ky*3 + kx) of output
// channel 6*h + t%6.  Rows 96..111: the 16-row tile of tap 8, row 96 + 8*h + c (c < 6) carrying
// output channel 6*h + c.  Every other row is padding (tap = -1).
__host__ __device__ inline void head_row_role(int m, int &tap, int &co) {
    if (m >= 96) {
        const int r = m - 96, h = (r >> 3) & 1, c = r & 7;
        tap = (r < 16 && c < 6) ? 8 : -1;
        co = 6 * h + c;
        return;
    }
    const int mb = m >> 5, rr = m & 31;
    const int h = (rr >> 2) & 1;
    const int t = 16 * mb + 4 * (rr >> 3) + (rr & 3);
    tap = t / 6;
    co = 6 * h + t % 6;
}

// The fused head's rows: the accumulators carry the stencil's vertical sum from Z row to Z row.
// Lane half hh of a wave holds three sets of 18 slots, set s = accumulator block s (16 slots) and
// register s of the two tap-8 tiles (the tile rows 4g + s, g = 2hh + j, j = 0, 1: slots 16 + j);
// slot q of a set holds horizontal tap kx = q / 6 of output channel 6hh + q % 6.  Set s belongs to
// the output rows o = s (mod 3): Z row zr adds its vertical tap ky = zr - o + 1 to the sets of
// output rows zr - 1, zr and zr + 1, so under the weight version v = zr mod 3 set s takes
// ky = (v + 1 - s) mod 3.  Sets tap = ky * 3 + kx (-1 for a padding row) and co of GEMM row m.
__host__ __device__ inline void head_fused_role(int m, int v, int &tap, int &co) {
    int s, hh, q;
    if (m < 96) {
        const int rr = m & 31;
        s = m >> 5;
        hh = (rr >> 2) & 1;
        q = 4 * (rr >> 3) + (rr & 3);
    } else {
        const int r8 = m - 96, g = r8 >> 2;
        s = r8 & 3;
        if (r8 >= 16 || s == 3) {
            tap = -1, co = 0;
            return;
        }
        hh = g >> 1;
        q = 16 + (g & 1);
    }
    const int ky = (v + 1 - s + 3) % 3;
    tap = ky * 3 + q / 6;
    co = 6 * hh + q % 6;
}

// ---- the head's temporal GEMM (packed like IG_TEMPORAL / IG_FUSED): plane output or fused
// stencil -----
struct HeadGemmParams {
    const void *x, *wp, *bias;
    void *out;         // the 112-channel plane (fused = false), y (fused = true) or, with rgb,
                       // the (N, D, 2H, 2W, 3) uint8 RGB frames of y
    int N, C_in, C_out, D, H, W;   // D, H: output extent
    ConvRegion rg;     // input region (full_region(D, H) for the plain convolution)
    bool bf16, fused;
    bool rgb;          // fused and C_out == 12 only
    int epilogue;      // fused only
};
hipError_t launch_head_gemm(const HeadGemmParams &p, hipStream_t stream);

// How the head kernels divide a request (pure host arithmetic).  A workgroup takes four
// consecutive output frames (a frame group) and one row range of the strip-major (strip, output
// row) order: range g is positions [bound[g], bound[g+1]), output row h of strip s being position
// s*H + h.  max_z_rows is the largest range's cost in Z rows (its output rows plus, fused, two
// halo rows per strip it touches).
constexpr int kHeadMaxRanges = 256;
struct HeadRangePlan {
    int strip_out, strips, fgroups, ranges, max_z_rows;
    long long workgroups;
    int bound[kHeadMaxRanges + 1];
};
HeadRangePlan plan_head_ranges(int N, int D, int H, int W, bool fused);

// ---- the head's 12-channel output as 8-bit RGB frames (factor-2 pixel shuffle) ------------
struct VideoParams {
    const void *y;     // (N, D, H, W, 12) NDHWC
    void *rgb;         // (N, D, 2H, 2W, 3) uint8
    int N, D, H, W;
    bool bf16;
};
hipError_t launch_video_rgb8(const VideoParams &p, hipStream_t stream);

}  // namespace cx
