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
#include "common.hpp"
#include "launch.hpp"

namespace cx {

namespace {

// Elements per LDS window position: 32 channels + 8 padding (80 bytes) so that the 16 positions
// one fragment reads fall on distinct bank groups.
constexpr int kPosStride = 40;

struct IgemmKArgs {
    const u16 *x;
    const u16 *wp;
    const u16 *bias;
    u16 *y;
    float *partial;
    int N, C_in, D, H, W;
    int Mrows, Mpad, Cy;
    int nchunks, chunks_per_split, splits;
    int tiles_h, tiles_w, mtiles;
    uint32_t total_wg;
};

// Stores the four rows (m0..m0+3) of one accumulator column: fp32 partials for split-K, or the
// bias + epilogue + one rounding to the storage type.
template <bool BF, int EPI, bool SPLITK>
__device__ __forceinline__ void store_col(const IgemmKArgs &a, f32x4_t v, size_t pos, int split,
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
        for (int i = 0; i < 4; ++i) {
            float s = v[i];
            if (a.bias != nullptr && m0 + i < a.Mrows) s += E::to_f32(a.bias[m0 + i]);
            o[i] = E::from_f32(epilogue<EPI>(s));
        }
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
    __shared__ __attribute__((aligned(16))) u16 win[2][FPOS * kPosStride];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM, wn = wave / WM;

    uint32_t lin = xcd_remap(blockIdx.x, a.total_wg);
    const int mt = lin % a.mtiles;
    lin /= a.mtiles;
    const int tw = lin % a.tiles_w;
    lin /= a.tiles_w;
    const int th = lin % a.tiles_h;
    lin /= a.tiles_h;
    const int od = lin % a.D;
    lin /= a.D;
    const int n = lin % a.N;
    const int split = lin / a.N;

    const int oh0 = th * TH, ow0 = tw * TW;
    const int c_begin = split * a.chunks_per_split;
    const int c_end = min(a.nchunks, c_begin + a.chunks_per_split);
    const int kd_lo = od == 0 ? 1 : 0;            // live temporal taps: frame od-1+kd in [0, D)
    const int kd_hi = od == a.D - 1 ? 1 : 2;
    const int nkd = kd_hi - kd_lo + 1;
    const int nst = (c_end - c_begin) * nkd;

    f32x4_t acc[MB][NBW];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NBW; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int mrow_lane = mt * BM + wm * MB * 16 + (lane & 15);
    const int kofs = (lane >> 4) * 8;
    const size_t frame_elems = (size_t)a.H * a.W * a.C_in;

    uint4 stg[PPT];
    auto fetch = [&](int s) {
        const int cc = c_begin + s / nkd, kd = kd_lo + s % nkd;
        const u16 *base = a.x + ((size_t)n * a.D + (od - 1 + kd)) * frame_elems + cc * 32;
#pragma unroll
        for (int j = 0; j < PPT; ++j) {
            const int i = tid + j * 256;
            uint4 v = {0u, 0u, 0u, 0u};
            if (PIECES % 256 == 0 || i < PIECES) {
                const int q = i & 3, pos = i >> 2;
                const int wh = pos / WW, ww = pos - wh * WW;
                const int h = oh0 - 1 + wh, w = ow0 - 1 + ww;
                if ((unsigned)h < (unsigned)a.H && (unsigned)w < (unsigned)a.W &&
                    cc * 32 + q * 8 < a.C_in)
                    v = *reinterpret_cast<const uint4 *>(base + ((size_t)h * a.W + w) * a.C_in + q * 8);
            }
            stg[j] = v;
        }
    };
    auto commit = [&](int buf) {
#pragma unroll
        for (int j = 0; j < PPT; ++j) {
            const int i = tid + j * 256;
            if (PIECES % 256 == 0 || i < PIECES)
                *reinterpret_cast<uint4 *>(&win[buf][(i >> 2) * kPosStride + (i & 3) * 8]) = stg[j];
        }
    };
    auto load_a = [&](int s, int j, vec8 *dst) {
        const int cc = c_begin + s / nkd, kd = kd_lo + s % nkd;
        const u16 *wb = a.wp + ((size_t)(cc * 27 + kd * 9 + j) * a.Mpad + mrow_lane) * 32 + kofs;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) dst[mb] = *reinterpret_cast<const vec8 *>(wb + mb * 16 * 32);
    };

    vec8 aq[PD][MB];
    if (nst > 0) {
        fetch(0);
        commit(0);
#pragma unroll
        for (int p = 0; p < PD; ++p) load_a(0, p, aq[p]);
    }
    __syncthreads();

    for (int s = 0; s < nst; ++s) {
        const int buf = s & 1;
        const bool more = s + 1 < nst;
        if (more) fetch(s + 1);
        const u16 *wsrc = win[buf];
#pragma unroll
        for (int j = 0; j < 9; ++j) {
            const int ky = j / 3, kx = j % 3;
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const int blk = wn * NBW + nb;
                const int r = blk / NBLK_ROW, c0 = (blk % NBLK_ROW) * 16;
                const vec8 B = *reinterpret_cast<const vec8 *>(
                    wsrc + ((r + ky) * WW + c0 + (lane & 15) + kx) * kPosStride + kofs);
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
        for (int mb = 0; mb < MB; ++mb)
            store_col<BF, EPI, SPLITK>(a, acc[mb][nb], pos, split, P,
                                       mt * BM + wm * MB * 16 + mb * 16 + 4 * (lane >> 4));
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
// Temporal (head kernels): 64-channel chunk c holds 3072 16-byte pieces in LDS order -- slot
// s = r*8 + q' of row r = kd*128 + m holds channels 64*c + 8*q .. +7, q = q' ^ head_lds_swizzle(r),
// of the weight for temporal tap kd and the (spatial tap, output channel) head_row_role(m) names.
// Rows past the real ones and channels past C_in are zero.
__global__ __launch_bounds__(256) void pack3d_kernel(const u16 *w, u16 *wp, int C_in, int C_out,
                                                     int NT, int Mpad, bool temporal,
                                                     long long total) {
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    u16 v = 0;
    if (!temporal) {
        const int k = (int)(idx & 31);
        long long r = idx >> 5;
        const int m = (int)(r % Mpad);
        r /= Mpad;
        const int tap = (int)(r % NT);
        const int cc = (int)(r / NT);
        const int ci = cc * 32 + k;
        if (ci < C_in && m < C_out) v = w[((size_t)m * C_in + ci) * 27 + tap];
    } else {
        const int cc = (int)(idx / (kHeadChunkPieces * 8));
        const int rem = (int)(idx - (long long)cc * (kHeadChunkPieces * 8));
        const int slot = rem >> 3, e = rem & 7;
        const int r = slot >> 3;
        const int q = (slot & 7) ^ head_lds_swizzle(r);
        const int kd = r >> 7, m = r & 127;
        const int ci = cc * 64 + 8 * q + e;
        int tap, co;
        head_row_role(m, tap, co);
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

template <bool BF>
hipError_t launch_igemm_dtype(const IgemmPlan &pl, const IgemmKArgs &ka, int epi, bool splitk,
                              hipStream_t s) {
    switch (pl.family) {
        case IG_WIDE:
            return launch_family<BF, 4, 4, 2, 2, 8, 16>(pl, ka, epi, splitk, s);
        case IG_NARROW:
            return launch_family<BF, 1, 4, 1, 4, 8, 32>(pl, ka, epi, splitk, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

IgemmPlan plan_igemm(int family, int N, int C_in, int C_out, int D, int H, int W) {
    IgemmPlan pl{};
    pl.family = family;
    switch (family) {
        case IG_WIDE:
            pl.BM = 128, pl.TH = 8, pl.TW = 16, pl.ntaps = 27;
            pl.Mrows = C_out;
            break;
        case IG_NARROW:
            pl.BM = 16, pl.TH = 8, pl.TW = 32, pl.ntaps = 27;
            pl.Mrows = C_out;
            break;
        default:   // the head kernels: 3 temporal taps x 128 rows (9 * C_out used)
            pl.BM = 128, pl.TH = 1, pl.TW = 256, pl.ntaps = 3;
            pl.Mrows = 128;
            break;
    }
    pl.Mpad = (pl.Mrows + pl.BM - 1) / pl.BM * pl.BM;
    pl.mtiles = pl.Mpad / pl.BM;
    // 32-channel chunks; the head kernels pack whole 64-channel chunks (an even count)
    pl.nchunks = family == IG_TEMPORAL ? (C_in + 63) / 64 * 2 : (C_in + 31) / 32;
    if (family == IG_TEMPORAL) {
        // 256 consecutive positions of one frame per workgroup (no spatial structure needed)
        pl.tiles_h = 1;
        pl.tiles_w = (int)(((long long)H * W + 255) / 256);
    } else {
        pl.tiles_h = (H + pl.TH - 1) / pl.TH;
        pl.tiles_w = (W + pl.TW - 1) / pl.TW;
    }
    const long long base = (long long)N * D * pl.tiles_h * pl.tiles_w * pl.mtiles;
    // Split K when the output alone cannot fill the 256 compute units a few times over.
    int splits = 1;
    if (family != IG_TEMPORAL && base > 0 && base < 1024) {
        splits = (int)((1024 + base - 1) / base);
        if (splits > pl.nchunks) splits = pl.nchunks;
    }
    pl.chunks_per_split = (pl.nchunks + splits - 1) / splits;
    pl.splits = (pl.nchunks + pl.chunks_per_split - 1) / pl.chunks_per_split;
    pl.workgroups = base * pl.splits;
    return pl;
}

size_t packed_bytes(const IgemmPlan &pl) {
    return (size_t)pl.nchunks * pl.ntaps * pl.Mpad * 32 * sizeof(u16);
}

size_t splitk_workspace_bytes(const IgemmPlan &pl, int N, int D, int H, int W, int C_out) {
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
    ka.N = p.N, ka.C_in = p.C_in, ka.D = p.D, ka.H = p.H, ka.W = p.W;
    ka.Mrows = pl.Mrows, ka.Mpad = pl.Mpad, ka.Cy = p.Cy;
    ka.nchunks = pl.nchunks, ka.chunks_per_split = pl.chunks_per_split, ka.splits = pl.splits;
    ka.tiles_h = pl.tiles_h, ka.tiles_w = pl.tiles_w, ka.mtiles = pl.mtiles;
    ka.total_wg = (uint32_t)pl.workgroups;
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
        pl.family == IG_TEMPORAL, total);
    return hipGetLastError();
}

}  // namespace cx
