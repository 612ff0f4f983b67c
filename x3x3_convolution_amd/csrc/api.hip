// The C ABI (include/conv3x3.h): argument validation, algorithm selection and dispatch to the
// gfx950 kernels.  Nothing is enqueued unless every check passes; errors carry a thread-local
// message (the role the TORCH_CHECK strings play in FastVideo head.cu's head_stencil wrapper).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "conv3x3.h"
#include "launch.hpp"

namespace {

thread_local char g_err[512];

int fail(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_err[0] = '\0';
    return CONV_OK;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

int device_present() {
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
        (void)hipGetLastError();  // clear the sticky "no device" error
        return fail(CONV_E_NODEVICE, "no HIP device is visible");
    }
    return CONV_OK;
}

int check_common(int stride, int layout, int dtype, int epilogue) {
    if (stride != 1 && stride != 2) return fail(CONV_E_INVAL, "stride must be 1 or 2 (got %d)", stride);
    if (layout != CONV_LAYOUT_CHANNELS_FIRST && layout != CONV_LAYOUT_CHANNELS_LAST)
        return fail(CONV_E_INVAL, "unknown layout %d", layout);
    if (dtype != CONV_DTYPE_F16 && dtype != CONV_DTYPE_BF16)
        return fail(CONV_E_INVAL, "unknown dtype %d", dtype);
    if (epilogue < CONV_EPI_NONE || epilogue > CONV_EPI_CLAMP1)
        return fail(CONV_E_INVAL, "unknown epilogue %d", epilogue);
    return CONV_OK;
}

// ---- 2D ------------------------------------------------------------------------------------
int check_2d(int N, int C_in, int C_out, int H, int W, int stride, int layout, int dtype,
             int epilogue, int algo) {
    int st = check_common(stride, layout, dtype, epilogue);
    if (st) return st;
    if (N < 0 || C_out < 0 || H < 0 || W < 0)
        return fail(CONV_E_INVAL, "negative size (N=%d C_out=%d H=%d W=%d)", N, C_out, H, W);
    if (C_in < 1) return fail(CONV_E_INVAL, "C_in must be >= 1 (got %d)", C_in);
    if (algo != CONV_ALGO_AUTO && algo != CONV_ALGO_SIMT && algo != CONV_ALGO_MFMA) {
        if (algo < CONV_ALGO_AUTO || algo > CONV_ALGO_FUSED_HEAD)
            return fail(CONV_E_INVAL, "unknown algo %d", algo);
        return fail(CONV_E_UNSUPPORTED, "2D convolution supports algo AUTO, SIMT or MFMA (got %d)", algo);
    }
    const bool nhwc = layout == CONV_LAYOUT_CHANNELS_LAST;
    if (nhwc && algo == CONV_ALGO_SIMT)
        return fail(CONV_E_UNSUPPORTED, "the SIMT 2D kernel supports the NCHW layout only");
    if (algo == CONV_ALGO_MFMA || nhwc) {
        if (!cx::mfma2d_supported(C_in, C_out, H, W, stride, nhwc))
            return fail(CONV_E_UNSUPPORTED,
                        nhwc ? "2D NHWC needs C_in a multiple of 8 up to 64 and C_out up to 64 "
                               "(got C_in=%d C_out=%d W=%d)"
                             : "2D MFMA needs C_in a multiple of 8 up to 64, C_out up to 64 and W a "
                               "multiple of 8 (got C_in=%d C_out=%d W=%d)", C_in, C_out, W);
        if ((long long)C_in * H * W * 2 >= (1ll << 31) ||
            (long long)C_out * ((H - 1) / stride + 1) * ((W - 1) / stride + 1) * 2 >= (1ll << 31))
            return fail(CONV_E_UNSUPPORTED, "2D MFMA needs one image of x and of y below 2 GiB");
    }
    const long long ho = (H - 1) / stride + 1, wo = (W - 1) / stride + 1;
    if ((long long)N * ((H + 31) / 32 + 1) * ((W + 31) / 32 + 1) * ((C_out + 15) / 16 + 1) >= (1ll << 31))
        return fail(CONV_E_UNSUPPORTED, "problem too large for one launch");
    (void)ho;
    (void)wo;
    return CONV_OK;
}

// The concrete 2D algorithm of a request that passed check_2d: MFMA when asked for or for NHWC
// (which only the matrix-core kernel takes), or for AUTO when the matrix-core kernel applies and
// its sample fits the 32-bit buffer ranges; else SIMT.
int select_2d(int C_in, int C_out, int H, int W, int stride, int layout, int algo) {
    if (algo == CONV_ALGO_MFMA || layout == CONV_LAYOUT_CHANNELS_LAST) return CONV_ALGO_MFMA;
    if (algo == CONV_ALGO_SIMT) return CONV_ALGO_SIMT;
    const bool fits = (long long)C_in * H * W * 2 < (1ll << 31) &&
                      (long long)C_out * ((H - 1) / stride + 1) * ((W - 1) / stride + 1) * 2 < (1ll << 31);
    return cx::mfma2d_supported(C_in, C_out, H, W, stride, false) && fits ? CONV_ALGO_MFMA
                                                                           : CONV_ALGO_SIMT;
}

// ---- 3D ------------------------------------------------------------------------------------
constexpr int kSplitHeadMaxCout = 12;  // 9 * C_out tap channels must fit the 112-channel plane

// The head kernels' buffer ranges: a workgroup reads six input frames of H_in rows and writes
// four output frames (at most 24 bytes per position: 12 channels, or the 12 RGB bytes).
bool head_frames_fit(long long H_in, long long W, long long C_in) {
    return 6 * H_in * W * C_in * 2 < (1ll << 31) && 4 * H_in * W * 24 < (1ll << 31);
}

int select_3d(int N, int C_in, int C_out, int D, int H, int W, int stride, int layout, int dtype,
              int algo) {
    int st = check_common(stride, layout, dtype, CONV_EPI_NONE);
    if (st) return st;
    if (N < 0 || C_out < 0 || D < 0 || H < 0 || W < 0)
        return fail(CONV_E_INVAL, "negative size (N=%d C_out=%d D=%d H=%d W=%d)", N, C_out, D, H, W);
    if (C_in < 1) return fail(CONV_E_INVAL, "C_in must be >= 1 (got %d)", C_in);
    if (algo < CONV_ALGO_AUTO || algo > CONV_ALGO_FUSED_HEAD)
        return fail(CONV_E_INVAL, "unknown algo %d", algo);
    if (layout != CONV_LAYOUT_CHANNELS_LAST)
        return fail(CONV_E_UNSUPPORTED, "3D convolution supports the NDHWC layout only");
    if (C_in % 8 != 0)
        return fail(CONV_E_UNSUPPORTED, "3D convolution needs C_in a multiple of 8 (got %d)", C_in);
    if (algo == CONV_ALGO_SIMT)
        return fail(CONV_E_UNSUPPORTED, "3D convolution has no SIMT algorithm");
    const bool head_algo = algo == CONV_ALGO_SPLIT_HEAD || algo == CONV_ALGO_FUSED_HEAD;
    if (stride == 2) {   // spatial stride 2 (the temporal stride stays 1): the MFMA path only
        if (head_algo)
            return fail(CONV_E_UNSUPPORTED, "the head algorithms support stride 1 only");
        if ((long long)H * W * C_in * 2 >= (1ll << 31))
            return fail(CONV_E_UNSUPPORTED, "3D stride 2 needs one input frame below 2 GiB");
        const long long pos = (long long)N * D * H * W;
        if (pos >= (1ll << 31) / 8 || (long long)C_out * 27 * C_in >= (1ll << 31))
            return fail(CONV_E_UNSUPPORTED, "problem too large for one launch");
        return CONV_ALGO_MFMA;
    }
    if (head_algo && C_out > kSplitHeadMaxCout)
        return fail(CONV_E_UNSUPPORTED, "the head algorithms need C_out <= %d (got %d)", kSplitHeadMaxCout, C_out);
    const long long pos = (long long)N * D * H * W;
    if (pos >= (1ll << 31) / 8 || (long long)C_out * 27 * C_in >= (1ll << 31))
        return fail(CONV_E_UNSUPPORTED, "problem too large for one launch");
    // the head kernels address a workgroup's six input frames and four output frames through
    // 32-bit buffer ranges (any number of frames)
    if (head_algo && !head_frames_fit(H, W, C_in))
        return fail(CONV_E_UNSUPPORTED, "the head algorithms need six input frames and four output "
                    "frames below 2 GiB (H=%d W=%d C_in=%d)", H, W, C_in);
    if (algo == CONV_ALGO_AUTO)
        return (C_out <= kSplitHeadMaxCout && head_frames_fit(H, W, C_in)) ? CONV_ALGO_FUSED_HEAD
                                                                          : CONV_ALGO_MFMA;
    return algo;
}

// The tile family of a request that passed select_3d (H, W: one input frame's extent).
int family_for(int algo, int C_in, int C_out, int H, int W, int stride) {
    if (algo == CONV_ALGO_SPLIT_HEAD) return cx::IG_TEMPORAL;
    if (algo == CONV_ALGO_FUSED_HEAD) return cx::IG_FUSED;
    if (stride == 2) return cx::IG_W32;
    // (the narrow kernel addresses a window of ten input rows through one 32-bit range)
    if (C_out <= 16 && 10LL * W * C_in * 2 < (1LL << 31)) return cx::IG_NARROW;
    return (long long)H * W * C_in * 2 < (1ll << 31) ? cx::IG_W32 : cx::IG_WIDE;
}

// Output extent of a pad-1, 3-tap dimension of a size that passed validation (0 stays 0).
int out_extent(int in, int stride) { return in > 0 ? (in - 1) / stride + 1 : 0; }

// The MFMA plan of a request given by its input extent (D, H, W) and stride.
cx::IgemmPlan plan_for(int a, int N, int C_in, int C_out, int D, int H, int W, int stride) {
    return cx::plan_igemm(family_for(a, C_in, C_out, H, W, stride), N, C_in, C_out, D,
                          out_extent(H, stride), out_extent(W, stride), stride);
}

size_t elem_bytes() { return 2; }

hipError_t launch_head(const void *x, const void *w_packed, const void *bias, void *out, int N,
                       int C_in, int C_out, int D, int H, int W, const cx::ConvRegion &rg, bool bf,
                       bool fused, int epilogue, hipStream_t s, bool rgb = false) {
    cx::HeadGemmParams hp{};
    hp.x = x, hp.wp = w_packed, hp.bias = bias, hp.out = out;
    hp.N = N, hp.C_in = C_in, hp.C_out = C_out, hp.D = D, hp.H = H, hp.W = W, hp.rg = rg;
    hp.bf16 = bf, hp.fused = fused, hp.epilogue = epilogue, hp.rgb = rgb;
    return cx::launch_head_gemm(hp, s);
}

hipError_t launch_stencil(const void *g, const void *bias, void *y, int N, int D, int H, int W,
                          int C_out, int g_off, bool bf, int epilogue, hipStream_t s) {
    cx::StencilParams sp{};
    sp.g = g, sp.bias = bias, sp.y = y;
    sp.N = N, sp.D = D, sp.H = H, sp.W = W, sp.C_out = C_out, sp.g_off = g_off;
    sp.bf16 = bf, sp.epilogue = epilogue;
    return cx::launch_head_stencil(sp, s);
}

}  // namespace

extern "C" {

int conv_abi_version(void) { return CONV_ABI_VERSION; }

const char *conv_status_str(int status) {
    switch (status) {
        case CONV_OK: return "ok";
        case CONV_E_INVAL: return "invalid argument";
        case CONV_E_UNSUPPORTED: return "unsupported request";
        case CONV_E_WORKSPACE: return "workspace missing or too small";
        case CONV_E_NODEVICE: return "no HIP device";
        case CONV_E_LAUNCH: return "kernel launch failed";
        default: return "unknown status";
    }
}

const char *conv_last_error(void) { return g_err; }

int conv_out_size(int in, int stride) {
    if (in < 0 || (stride != 1 && stride != 2)) return -1;
    if (in == 0) return 0;
    return (in - 1) / stride + 1;
}

int conv_band_region(int lo, int rows, int g_off, int H_global, int *H_in, int *h_org, int *h_lo,
                     int *h_hi) {
    if (!H_in || !h_org || !h_lo || !h_hi)
        return fail(CONV_E_INVAL, "H_in, h_org, h_lo and h_hi must be non-NULL");
    if (lo < 0 || rows < 0 || g_off < 0 || (long long)lo + rows > H_global)
        return fail(CONV_E_INVAL,
                    "a band needs lo >= 0, rows >= 0, g_off >= 0 and lo + rows <= H_global (got lo=%d "
                    "rows=%d g_off=%d H_global=%d)", lo, rows, g_off, H_global);
    if ((long long)rows + 2ll * g_off > 0x7FFFFFFF)
        return fail(CONV_E_INVAL, "rows + 2*g_off overflows an int");
    // input row r holds global row lo - g_off + r, which holds data when it lies in [0, H_global)
    const int hin = rows + 2 * g_off;
    const long long top = (long long)g_off - lo, bottom = (long long)H_global + g_off - lo;
    *H_in = hin;
    *h_org = g_off;
    *h_lo = top > 0 ? (int)top : 0;
    *h_hi = bottom < hin ? (int)bottom : hin;
    return ok();
}

int conv_causal_region(int D_out, int cached, int *D_in, int *d_org, int *d_lo, int *d_hi) {
    if (!D_in || !d_org || !d_lo || !d_hi)
        return fail(CONV_E_INVAL, "D_in, d_org, d_lo and d_hi must be non-NULL");
    if (D_out < 0 || cached < 0 || cached > 2 || D_out > 0x7FFFFFFF - 2)
        return fail(CONV_E_INVAL, "a causal chunk needs D_out >= 0 and 0 <= cached <= 2 (got D_out=%d "
                    "cached=%d)", D_out, cached);
    // output frame t of the chunk reads stored frames t + cached - 2 .. t + cached: the cached
    // frames first, zeros (frames before 0) where fewer than two are cached
    *D_in = D_out + cached;
    *d_org = cached - 1;
    *d_lo = 0;
    *d_hi = D_out + cached;
    return ok();
}

int conv3x3_is_supported(int N, int C_in, int C_out, int H, int W, int stride, int layout,
                         int dtype, int epilogue, int algo) {
    const int st = check_2d(N, C_in, C_out, H, W, stride, layout, dtype, epilogue, algo);
    return st ? st : ok();
}

int conv3x3_select_algo(int N, int C_in, int C_out, int H, int W, int stride, int layout,
                        int dtype, int algo) {
    const int st = check_2d(N, C_in, C_out, H, W, stride, layout, dtype, CONV_EPI_NONE, algo);
    if (st) return st;
    ok();
    return select_2d(C_in, C_out, H, W, stride, layout, algo);
}

int conv3x3_fwd(const void *x, const void *w, const void *bias, void *y, int N, int C_in,
                int C_out, int H, int W, int stride, int layout, int dtype, int epilogue,
                int algo, void *stream) {
    int st = check_2d(N, C_in, C_out, H, W, stride, layout, dtype, epilogue, algo);
    if (st) return st;
    if (N == 0 || C_out == 0 || H == 0 || W == 0) return ok();
    const int Ho = (H - 1) / stride + 1, Wo = (W - 1) / stride + 1;
    if (!x || !w || !y) return fail(CONV_E_INVAL, "x, w and y must be non-NULL");
    if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16))
        return fail(CONV_E_INVAL, "x, w and y must be 16-byte aligned");
    if (bias && !aligned(bias, 2)) return fail(CONV_E_INVAL, "bias must be 2-byte aligned");
    const size_t xb = (size_t)N * C_in * H * W * elem_bytes();
    const size_t yb = (size_t)N * C_out * Ho * Wo * elem_bytes();
    if (overlaps(x, xb, y, yb)) return fail(CONV_E_INVAL, "x and y overlap (in-place is unsupported)");
    if (overlaps(w, (size_t)C_out * C_in * 9 * elem_bytes(), y, yb))
        return fail(CONV_E_INVAL, "w and y overlap");
    if (bias && overlaps(bias, (size_t)C_out * elem_bytes(), y, yb))
        return fail(CONV_E_INVAL, "bias and y overlap");
    st = device_present();
    if (st) return st;
    cx::Simt2dParams p{};
    p.x = x, p.w = w, p.bias = bias, p.y = y;
    p.N = N, p.C_in = C_in, p.C_out = C_out, p.H = H, p.W = W, p.Hout = Ho, p.Wout = Wo;
    p.stride = stride, p.bf16 = dtype == CONV_DTYPE_BF16, p.epilogue = epilogue;
    p.nhwc = layout == CONV_LAYOUT_CHANNELS_LAST;
    if (select_2d(C_in, C_out, H, W, stride, layout, algo) == CONV_ALGO_MFMA) {
        const hipError_t e = cx::launch_mfma2d(p, (hipStream_t)stream);
        if (e != hipSuccess) return fail(CONV_E_LAUNCH, "MFMA 2D launch failed: %s", hipGetErrorString(e));
        return ok();
    }
    const hipError_t e = cx::launch_simt2d(p, (hipStream_t)stream);
    if (e != hipSuccess) return fail(CONV_E_LAUNCH, "SIMT 2D launch failed: %s", hipGetErrorString(e));
    return ok();
}

int conv3x3x3_select_algo(int N, int C_in, int C_out, int D, int H, int W, int stride,
                          int layout, int dtype, int algo) {
    const int a = select_3d(N, C_in, C_out, D, H, W, stride, layout, dtype, algo);
    if (a < 0) return a;
    ok();
    return a;
}

int conv3x3x3_is_supported(int N, int C_in, int C_out, int D, int H, int W, int stride,
                           int layout, int dtype, int epilogue, int algo) {
    if (epilogue < CONV_EPI_NONE || epilogue > CONV_EPI_CLAMP1)
        return fail(CONV_E_INVAL, "unknown epilogue %d", epilogue);
    const int a = select_3d(N, C_in, C_out, D, H, W, stride, layout, dtype, algo);
    return a < 0 ? a : ok();
}

size_t conv3x3x3_workspace_bytes(int N, int C_in, int C_out, int D, int H, int W, int stride,
                                 int layout, int dtype, int algo) {
    const int a = select_3d(N, C_in, C_out, D, H, W, stride, layout, dtype, algo);
    if (a < 0) return 0;
    ok();
    if (a == CONV_ALGO_SPLIT_HEAD)   // the plane, with room for one Z row above and below
        return (size_t)N * D * (H + 2) * W * cx::kHeadPlaneChannels * elem_bytes();
    const cx::IgemmPlan pl = plan_for(a, N, C_in, C_out, D, H, W, stride);
    return cx::splitk_workspace_bytes(pl, N, D, out_extent(H, stride), out_extent(W, stride), C_out);
}

size_t conv3x3x3_packed_weight_bytes(int N, int C_in, int C_out, int D, int H, int W,
                                     int stride, int layout, int dtype, int algo) {
    const int a = select_3d(N, C_in, C_out, D, H, W, stride, layout, dtype, algo);
    if (a < 0) return 0;
    ok();
    return cx::packed_bytes(plan_for(a, N, C_in, C_out, D, H, W, stride));
}

int conv3x3x3_describe(int N, int C_in, int C_out, int D, int H, int W, int stride, int layout,
                       int dtype, int algo, char *buf, int buf_len) {
    const int a = select_3d(N, C_in, C_out, D, H, W, stride, layout, dtype, algo);
    if (a < 0) return a;
    if (!buf || buf_len < 1) return fail(CONV_E_INVAL, "buf must be non-NULL with buf_len >= 1");
    char tmp[160];
    if (a == CONV_ALGO_SPLIT_HEAD || a == CONV_ALGO_FUSED_HEAD) {
        // the temporal GEMM's launch (the split head's plane holds the output rows: a plain
        // convolution's rows above and below read padding)
        const bool fused = a == CONV_ALGO_FUSED_HEAD;
        const cx::HeadRangePlan rp = cx::plan_head_ranges(N, D, H, W, fused);
        snprintf(tmp, sizeof tmp, "%s strips=%d frame_groups=%d row_ranges=%d z_rows=%d workgroups=%lld",
                 fused ? "fused_head" : "split_head", rp.strips, rp.fgroups, rp.ranges,
                 rp.max_z_rows, rp.workgroups);
    } else {
        const cx::IgemmPlan pl = plan_for(a, N, C_in, C_out, D, H, W, stride);
        const char *k = pl.family == cx::IG_W32 ? (pl.kq ? "igemm32_kq" : pl.sk ? "igemm32_sk" : "igemm32")
                        : pl.family == cx::IG_WIDE ? "igemm16_wide" : "igemm16_narrow";
        snprintf(tmp, sizeof tmp, "%s tile=%dx%d rows=%d splits=%d workgroups=%lld", k, pl.TH,
                 pl.TW, pl.kq ? 64 : pl.BM, pl.splits, pl.workgroups);
    }
    snprintf(buf, (size_t)buf_len, "%s", tmp);
    ok();
    return (int)strlen(tmp);
}

int conv3x3x3_pack_weights(const void *w_oidhw, void *w_packed, int N, int C_in, int C_out,
                           int D, int H, int W, int stride, int layout, int dtype, int algo,
                           void *stream) {
    const int a = select_3d(N, C_in, C_out, D, H, W, stride, layout, dtype, algo);
    if (a < 0) return a;
    if (C_out == 0) return ok();
    if (!w_oidhw || !w_packed) return fail(CONV_E_INVAL, "w_oidhw and w_packed must be non-NULL");
    if (!aligned(w_oidhw, 2) || !aligned(w_packed, 16))
        return fail(CONV_E_INVAL, "w_oidhw must be 2-byte and w_packed 16-byte aligned");
    const cx::IgemmPlan pl = plan_for(a, N, C_in, C_out, D, H, W, stride);
    if (overlaps(w_oidhw, (size_t)C_out * C_in * 27 * elem_bytes(), w_packed, cx::packed_bytes(pl)))
        return fail(CONV_E_INVAL, "w_oidhw and w_packed overlap");
    int st = device_present();
    if (st) return st;
    const hipError_t e = cx::launch_pack3d(pl, w_oidhw, w_packed, C_in, C_out, (hipStream_t)stream);
    if (e != hipSuccess) return fail(CONV_E_LAUNCH, "weight pack launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"

namespace {

// The forward pass of the 3D convolution over an input region (the full region for the plain
// convolution).  D, H, W are the output extent, W_in the input width; at stride 2 (plain
// convolution only) output row oh reads input rows 2*oh - 1 .. 2*oh + 1, column ow input columns
// 2*ow - 1 .. 2*ow + 1.  Algorithm, packing and workspace follow from the request as the caller
// states it to the size queries: the input extent and the stride.
int fwd3d(const void *x, const void *w_packed, const void *bias, void *y, int N, int C_in,
          int C_out, int D, int H, int W, int W_in, const cx::ConvRegion &rg, int stride,
          int layout, int dtype, int epilogue, int algo, void *workspace, size_t workspace_bytes,
          void *stream) {
    if (epilogue < CONV_EPI_NONE || epilogue > CONV_EPI_CLAMP1)
        return fail(CONV_E_INVAL, "unknown epilogue %d", epilogue);
    // the request as the size queries see it: input extent (region calls: output extent)
    const int Hq = stride == 1 ? H : rg.H_in, Wq = W_in;
    const int a = select_3d(N, C_in, C_out, D, Hq, Wq, stride, layout, dtype, algo);
    if (a < 0) return a;
    if (rg.D_in < 0 || rg.H_in < 0)
        return fail(CONV_E_INVAL, "negative input extent (D_in=%d H_in=%d)", rg.D_in, rg.H_in);
    if (rg.d_lo < 0 || rg.d_lo > rg.d_hi || rg.d_hi > rg.D_in || rg.h_lo < 0 || rg.h_lo > rg.h_hi ||
        rg.h_hi > rg.H_in)
        return fail(CONV_E_INVAL,
                    "valid ranges must lie inside the input: 0 <= d_lo <= d_hi <= D_in and "
                    "0 <= h_lo <= h_hi <= H_in (got d %d..%d of %d, h %d..%d of %d)",
                    rg.d_lo, rg.d_hi, rg.D_in, rg.h_lo, rg.h_hi, rg.H_in);
    if (N == 0 || C_out == 0 || D == 0 || H == 0 || W == 0) return ok();
    // output frame od reads input frames od + d_org - 1 .. od + d_org + 1
    if (rg.d_lo >= rg.d_hi || rg.d_lo > rg.d_org + 1 || (long long)D + rg.d_org - 1 > rg.d_hi)
        return fail(CONV_E_UNSUPPORTED,
                    "every output frame must read at least one valid input frame (d_org=%d, valid "
                    "frames %d..%d, D_out=%d)", rg.d_org, rg.d_lo, rg.d_hi, D);
    const long long frame_in = (long long)rg.H_in * W_in * C_in * 2;
    if ((long long)N * rg.D_in * rg.H_in * W_in >= (1ll << 31) / 8)
        return fail(CONV_E_UNSUPPORTED, "input too large for one launch");
    const bool head_algo = a == CONV_ALGO_SPLIT_HEAD || a == CONV_ALGO_FUSED_HEAD;
    if (head_algo && !head_frames_fit(rg.H_in, W_in, C_in))
        return fail(CONV_E_UNSUPPORTED, "the head algorithms need six input frames below 2 GiB "
                    "(H_in=%d W=%d C_in=%d)", rg.H_in, W_in, C_in);
    const int family = family_for(a, C_in, C_out, Hq, Wq, stride);
    if (family == cx::IG_W32 && frame_in >= (1ll << 31))
        return fail(CONV_E_UNSUPPORTED, "one input frame must stay below 2 GiB for this packing");
    // the split head's plane: the output rows alone when the Z rows next to them read no data
    // (the stencil takes those as zero), else one more Z row above and below (g_off = 1)
    const bool row_edges_zero = (rg.h_org - 1 < rg.h_lo || rg.h_org - 1 >= rg.h_hi) &&
                                ((long long)H + rg.h_org < rg.h_lo || (long long)H + rg.h_org >= rg.h_hi);
    const int g_off = row_edges_zero ? 0 : 1;
    if (!x || !w_packed || !y) return fail(CONV_E_INVAL, "x, w_packed and y must be non-NULL");
    if (!aligned(x, 16) || !aligned(w_packed, 16) || !aligned(y, 16))
        return fail(CONV_E_INVAL, "x, w_packed and y must be 16-byte aligned");
    if (bias && !aligned(bias, 2)) return fail(CONV_E_INVAL, "bias must be 2-byte aligned");
    const size_t P = (size_t)N * D * H * W;
    const size_t xb = (size_t)N * rg.D_in * rg.H_in * W_in * C_in * elem_bytes();
    const size_t yb = P * C_out * elem_bytes();
    if (overlaps(x, xb, y, yb)) return fail(CONV_E_INVAL, "x and y overlap (in-place is unsupported)");
    const size_t need = conv3x3x3_workspace_bytes(N, C_in, C_out, D, Hq, Wq, stride, layout, dtype, a);
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(CONV_E_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                        workspace ? workspace_bytes : (size_t)0);
        if (!aligned(workspace, 16)) return fail(CONV_E_INVAL, "workspace must be 16-byte aligned");
        if (overlaps(workspace, need, x, xb) || overlaps(workspace, need, y, yb))
            return fail(CONV_E_INVAL, "workspace overlaps x or y");
    }
    int st = device_present();
    if (st) return st;
    const bool bf = dtype == CONV_DTYPE_BF16;
    hipStream_t s = (hipStream_t)stream;
    if (a == CONV_ALGO_SPLIT_HEAD) {
        cx::ConvRegion prg = rg;      // plane row z holds the Z row of output row z - g_off
        prg.h_org -= g_off;
        hipError_t e = launch_head(x, w_packed, nullptr, workspace, N, C_in, C_out, D, H + 2 * g_off,
                                   W, prg, bf, false, CONV_EPI_NONE, s);
        if (e != hipSuccess) return fail(CONV_E_LAUNCH, "split-head temporal launch failed: %s", hipGetErrorString(e));
        e = launch_stencil(workspace, bias, y, N, D, H, W, C_out, g_off, bf, epilogue, s);
        if (e != hipSuccess) return fail(CONV_E_LAUNCH, "split-head stencil launch failed: %s", hipGetErrorString(e));
        return ok();
    }
    if (a == CONV_ALGO_FUSED_HEAD) {
        const hipError_t e = launch_head(x, w_packed, bias, y, N, C_in, C_out, D, H, W, rg, bf, true,
                                         epilogue, s);
        if (e != hipSuccess) return fail(CONV_E_LAUNCH, "fused head launch failed: %s", hipGetErrorString(e));
        return ok();
    }
    const cx::IgemmPlan pl = cx::plan_igemm(family, N, C_in, C_out, D, H, W, stride);
    cx::IgemmParams ip{};
    ip.x = x, ip.wp = w_packed, ip.bias = bias, ip.y = y;
    ip.partial = static_cast<float *>(pl.splits > 1 || pl.sk ? workspace : nullptr);
    ip.N = N, ip.C_in = C_in, ip.D = D, ip.H = H, ip.W = W, ip.W_in = W_in, ip.rg = rg;
    ip.Cy = C_out, ip.bf16 = bf, ip.epilogue = epilogue;
    const hipError_t e = cx::launch_igemm3d(pl, ip, s);
    if (e != hipSuccess) return fail(CONV_E_LAUNCH, "MFMA 3D launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

int conv3x3x3_fwd(const void *x, const void *w_packed, const void *bias, void *y, int N,
                  int C_in, int C_out, int D, int H, int W, int stride, int layout, int dtype,
                  int epilogue, int algo, void *workspace, size_t workspace_bytes, void *stream) {
    // the output extent; the input region is the whole input
    const int Ho = stride == 2 ? out_extent(H, 2) : H, Wo = stride == 2 ? out_extent(W, 2) : W;
    return fwd3d(x, w_packed, bias, y, N, C_in, C_out, D, Ho, Wo, W, cx::full_region(D, H), stride,
                 layout, dtype, epilogue, algo, workspace, workspace_bytes, stream);
}

int conv3x3x3_fwd_region(const void *x, const void *w_packed, const void *bias, void *y, int N,
                         int C_in, int C_out, int D_in, int H_in, int W, int D_out, int H_out,
                         int d_org, int h_org, int d_lo, int d_hi, int h_lo, int h_hi, int layout,
                         int dtype, int epilogue, int algo, void *workspace,
                         size_t workspace_bytes, void *stream) {
    return fwd3d(x, w_packed, bias, y, N, C_in, C_out, D_out, H_out, W, W,
                 cx::ConvRegion{D_in, H_in, d_org, h_org, d_lo, d_hi, h_lo, h_hi}, 1, layout, dtype,
                 epilogue, algo, workspace, workspace_bytes, stream);
}

int conv_head_temporal(const void *x, const void *w_packed, void *g, int N, int C_in, int C_out,
                       int D, int H, int W, int dtype, void *stream) {
    const int a = select_3d(N, C_in, C_out, D, H, W, 1, CONV_LAYOUT_CHANNELS_LAST, dtype,
                            CONV_ALGO_SPLIT_HEAD);
    if (a < 0) return a;
    if (N == 0 || C_out == 0 || D == 0 || H == 0 || W == 0) return ok();
    if (!x || !w_packed || !g) return fail(CONV_E_INVAL, "x, w_packed and g must be non-NULL");
    if (!aligned(x, 16) || !aligned(w_packed, 16) || !aligned(g, 16))
        return fail(CONV_E_INVAL, "x, w_packed and g must be 16-byte aligned");
    const size_t P = (size_t)N * D * H * W;
    if (overlaps(x, P * C_in * elem_bytes(), g, P * cx::kHeadPlaneChannels * elem_bytes()))
        return fail(CONV_E_INVAL, "x and g overlap");
    int st = device_present();
    if (st) return st;
    const hipError_t e = launch_head(x, w_packed, nullptr, g, N, C_in, C_out, D, H, W,
                                     cx::full_region(D, H), dtype == CONV_DTYPE_BF16, false,
                                     CONV_EPI_NONE, (hipStream_t)stream);
    if (e != hipSuccess) return fail(CONV_E_LAUNCH, "head temporal launch failed: %s", hipGetErrorString(e));
    return ok();
}

int conv_head_stencil(const void *g, const void *bias, void *y, int N, int D, int H, int W,
                      int C_out, int dtype, int epilogue, void *stream) {
    int st = check_common(1, CONV_LAYOUT_CHANNELS_LAST, dtype, epilogue);
    if (st) return st;
    if (N < 0 || D < 0 || H < 0 || W < 0 || C_out < 0)
        return fail(CONV_E_INVAL, "negative size (N=%d D=%d H=%d W=%d C_out=%d)", N, D, H, W, C_out);
    if (C_out > kSplitHeadMaxCout)
        return fail(CONV_E_UNSUPPORTED, "the head stencil needs C_out <= %d (got %d)", kSplitHeadMaxCout, C_out);
    const long long pos = (long long)N * D * H * W;
    if (pos >= (1ll << 31) / 8) return fail(CONV_E_UNSUPPORTED, "problem too large for one launch");
    if (pos == 0 || C_out == 0) return ok();
    if (!g || !y) return fail(CONV_E_INVAL, "g and y must be non-NULL");
    if (!aligned(g, 16) || !aligned(y, 16)) return fail(CONV_E_INVAL, "g and y must be 16-byte aligned");
    if (bias && !aligned(bias, 2)) return fail(CONV_E_INVAL, "bias must be 2-byte aligned");
    if (overlaps(g, (size_t)pos * cx::kHeadPlaneChannels * elem_bytes(), y, (size_t)pos * C_out * elem_bytes()))
        return fail(CONV_E_INVAL, "g and y overlap");
    st = device_present();
    if (st) return st;
    const hipError_t e = launch_stencil(g, bias, y, N, D, H, W, C_out, 0, dtype == CONV_DTYPE_BF16,
                                        epilogue, (hipStream_t)stream);
    if (e != hipSuccess) return fail(CONV_E_LAUNCH, "head stencil launch failed: %s", hipGetErrorString(e));
    return ok();
}

int conv_video_rgb8(const void *y, void *rgb, int N, int D, int H, int W, int C, int dtype,
                    void *stream) {
    int st = check_common(1, CONV_LAYOUT_CHANNELS_LAST, dtype, CONV_EPI_NONE);
    if (st) return st;
    if (N < 0 || D < 0 || H < 0 || W < 0)
        return fail(CONV_E_INVAL, "negative size (N=%d D=%d H=%d W=%d)", N, D, H, W);
    if (C != 12)
        return fail(CONV_E_UNSUPPORTED, "the video step takes 12 channels (3 colours x 2 x 2), got %d", C);
    const long long pos = (long long)N * D * H * W;
    if (pos == 0) return ok();
    if ((long long)N * D * H * ((W + 255) / 256) >= (1ll << 31) || pos >= (1ll << 40))
        return fail(CONV_E_UNSUPPORTED, "problem too large for one launch");
    if (!y || !rgb) return fail(CONV_E_INVAL, "y and rgb must be non-NULL");
    if (!aligned(y, 16)) return fail(CONV_E_INVAL, "y must be 16-byte aligned");
    if (overlaps(y, (size_t)pos * 12 * elem_bytes(), rgb, (size_t)pos * 12))
        return fail(CONV_E_INVAL, "y and rgb overlap");
    st = device_present();
    if (st) return st;
    cx::VideoParams vp{};
    vp.y = y, vp.rgb = rgb, vp.N = N, vp.D = D, vp.H = H, vp.W = W;
    vp.bf16 = dtype == CONV_DTYPE_BF16;
    const hipError_t e = cx::launch_video_rgb8(vp, (hipStream_t)stream);
    if (e != hipSuccess) return fail(CONV_E_LAUNCH, "video launch failed: %s", hipGetErrorString(e));
    return ok();
}

int conv3x3x3_head_rgb8(const void *x, const void *w_packed, const void *bias, void *rgb, int N,
                        int C_in, int D, int H, int W, int dtype, int epilogue, void *stream) {
    if (epilogue < CONV_EPI_NONE || epilogue > CONV_EPI_CLAMP1)
        return fail(CONV_E_INVAL, "unknown epilogue %d", epilogue);
    const int a = select_3d(N, C_in, 12, D, H, W, 1, CONV_LAYOUT_CHANNELS_LAST, dtype,
                            CONV_ALGO_FUSED_HEAD);
    if (a < 0) return a;
    if (N == 0 || D == 0 || H == 0 || W == 0) return ok();
    const size_t rgb_sample = (size_t)D * H * W * 12;
    if (!x || !w_packed || !rgb) return fail(CONV_E_INVAL, "x, w_packed and rgb must be non-NULL");
    if (!aligned(x, 16) || !aligned(w_packed, 16) || !aligned(rgb, 2))
        return fail(CONV_E_INVAL, "x and w_packed must be 16-byte and rgb 2-byte aligned");
    if (bias && !aligned(bias, 2)) return fail(CONV_E_INVAL, "bias must be 2-byte aligned");
    const size_t xb = (size_t)N * D * H * W * C_in * elem_bytes();
    if (overlaps(x, xb, rgb, (size_t)N * rgb_sample)) return fail(CONV_E_INVAL, "x and rgb overlap");
    int st = device_present();
    if (st) return st;
    const hipError_t e = launch_head(x, w_packed, bias, rgb, N, C_in, 12, D, H, W,
                                     cx::full_region(D, H), dtype == CONV_DTYPE_BF16, true,
                                     epilogue, (hipStream_t)stream, true);
    if (e != hipSuccess) return fail(CONV_E_LAUNCH, "RGB head launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"

// ---- allocation-free forward pass -------------------------------------------------------------
// A static device array serves as the workspace of conv3x3x3_fwd_noalloc, so that callers that
// cannot allocate (graph capture, serving loops) still reach the algorithms that need one (the
// MFMA path's split-K partial sums and its stream-K partial tiles and arrival counters, which a
// kernel clears at every call; the split head's plane when it fits).  Each GPU the
// library runs on holds its own copy of the array until the process ends.  In host code the
// array's name is only a stand-in: its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and only that address is passed to kernels.
namespace cx {
__device__ __align__(256) unsigned char scratch[CONV_NOALLOC_SCRATCH_BYTES];
}  // namespace cx

namespace {

constexpr size_t kScratchBytes = (size_t)CONV_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device, once looked up

// The scratch array's device address on the current device (nullptr and a message on failure).
void *scratch_on_current_device(int *status) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        *status = fail(CONV_E_NODEVICE, "no current HIP device for the static scratch");
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(cx::scratch));
        if (e != hipSuccess || !ptr) {
            (void)hipGetLastError();
            *status = fail(CONV_E_LAUNCH, "looking up the static scratch on device %d failed: %s", dev,
                           hipGetErrorString(e));
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    *status = CONV_OK;
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int conv3x3x3_fwd_noalloc(const void *x, const void *w_packed, const void *bias, void *y,
                                     int N, int C_in, int C_out, int D, int H, int W, int stride,
                                     int layout, int dtype, int epilogue, int algo, void *stream) {
    // the request's workspace, checked against the array before anything else touches a device
    const int a = select_3d(N, C_in, C_out, D, H, W, stride, layout, dtype, algo);
    if (a < 0) return a;
    const size_t need = conv3x3x3_workspace_bytes(N, C_in, C_out, D, H, W, stride, layout, dtype, a);
    if (need > kScratchBytes)
        return fail(CONV_E_WORKSPACE,
                    "this request needs %zu bytes of workspace; the static scratch of the "
                    "allocation-free entry point holds %zu (use conv3x3x3_fwd with a workspace, or "
                    "an algorithm that needs less)", need, kScratchBytes);
    void *ws = nullptr;
    if (need > 0) {
        int st = device_present();
        if (st) return st;
        ws = scratch_on_current_device(&st);
        if (!ws) return st;
    }
    return conv3x3x3_fwd(x, w_packed, bias, y, N, C_in, C_out, D, H, W, stride, layout, dtype,
                         epilogue, a, ws, ws ? kScratchBytes : 0, stream);
}
