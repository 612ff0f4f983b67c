/*
 * conv3x3.h -- C ABI of the MI355X (gfx950) pad-1 3x3 / 3x3x3 convolution library.
 *
 * The operation (cited by page title and section):
 *   2D  [musetalk-bench patches/taesd_conv.cuh.new, header comment and taesd_conv3x3_impl]:
 *       y[n,co,oh,ow] = E( b[co] + sum_{ci,ky,kx} w[co,ci,ky,kx] * X[n,ci, s*oh-1+ky, s*ow-1+kx] )
 *   3D  [FastVideo fastvideo-kernel/wan22_vae_decode/solution/head.cu, header comment: the
 *       27-tap output convolution]:
 *       y[n,co,d,oh,ow] = E( b[co] + sum_{ci,kd,ky,kx} w[co,ci,kd,ky,kx]
 *                                        * X[n,ci, d-1+kd, s*oh-1+ky, s*ow-1+kx] )
 *   X is zero outside the tensor (pad 1 in every convolved dimension; one zero frame at each
 *   temporal end, so D_out = D).  Cross-correlation (no kernel flip).  H_out = (H-1)/s + 1 and
 *   W_out likewise (integer division).  b = 0 when bias is NULL.  E is the fused epilogue:
 *   identity, ReLU (v < 0 ? 0 : v) or clamp to [-1, 1].  Inputs, weights, bias and outputs are
 *   fp16 or bf16; products are accumulated in fp32 and rounded once, to nearest-even, on the
 *   store -- except the split head (CONV_ALGO_SPLIT_HEAD), which rounds the 3x1x1 temporal
 *   partial sums to the activation dtype once in its intermediate plane, as the head.cu page
 *   describes for its value path.
 *
 * Conventions
 *   - Every pointer is a device pointer the caller allocated (the library allocates no device
 *     memory and keeps no per-call state; calls are thread-safe).  x, w/w_packed, y and the
 *     workspace must be 16-byte aligned; bias 2-byte aligned.  x and y must not overlap.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Work is enqueued
 *     on it and the call returns without synchronising.  Multi-launch algorithms order their
 *     launches on that stream.  A workspace holds one call's intermediate state (plane,
 *     partial sums, stream-K arrival counters) while that call runs: calls that may run at the
 *     same time (on different streams) need workspaces of their own.
 *   - All argument checks happen before anything is enqueued; on error nothing is launched
 *     and conv_last_error() returns a message.  A kernel fault surfaces at the caller's next
 *     synchronisation, as with any HIP launch.
 *   - An empty output (N, C_out, D, H or W equal to 0) is a no-op that returns CONV_OK.
 */
#ifndef CONV3X3_H_
#define CONV3X3_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CONV_ABI_VERSION 1

/* storage dtypes */
enum { CONV_DTYPE_F16 = 0, CONV_DTYPE_BF16 = 1 };
/* layouts: 2D channels-first = NCHW, channels-last = NHWC;
 *          3D channels-first = NCDHW, channels-last = NDHWC */
enum { CONV_LAYOUT_CHANNELS_FIRST = 0, CONV_LAYOUT_CHANNELS_LAST = 1 };
/* fused epilogues (applied after the bias) */
enum { CONV_EPI_NONE = 0, CONV_EPI_RELU = 1, CONV_EPI_CLAMP1 = 2 };
/* algorithms.  AUTO resolves deterministically from the shape (conv3x3_select_algo,
 * conv3x3x3_select_algo).
 *   SIMT        2D: direct LDS-halo kernel on the vector ALUs (fp32 accumulation via dot2).
 *   MFMA        2D: the same sum on the matrix cores (9 taps x C_in in one fp32 accumulator)
 *               for C_in a multiple of 8 up to 64, C_out up to 64, W a multiple of 8 [the
 *               contraction the taesd_conv.cuh.new header comment defines; the matrix-core route
 *               its rationale argues against, measured here].  AUTO picks it when it applies.
 *               3D: implicit GEMM on the matrix cores, 27 taps in one fp32 accumulator.
 *   SPLIT_HEAD  3D, C_out <= 12, stride 1: 3x1x1 temporal conv into 9*C_out tap channels of a
 *               112-channel bf16/fp16 plane in the workspace, then a nine-tap stencil + bias +
 *               epilogue [head.cu, header comment and head_stencil_kernel].
 *   FUSED_HEAD  3D, C_out <= 12, stride 1: the same temporal GEMM as SPLIT_HEAD, but its tap
 *               sums stay in the matrix cores' fp32 accumulator registers and the stencil + bias
 *               + epilogue run in the same kernel: the 27 taps reach the output in fp32 and are
 *               rounded once, on the store (like MFMA; only SPLIT_HEAD rounds the plane), and
 *               the plane never goes to HBM; no workspace.  [head.cu, header comment: the split
 *               of the 27-tap conv; its value path places the first rounding after the three
 *               temporal taps, which this fused form leaves out.]
 *   AUTO: 2D: MFMA when it applies, else SIMT.  3D: FUSED_HEAD when C_out <= 12, stride 1 and
 *   the head's frame windows fit (see conv3x3x3_fwd), else MFMA.  [taesd_conv.cuh.new header comment: direct kernels for the C <= 64 layers;
 *   head.cu header comment: the split form for the 12-channel head.] */
enum {
    CONV_ALGO_AUTO = 0,
    CONV_ALGO_SIMT = 1,
    CONV_ALGO_MFMA = 2,
    CONV_ALGO_SPLIT_HEAD = 3,
    CONV_ALGO_FUSED_HEAD = 4
};
/* status codes */
enum {
    CONV_OK = 0,
    CONV_E_INVAL = -1,       /* bad pointer, size, enum, alignment or overlap */
    CONV_E_UNSUPPORTED = -2, /* valid request this library does not implement */
    CONV_E_WORKSPACE = -3,   /* workspace missing or smaller than the query returned */
    CONV_E_NODEVICE = -4,    /* no HIP device visible */
    CONV_E_LAUNCH = -5       /* the HIP runtime rejected a launch */
};

/* ABI version of the loaded library (CONV_ABI_VERSION it was built with).  Library plumbing: no
 * page defines it. */
int conv_abi_version(void);

/* Static text for a status code.  [head.cu, head_stencil host function: every argument check
 * fails with a message, and a rejected launch is reported after the launch.]  The pointer is to
 * static storage; the caller never frees it. */
const char *conv_status_str(int status);

/* Detail of the last error on the calling thread ("" after a successful call), the message the
 * failed check wrote [head.cu, head_stencil host function: the checks' messages].  Thread-local
 * storage owned by the library, valid until the thread's next call. */
const char *conv_last_error(void);

/* Output extent of a pad-1, 3-tap dimension: (in-1)/stride + 1 for in >= 1; 0 for in == 0;
 * -1 for a negative size or a stride outside {1, 2}.  [taesd_conv.cuh.new, taesd_conv3x3_impl:
 * the window of output oh starts at input row oh*stride - 1, so the last output whose window
 * still starts inside the padded input is (in-1)/stride; the extern "C" wrappers take H_out and
 * W_out from the caller.] */
int conv_out_size(int in, int stride);

/* ------------------------------------------------------------------------------------------
 * Region fields of the row bands and causal chunks of conv3x3x3_fwd_region (pure host
 * arithmetic, no device work; for callers that shard rows or decode in chunks).
 *
 * conv_band_region: output rows [lo, lo + rows) of a frame of global height H_global, computed
 * from an input tensor that holds global rows lo - g_off .. lo + rows + g_off - 1 (rows outside
 * [0, H_global) may hold anything: they are never read).  [head.cu, head_stencil host function:
 * an output band [lo, lo + rows) whose input carries g_off extra rows on each side, zero padding
 * decided against the global height H_global, buffer bounds against the band.]  Writes
 *   *H_in = rows + 2*g_off,  *h_org = g_off,
 *   *h_lo = max(0, g_off - lo),  *h_hi = min(rows + 2*g_off, H_global + g_off - lo),
 * the fields to pass to conv3x3x3_fwd_region with H_out = rows.  With g_off >= 1 the band's
 * output equals rows [lo, lo + rows) of the convolution of the whole frame.  Returns CONV_OK, or
 * CONV_E_INVAL (nothing written) for a NULL output pointer, lo < 0, rows < 0, g_off < 0 or
 * lo + rows > H_global.
 *
 * conv_causal_region: a chunk of D_out new frames of a causal pass (output frame t reads input
 * frames t-2 .. t, zeros before the first frame of the video), with `cached` (0, 1 or 2) frames
 * of the previous chunk stored in front of the new ones in x.  [head.cu, commit summary: the
 * decoder carries a few latent frames per pass to bound its memory.]  Writes
 *   *D_in = D_out + cached,  *d_org = cached - 1,  *d_lo = 0,  *d_hi = D_out + cached.
 * Returns CONV_OK, or CONV_E_INVAL (nothing written) for a NULL output pointer, D_out < 0 or
 * cached outside 0..2.
 * ---------------------------------------------------------------------------------------- */
int conv_band_region(int lo, int rows, int g_off, int H_global, int *H_in, int *h_org, int *h_lo,
                     int *h_hi);
int conv_causal_region(int D_out, int cached, int *D_in, int *d_org, int *d_lo, int *d_hi);

/* ------------------------------------------------------------------------------------------
 * 2D: x (N,C_in,H,W) NCHW, w (C_out,C_in,3,3) OIHW as stored by PyTorch (no packing), bias
 * (C_out) or NULL, y (N,C_out,H_out,W_out) NCHW; all of `dtype`.  stride 1 or 2.
 * layout CHANNELS_LAST: x (N,H,W,C_in) and y (N,H_out,W_out,C_out) NHWC, same w and bias.
 * Supported: dtype F16 or BF16.  NCHW: algo SIMT: any C_in/C_out >= 1; algo MFMA: C_in % 8 ==
 * 0, C_in <= 64, C_out <= 64, W % 8 == 0, one image of x and of y below 2 GiB (else
 * CONV_E_UNSUPPORTED); AUTO: MFMA when it applies, else SIMT.  NHWC: MFMA only (AUTO selects
 * it), C_in % 8 == 0, C_in <= 64, C_out <= 64, any W, one image of x and of y below 2 GiB.
 * [taesd_conv.cuh.new: operator contract in the header comment; the kernels' argument lists]
 * ---------------------------------------------------------------------------------------- */
int conv3x3_fwd(const void *x, const void *w, const void *bias, void *y, int N, int C_in,
                int C_out, int H, int W, int stride, int layout, int dtype, int epilogue,
                int algo, void *stream);

/* CONV_OK if conv3x3_fwd would accept this request (pointers aside), else the status it
 * would return.  Host-only, no device work.  [head.cu, commit summary: the ranks agree on whether
 * every one of them could build the kernel before they take its path; this query is what each
 * of them would contribute to that agreement.] */
int conv3x3_is_supported(int N, int C_in, int C_out, int H, int W, int stride, int layout,
                         int dtype, int epilogue, int algo);

/* The concrete 2D algorithm (CONV_ALGO_SIMT or CONV_ALGO_MFMA) conv3x3_fwd runs for this
 * request, or a negative status if it would reject it.  [taesd_conv.cuh.new, header comment:
 * which kernel serves the C <= 64 layers.] */
int conv3x3_select_algo(int N, int C_in, int C_out, int H, int W, int stride, int layout,
                        int dtype, int algo);

/* ------------------------------------------------------------------------------------------
 * 3D: x (N,D,H,W,C_in) NDHWC, w_packed from conv3x3x3_pack_weights, bias (C_out) or NULL,
 * y (N,D,H_out,W_out,C_out) NDHWC.  Supported: layout CHANNELS_LAST, dtype BF16 or F16,
 * C_in a multiple of 8, stride 1 or 2.  Stride 2 is spatial: H_out = (H-1)/2+1, W_out likewise,
 * output (d, oh, ow) reads input rows 2*oh-1+ky and columns 2*ow-1+kx, the D frames keep stride
 * 1 (the oracle's reading of a strided 3x3x3 video convolution); it runs on algo MFMA only
 * (AUTO selects it) and needs one input frame below 2 GiB.
 *   algo MFMA: any C_out >= 1.  algo SPLIT_HEAD / FUSED_HEAD: C_out <= 12, stride 1, any number
 *   of frames; a workgroup's six input frames (6*H*W*C_in elements) and four output frames
 *   (4*H*W*12 elements) each below 2 GiB.  AUTO: see select_algo.
 * workspace: at least conv3x3x3_workspace_bytes(...) bytes (may be NULL when that is 0).
 * The same (shape, dtype, algo) arguments must be given to the size queries, to
 * conv3x3x3_pack_weights and to conv3x3x3_fwd.
 * ---------------------------------------------------------------------------------------- */
int conv3x3x3_fwd(const void *x, const void *w_packed, const void *bias, void *y, int N,
                  int C_in, int C_out, int D, int H, int W, int stride, int layout, int dtype,
                  int epilogue, int algo, void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------------------------
 * 3D over an input region: row bands with halo rows, frame chunks and causal temporal padding.
 * [head.cu, head_stencil: an output band of rows [lo, lo+rows) of a global height, its input
 * carrying g_off extra rows each side, zero padding decided by the global height; head.cu,
 * commit summary: the decoder carries a few latent frames per pass to bound its memory.]
 *
 *   y[n,od,oh,ow,co] = E( b[co] + sum_{ci,kd,ky,kx} w[co,ci,kd,ky,kx]
 *                                 * X[n, od+d_org-1+kd, oh+h_org-1+ky, ow-1+kx, ci] )
 * for od < D_out, oh < H_out, ow < W, where X is x (N,D_in,H_in,W,C_in) NDHWC inside input frames
 * [d_lo, d_hi) and rows [h_lo, h_hi) and columns [0, W), and zero everywhere else: frames and
 * rows outside the valid ranges are never read, whatever they hold.  y is (N,D_out,H_out,W,
 * C_out) NDHWC.  With D_in = D_out, H_in = H_out, origins 0 and the whole tensor valid this is
 * conv3x3x3_fwd.  Examples:
 *   - row band [lo, lo+rows) of a global height Hg, x holding global rows lo-g .. lo+rows+g-1:
 *     H_out = rows, H_in = rows + 2g, h_org = g, h_lo = max(0, g-lo), h_hi = min(H_in, Hg+g-lo);
 *   - causal temporal padding (output frame t reads frames t-2 .. t, zeros before frame 0):
 *     D_in = D_out, d_org = -1, d_lo = 0, d_hi = D_in;
 *   - the next chunk of a causal pass with the previous chunk's last two frames in front of x:
 *     D_in = D_out + 2, d_org = 1, d_lo = 0, d_hi = D_in.
 * Requirements beyond conv3x3x3_fwd's: 0 <= d_lo <= d_hi <= D_in, 0 <= h_lo <= h_hi <= H_in
 * (else CONV_E_INVAL); every output frame reads at least one valid input frame, i.e. d_lo < d_hi,
 * d_lo <= d_org + 1 and D_out + d_org - 1 <= d_hi (else CONV_E_UNSUPPORTED).  SPLIT_HEAD
 * computes its plane for the output rows plus, when input rows h_org-1 or H_out+h_org hold
 * data, the Z rows just above and below the band (head.cu's g_off = 1).  The algorithm, the
 * weight packing and the
 * workspace are those of conv3x3x3_fwd for the OUTPUT extent: pass (N, C_in, C_out, D_out,
 * H_out, W) to conv3x3x3_select_algo, _packed_weight_bytes, _pack_weights and _workspace_bytes.
 * x, y and the workspace must not overlap.
 * ---------------------------------------------------------------------------------------- */
int conv3x3x3_fwd_region(const void *x, const void *w_packed, const void *bias, void *y, int N,
                         int C_in, int C_out, int D_in, int H_in, int W, int D_out, int H_out,
                         int d_org, int h_org, int d_lo, int d_hi, int h_lo, int h_hi, int layout,
                         int dtype, int epilogue, int algo, void *workspace,
                         size_t workspace_bytes, void *stream);

/* The concrete algorithm conv3x3x3_fwd runs for `algo` (AUTO resolved), or a negative status
 * if the request is unsupported.  [head.cu, header comment: the 27-tap head computed directly or
 * as the temporal conv + stencil split.] */
int conv3x3x3_select_algo(int N, int C_in, int C_out, int D, int H, int W, int stride,
                          int layout, int dtype, int algo);

/* CONV_OK if conv3x3x3_fwd would accept this request (pointers aside), else its status.
 * Host-only, no device work.  [head.cu, commit summary: the ranks' agreement on whether every
 * one of them could build the kernel.] */
int conv3x3x3_is_supported(int N, int C_in, int C_out, int D, int H, int W, int stride,
                           int layout, int dtype, int epilogue, int algo);

/* Bytes of workspace conv3x3x3_fwd (and conv3x3x3_fwd_region for this output extent) needs:
 * the split head's intermediate plane with room for one row above and below the output rows
 * (N*D*(H+2)*W*112 elements of dtype), the split-K partial sums of the MFMA path for small
 * position counts (fp32), the stream-K partial tiles and per-tile arrival counters of the MFMA
 * path where a single round of whole tiles would leave compute units idle (256 KiB per
 * workgroup, at most 256 of them, + 4 bytes per tile; the counters are cleared by a small kernel
 * the call enqueues first, so the workspace needs no initial contents), or 0.  Returns 0 for an unsupported request as well.  The caller
 * allocates and frees the workspace.  [head.cu, head_stencil host function: the caller hands in
 * the 112-channel plane g that the temporal conv wrote.] */
size_t conv3x3x3_workspace_bytes(int N, int C_in, int C_out, int D, int H, int W, int stride,
                                 int layout, int dtype, int algo);

/* Bytes of the packed weight buffer for this request (0 if unsupported).  [head.cu, header
 * comment: the head's weight stays resident across the pass, so its layout is the kernel's
 * choice.] */
size_t conv3x3x3_packed_weight_bytes(int N, int C_in, int C_out, int D, int H, int W,
                                     int stride, int layout, int dtype, int algo);

/* A one-line description of the launch plan conv3x3x3_fwd would use for this request, written
 * to buf (host memory of buf_len bytes, caller-owned; truncated to buf_len - 1 characters and
 * NUL-terminated): "fused_head" / "split_head" with the head's work split (strips of 126 / 128
 * positions, groups of four frames, row ranges per frame group, the largest range's Z rows,
 * workgroups), or the MFMA kernel ("igemm32", "igemm32_kq" when the four waves of a workgroup
 * split K, "igemm32_sk" for the stream-K schedule, "igemm16_wide", "igemm16_narrow") with its
 * position tile (rows x columns of one frame), output rows per workgroup, split-K factor and
 * workgroup count.  Returns the full length of the description, or a negative status (CONV_E_INVAL for a
 * NULL buf or buf_len < 1, else what conv3x3x3_select_algo returns).  Host-only.  [head.cu,
 * header comment: which of the head's forms, direct or split, a pass runs.] */
int conv3x3x3_describe(int N, int C_in, int C_out, int D, int H, int W, int stride, int layout,
                       int dtype, int algo, char *buf, int buf_len);

/* One-time repack of PyTorch Conv3d weights w_oidhw (C_out,C_in,3,3,3) of `dtype` (device
 * memory) into w_packed (device memory of conv3x3x3_packed_weight_bytes bytes), enqueued on
 * `stream`.  Weights are constant across passes, so this runs outside the timed pass.  The
 * caller owns both buffers; w_oidhw may be freed once the stream has passed this call.
 * [head.cu, header comment: the weight is resident while the pass streams the activations.]
 * Errors: CONV_E_INVAL for NULL or misaligned pointers or overlapping buffers, otherwise the
 * status conv3x3x3_fwd would return for the request; nothing is enqueued on error. */
int conv3x3x3_pack_weights(const void *w_oidhw, void *w_packed, int N, int C_in, int C_out,
                           int D, int H, int W, int stride, int layout, int dtype, int algo,
                           void *stream);

/* ------------------------------------------------------------------------------------------
 * The head's output as 8-bit RGB video frames.  [head.cu, header comment: the clamped
 * 12-channel output is what the video writer consumes; commit summary: the decoded RGB video's
 * frames are copied to the host once.]  The mapping is not given there; this library takes a
 * factor-2 pixel shuffle and a linear [-1, 1] -> [0, 255] code:
 *   rgb[n,d,2h+dy,2w+dx,c] = clamp(RNE(127.5 * (y[n,d,h,w,4c+2dy+dx] + 1)), 0, 255)
 * rounded from the exact value (half to even), NaN -> 0, +inf -> 255, -inf -> 0.
 * y: (N,D,H,W,C) NDHWC of `dtype` (device, 16-byte aligned), C must be 12 (else
 * CONV_E_UNSUPPORTED); rgb: (N,D,2H,2W,3) uint8 (device; 16-byte aligned with W % 8 == 0 takes
 * the widest stores).  y and rgb must not overlap.  Enqueued on `stream`.
 * ---------------------------------------------------------------------------------------- */
int conv_video_rgb8(const void *y, void *rgb, int N, int D, int H, int W, int C, int dtype,
                    void *stream);

/* The fused head (CONV_ALGO_FUSED_HEAD, C_out = 12) writing the RGB frames of its output directly:
 * rgb equals conv_video_rgb8 applied to the y that conv3x3x3_fwd computes for the same
 * arguments (each value rounded to `dtype`, then coded), but y is never stored.  x (N,D,H,W,C_in)
 * NDHWC, w_packed from conv3x3x3_pack_weights(..., C_out = 12, ..., CONV_ALGO_FUSED_HEAD), bias
 * (12) or NULL, rgb (N,D,2H,2W,3) uint8 (2-byte aligned).  Requirements
 * and errors otherwise as conv3x3x3_fwd with CONV_ALGO_FUSED_HEAD.  [head.cu, header comment:
 * the clamped 12-channel output feeds the video writer.] */
int conv3x3x3_head_rgb8(const void *x, const void *w_packed, const void *bias, void *rgb, int N,
                        int C_in, int D, int H, int W, int dtype, int epilogue, void *stream);

/* ------------------------------------------------------------------------------------------
 * The split head's two stages as separate calls (conv3x3x3_fwd with CONV_ALGO_SPLIT_HEAD runs
 * both on one stream).  [head.cu: the temporal 3x1x1 convolution that writes the plane, and the
 * host function head_stencil(g, bias, out, ...) that sums it.]
 *
 * conv_head_temporal: x (N,D,H,W,C_in) NDHWC, w_packed packed with CONV_ALGO_SPLIT_HEAD for
 *   this shape, g (N,D,H,W,112) channels-last of `dtype`:
 *     g[n,d,h,w,(ky*3+kx)*C_out+co] = round( sum_{ci,kd} w[co,ci,kd,ky,kx] * X[n,ci,d-1+kd,h,w] )
 *   channels 9*C_out..111 are written as zero.  No bias.  C_out <= 12, C_in % 8 == 0.
 * conv_head_stencil: g as above, bias (C_out) or NULL, y (N,D,H,W,C_out) NDHWC:
 *     y[n,d,h,w,co] = round( E( b[co] + sum_{ky,kx} g[n,d,h+ky-1,w+kx-1,(ky*3+kx)*C_out+co] ) )
 *   with g zero outside the plane.  g and y must not overlap.
 * ---------------------------------------------------------------------------------------- */
int conv_head_temporal(const void *x, const void *w_packed, void *g, int N, int C_in, int C_out,
                       int D, int H, int W, int dtype, void *stream);
int conv_head_stencil(const void *g, const void *bias, void *y, int N, int D, int H, int W,
                      int C_out, int dtype, int epilogue, void *stream);

/* ------------------------------------------------------------------------------------------
 * For callers that cannot allocate device memory -- code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc: conv3x3x3_fwd with the same arguments and results, but
 * without a workspace argument.  Where the request needs a workspace (the split-K partial sums of
 * the MFMA path for small position counts, its stream-K partial tiles and arrival counters --
 * up to 64 MiB plus 4 bytes per tile --, the split head's plane), it uses a static device
 * array of CONV_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on until the
 * process ends; nothing else is allocated, by the library or by any routine it calls.
 *   - Returns CONV_E_WORKSPACE, with nothing enqueued, when the request needs more than
 *     CONV_NOALLOC_SCRATCH_BYTES (conv3x3x3_workspace_bytes says how much it needs); other
 *     errors as conv3x3x3_fwd.  AUTO resolves as in conv3x3x3_fwd (the fused head needs no
 *     workspace; the split head's plane fits only small frames).
 *   - Every call on a GPU shares that GPU's array, which keeps the last call's contents (no call
 *     relies on them: every value read is written first in the same call).  Calls that overlap
 *     on one GPU -- on different streams, or from different threads -- race on the array; the
 *     caller orders them (one stream, or events).
 *   - The first call on a device looks up the array's device address (no allocation, no work
 *     enqueued); a caller that captures a graph makes one call before the capture.
 * ---------------------------------------------------------------------------------------- */
#define CONV_NOALLOC_SCRATCH_BYTES (80u << 20)
int conv3x3x3_fwd_noalloc(const void *x, const void *w_packed, const void *bias, void *y, int N,
                          int C_in, int C_out, int D, int H, int W, int stride, int layout,
                          int dtype, int epilogue, int algo, void *stream);

/* ------------------------------------------------------------------------------------------
 * Measurement aid, not part of the convolution: enqueues `workgroups` workgroups of four waves,
 * each wave issuing `iters` x 8 independent bf16 32x32x16 MFMAs on register operands (2 * 32 *
 * 32 * 16 FLOP each), and writes one float per lane to `out` (device memory of workgroups * 256
 * floats, caller-owned).  Timed by the caller, it gives the rate this machine's matrix cores
 * sustain under a pure MFMA load.  Returns CONV_E_INVAL for a NULL `out`, workgroups outside
 * 1..2^20 or iters < 1, CONV_E_LAUNCH if the launch is rejected.
 * ---------------------------------------------------------------------------------------- */
int conv_calib_mfma_bf16(void *out, int workgroups, int iters, void *stream);

/* Measurement aid, not part of the convolution: enqueues `workgroups` workgroups of four waves,
 * each wave issuing iters x 16 global -> LDS copies of 1 KiB (16 bytes per lane) from `src`
 * (device memory of src_bytes bytes, caller-owned, 1 MiB <= src_bytes < 2 GiB; only the first
 * half plus one copy's span is read).  whole_lines != 0: each copy reads 1 KiB of consecutive
 * bytes (eight whole 128-byte lines); 0: 16 pieces of 64 bytes 512 bytes apart (half lines).
 * Timed by the caller, bytes = workgroups * 4 * iters * 16 KiB.  Returns CONV_E_INVAL for bad
 * arguments, CONV_E_LAUNCH if the launch is rejected. */
int conv_calib_lds_dma(const void *src, size_t src_bytes, int whole_lines, int workgroups,
                       int iters, void *stream);

/* Measurement aid, not part of the convolution: enqueues `workgroups` workgroups of `waves`
 * waves (4 or 8; 64 KiB of LDS each, so two share a CU), each wave issuing iters x 8
 * conflict-free 16-byte-per-lane LDS reads of 1 KiB; `out` (device memory, caller-owned) takes
 * workgroups * waves * 64 * 16 bytes of folded values.  Timed by the caller, bytes = workgroups
 * * waves * 64 * 16 * 8 * iters.  Returns CONV_E_INVAL for bad arguments, CONV_E_LAUNCH if the
 * launch is rejected. */
int conv_calib_lds_read(void *out, int workgroups, int waves, int iters, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* CONV3X3_H_ */
