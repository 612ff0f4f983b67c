/*
 * conv_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * The plain, slow, obviously-correct CPU definition of the pad-1 3x3 (2D) and 3x3x3 (3D)
 * convolution with fused bias and ReLU / [-1,1] clamp / identity epilogue, written out as nested
 * loops in fp64.  Only the tests, the smoke check and the benchmark's CPU-baseline leg may load
 * this library.  It shares no code, header, table or constant with the HIP library: it has its
 * own fp16/bf16 decoders and its own round-to-nearest-even encoder.
 *
 * Pages followed (cited by title and section):
 *   [taesd]  musetalk-bench, patches/taesd_conv.cuh.new -- header comment (operator contract:
 *            NCHW, fp16 storage, fp32 accumulation, 3x3, pad 1, stride 1 or 2, optional bias,
 *            optional fused ReLU) and taesd_conv3x3_impl (the receptive field of output
 *            (oh,ow) starts at input (oh*s-1, ow*s-1); weights are (C_out, C_in, 3, 3); the tap
 *            (ky,kx) multiplies input (oh*s-1+ky, ow*s-1+kx): cross-correlation, no flip;
 *            the accumulator starts at the bias; ReLU maps negative values to zero).
 *   [head]   FastVideo, fastvideo-kernel/wan22_vae_decode/solution/head.cu -- header comment
 *            (the 27-tap 3x3x3 output convolution, its split into a 3x1x1 temporal convolution
 *            that writes the nine spatial taps as 9*12 channels, a nine-tap shifted sum, the
 *            bias, the clamp to [-1,1], and where the value path rounds) and head_stencil_kernel
 *            (channel index (i*3+j)*12+c of the plane, i = row tap, j = column tap; zero padding
 *            outside the plane; clamp before the bf16 store).
 *
 * Readings of points the pages leave open (each also listed in the design notes):
 *   - temporal padding of the 3D convolution is one zero frame at each end, D_out = D;
 *   - the 3D weight layout is (C_out, C_in, 3, 3, 3) = (co, ci, kd, ky, kx);
 *   - stride applies to H and W only; H_out = floor((H-1)/s)+1;
 *   - bias is added before the activation; a NULL bias means zero;
 *   - ReLU keeps NaN (v<0 ? 0 : v); the clamp is min(1, max(-1, v)).
 *
 * Every sum is taken in fp64 from exactly-decoded inputs; outputs are returned unrounded in fp64.
 * Parity pins: see the header of oracle/__init__.py for what fixes each function.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F16 = 0, OR_BF16 = 1 };
enum { OR_CHANNELS_FIRST = 0, OR_CHANNELS_LAST = 1 };
enum { OR_EPI_NONE = 0, OR_EPI_RELU = 1, OR_EPI_CLAMP1 = 2 };

/* ---------------------------------------------------------------------------------------------
 * Number formats.  IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * bfloat16: the upper 16 bits of an IEEE binary32 (1 sign, 8 exponent bits with bias 127,
 * 7 fraction bits).  Both decoders are exact in fp64.
 * ------------------------------------------------------------------------------------------- */
static double decode_f16(uint16_t h) {
    int sign = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24); /* subnormal: m * 2^(1-15-10) */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25); /* (1 + m/2^10) * 2^(e-15) */
    return sign ? -v : v;
}

static double decode_bf16(uint16_t b) {
    int sign = b >> 15, e = (b >> 7) & 0xff, m = b & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)m, -133); /* subnormal: m * 2^(1-127-7) */
    else if (e == 255)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + m), e - 134); /* (1 + m/2^7) * 2^(e-127) */
    return sign ? -v : v;
}

double oracle_decode_one(uint16_t bits, int dtype) {
    return dtype == OR_BF16 ? decode_bf16(bits) : decode_f16(bits);
}

/* Round an fp64 value to the nearest fp16/bf16, ties to even, overflow to infinity. */
uint16_t oracle_encode_one(double v, int dtype) {
    const int p = dtype == OR_BF16 ? 7 : 10;          /* fraction bits */
    const int bias = dtype == OR_BF16 ? 127 : 15;
    const int emin = 1 - bias;                        /* exponent of the smallest normal */
    const int emax = bias;                            /* exponent of the largest finite */
    const int ebits = dtype == OR_BF16 ? 8 : 5;
    const uint16_t inf_bits = (uint16_t)(((1u << ebits) - 1u) << p);
    if (isnan(v)) return (uint16_t)(inf_bits | (1u << (p - 1)));
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    if (isinf(a)) return sign | inf_bits;
    int e2;
    frexp(a, &e2);          /* a = f * 2^e2, f in [0.5, 1): a lies in [2^(e2-1), 2^e2) */
    int E = e2 - 1;
    if (E < emin) E = emin; /* subnormal range shares the smallest normal's quantum */
    double q = ldexp(1.0, E - p);
    double n = rint(a / q); /* a/q is exact (power-of-two scale); rint rounds half to even */
    double r = n * q;
    /* The largest finite value is (2 - 2^-p) * 2^emax; at or past it plus half a quantum the
     * ties-to-even rule lands on 2^(emax+1), i.e. overflow. */
    if (r >= ldexp(1.0, emax + 1)) return sign | inf_bits;
    if (r < ldexp(1.0, emin)) {
        /* subnormal (or the smallest normal reached by rounding up, which encodes the same way:
         * fraction 2^p means exponent field 1, fraction 0) */
        uint32_t m = (uint32_t)(r / ldexp(1.0, emin - p));
        return sign | (uint16_t)m;
    }
    int er;
    frexp(r, &er);
    int Er = er - 1;
    uint32_t frac = (uint32_t)(r / ldexp(1.0, Er - p)) - (1u << p);
    return sign | (uint16_t)(((uint32_t)(Er + bias) << p) | frac);
}

void oracle_decode(const uint16_t *in, double *out, int64_t n, int dtype) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_decode_one(in[i], dtype);
}

void oracle_encode(const double *in, uint16_t *out, int64_t n, int dtype) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_encode_one(in[i], dtype);
}

/* Lookup table of all 65536 decoded values, so that the loops below read decoded inputs
 * without a per-element branchy decode.  It is filled with the decoder above. */
static double *make_table(int dtype) {
    double *t = (double *)malloc(65536 * sizeof(double));
    if (!t) return NULL;
    for (int i = 0; i < 65536; ++i) t[i] = oracle_decode_one((uint16_t)i, dtype);
    return t;
}

/* The epilogue: bias already in the sum; ReLU as a compare-and-zero, clamp as min/max. */
static double epilogue(double v, int epi) {
    if (epi == OR_EPI_RELU) return v < 0.0 ? 0.0 : v;
    if (epi == OR_EPI_CLAMP1) return fmin(1.0, fmax(-1.0, v));
    return v;
}

int oracle_out_size(int in, int stride) { return (in - 1) / stride + 1; }

/* Element offset of logical (n, c, d, h, w) in a tensor of logical shape (N, C, D, H, W) stored
 * channels-first (N, C, D, H, W) or channels-last (N, D, H, W, C).  2D tensors use D = 1. */
static int64_t offset5(int layout, int64_t n, int64_t c, int64_t d, int64_t h, int64_t w,
                       int64_t C, int64_t D, int64_t H, int64_t W) {
    if (layout == OR_CHANNELS_LAST) return (((n * D + d) * H + h) * W + w) * C + c;
    return (((n * C + c) * D + d) * H + h) * W + w;
}

static int check_enums(int stride, int dtype, int epi, int layout) {
    if (stride != 1 && stride != 2) return -1;
    if (dtype != OR_F16 && dtype != OR_BF16) return -1;
    if (epi < OR_EPI_NONE || epi > OR_EPI_CLAMP1) return -1;
    if (layout != OR_CHANNELS_FIRST && layout != OR_CHANNELS_LAST) return -1;
    return 0;
}

/* ---------------------------------------------------------------------------------------------
 * 2D [taesd, operator contract and taesd_conv3x3_impl]:
 *   y[n,co,oh,ow] = E( b[co] + sum_{ci,ky,kx} w[co,ci,ky,kx] * X[n,ci, s*oh-1+ky, s*ow-1+kx] )
 * with X zero outside the image, 0 <= oh < floor((H-1)/s)+1, likewise ow.
 * x: (N,C_in,H,W); w: (C_out,C_in,3,3); b: (C_out) or NULL; y: (N,C_out,H_out,W_out) in fp64,
 * x and y in `layout` (channels-first = NCHW, channels-last = NHWC).
 * ------------------------------------------------------------------------------------------- */
int oracle_conv2d(const uint16_t *x, const uint16_t *w, const uint16_t *b, double *y, int N,
                  int C_in, int C_out, int H, int W, int stride, int dtype, int epi, int layout) {
    if (check_enums(stride, dtype, epi, layout) || N < 0 || C_in < 1 || C_out < 1 || H < 1 ||
        W < 1)
        return -1;
    double *tab = make_table(dtype);
    if (!tab) return -2;
    const int Ho = oracle_out_size(H, stride), Wo = oracle_out_size(W, stride);
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int n = 0; n < N; ++n)
        for (int oh = 0; oh < Ho; ++oh)
            for (int ow = 0; ow < Wo; ++ow)
                for (int co = 0; co < C_out; ++co) {
                    double acc = b ? tab[b[co]] : 0.0;
                    for (int ky = 0; ky < 3; ++ky) {
                        const int ih = stride * oh - 1 + ky;
                        if (ih < 0 || ih >= H) continue; /* zero padding */
                        for (int kx = 0; kx < 3; ++kx) {
                            const int iw = stride * ow - 1 + kx;
                            if (iw < 0 || iw >= W) continue; /* zero padding */
                            for (int ci = 0; ci < C_in; ++ci) {
                                const double wv = tab[w[(((int64_t)co * C_in + ci) * 3 + ky) * 3 + kx]];
                                const double xv = tab[x[offset5(layout, n, ci, 0, ih, iw, C_in, 1, H, W)]];
                                acc += wv * xv;
                            }
                        }
                    }
                    y[offset5(layout, n, co, 0, oh, ow, C_out, 1, Ho, Wo)] = epilogue(acc, epi);
                }
    free(tab);
    return 0;
}

/* One 3D output vector (all C_out at one position), the definition below written for a single
 * (n, od, oh, ow): shared by the whole-tensor and the sampled-position entry points. */
static void conv3d_point(const double *tab, const uint16_t *x, const uint16_t *w,
                         const uint16_t *b, double *yv, int n, int od, int oh, int ow, int C_in,
                         int C_out, int D, int H, int W, int stride, int epi, int layout) {
    for (int co = 0; co < C_out; ++co) {
        double acc = b ? tab[b[co]] : 0.0;
        for (int kd = 0; kd < 3; ++kd) {
            const int id = od - 1 + kd;
            if (id < 0 || id >= D) continue; /* temporal zero padding, one frame each end */
            for (int ky = 0; ky < 3; ++ky) {
                const int ih = stride * oh - 1 + ky;
                if (ih < 0 || ih >= H) continue;
                for (int kx = 0; kx < 3; ++kx) {
                    const int iw = stride * ow - 1 + kx;
                    if (iw < 0 || iw >= W) continue;
                    for (int ci = 0; ci < C_in; ++ci) {
                        const double wv =
                            tab[w[((((int64_t)co * C_in + ci) * 3 + kd) * 3 + ky) * 3 + kx]];
                        const double xv = tab[x[offset5(layout, n, ci, id, ih, iw, C_in, D, H, W)]];
                        acc += wv * xv;
                    }
                }
            }
        }
        yv[co] = epilogue(acc, epi);
    }
}

/* ---------------------------------------------------------------------------------------------
 * 3D [head, header comment: the 27-tap output convolution with one accumulator; the 2D operator
 * of taesd extended by a temporal tap with the same zero padding]:
 *   y[n,co,od,oh,ow] = E( b[co] + sum_{ci,kd,ky,kx} w[co,ci,kd,ky,kx]
 *                                  * X[n,ci, od-1+kd, s*oh-1+ky, s*ow-1+kx] ),  D_out = D.
 * x: (N,C_in,D,H,W); w: (C_out,C_in,3,3,3); y: (N,C_out,D,H_out,W_out), in `layout`
 * (channels-first = NCDHW, channels-last = NDHWC).
 * ------------------------------------------------------------------------------------------- */
int oracle_conv3d(const uint16_t *x, const uint16_t *w, const uint16_t *b, double *y, int N,
                  int C_in, int C_out, int D, int H, int W, int stride, int dtype, int epi,
                  int layout) {
    if (check_enums(stride, dtype, epi, layout) || N < 0 || C_in < 1 || C_out < 1 || D < 1 ||
        H < 1 || W < 1)
        return -1;
    double *tab = make_table(dtype);
    if (!tab) return -2;
    const int Ho = oracle_out_size(H, stride), Wo = oracle_out_size(W, stride);
    int rc = 0;
#pragma omp parallel
    {
        double *yv = (double *)malloc((size_t)C_out * sizeof(double));
        if (!yv) {
#pragma omp atomic write
            rc = -2;
        }
#pragma omp for collapse(3) schedule(dynamic)
        for (int n = 0; n < N; ++n)
            for (int od = 0; od < D; ++od)
                for (int oh = 0; oh < Ho; ++oh) {
                    if (!yv) continue;
                    for (int ow = 0; ow < Wo; ++ow) {
                        conv3d_point(tab, x, w, b, yv, n, od, oh, ow, C_in, C_out, D, H, W,
                                     stride, epi, layout);
                        for (int co = 0; co < C_out; ++co)
                            y[offset5(layout, n, co, od, oh, ow, C_out, D, Ho, Wo)] = yv[co];
                    }
                }
        free(yv);
    }
    free(tab);
    return rc;
}

/* The same definition evaluated only at `npts` output positions pts[4*i..4*i+3] = (n,od,oh,ow);
 * y_pts[i*C_out + co] receives y[n,co,od,oh,ow].  Lets a full-size tensor be checked at sampled
 * positions, one by one. */
int oracle_conv3d_points(const uint16_t *x, const uint16_t *w, const uint16_t *b,
                         const int32_t *pts, int64_t npts, double *y_pts, int N, int C_in,
                         int C_out, int D, int H, int W, int stride, int dtype, int epi,
                         int layout) {
    if (check_enums(stride, dtype, epi, layout) || C_in < 1 || C_out < 1 || D < 1 || H < 1 ||
        W < 1)
        return -1;
    const int Ho = oracle_out_size(H, stride), Wo = oracle_out_size(W, stride);
    for (int64_t i = 0; i < npts; ++i) {
        const int32_t *p = pts + 4 * i;
        if (p[0] < 0 || p[0] >= N || p[1] < 0 || p[1] >= D || p[2] < 0 || p[2] >= Ho ||
            p[3] < 0 || p[3] >= Wo)
            return -1;
    }
    double *tab = make_table(dtype);
    if (!tab) return -2;
#pragma omp parallel for schedule(dynamic)
    for (int64_t i = 0; i < npts; ++i) {
        const int32_t *p = pts + 4 * i;
        conv3d_point(tab, x, w, b, y_pts + i * C_out, p[0], p[1], p[2], p[3], C_in, C_out, D,
                     H, W, stride, epi, layout);
    }
    free(tab);
    return 0;
}

/* 2D at sampled output positions pts[3*i..3*i+2] = (n,oh,ow); y_pts[i*C_out+co]. */
int oracle_conv2d_points(const uint16_t *x, const uint16_t *w, const uint16_t *b,
                         const int32_t *pts, int64_t npts, double *y_pts, int N, int C_in,
                         int C_out, int H, int W, int stride, int dtype, int epi, int layout) {
    if (check_enums(stride, dtype, epi, layout) || C_in < 1 || C_out < 1 || H < 1 || W < 1)
        return -1;
    const int Ho = oracle_out_size(H, stride), Wo = oracle_out_size(W, stride);
    for (int64_t i = 0; i < npts; ++i) {
        const int32_t *p = pts + 3 * i;
        if (p[0] < 0 || p[0] >= N || p[1] < 0 || p[1] >= Ho || p[2] < 0 || p[2] >= Wo) return -1;
    }
    double *tab = make_table(dtype);
    if (!tab) return -2;
#pragma omp parallel for schedule(dynamic)
    for (int64_t i = 0; i < npts; ++i) {
        const int n = pts[3 * i], oh = pts[3 * i + 1], ow = pts[3 * i + 2];
        for (int co = 0; co < C_out; ++co) {
            double acc = b ? tab[b[co]] : 0.0;
            for (int ky = 0; ky < 3; ++ky) {
                const int ih = stride * oh - 1 + ky;
                if (ih < 0 || ih >= H) continue;
                for (int kx = 0; kx < 3; ++kx) {
                    const int iw = stride * ow - 1 + kx;
                    if (iw < 0 || iw >= W) continue;
                    for (int ci = 0; ci < C_in; ++ci) {
                        const double wv = tab[w[(((int64_t)co * C_in + ci) * 3 + ky) * 3 + kx]];
                        const double xv = tab[x[offset5(layout, n, ci, 0, ih, iw, C_in, 1, H, W)]];
                        acc += wv * xv;
                    }
                }
            }
            y_pts[i * C_out + co] = epilogue(acc, epi);
        }
    }
    free(tab);
    return 0;
}

/* ---------------------------------------------------------------------------------------------
 * Split head [head, header comment and head_stencil_kernel], stride 1 only:
 *   G[n,d,h,w,(ky*3+kx)*C_out+co] = sum_{ci,kd} w[co,ci,kd,ky,kx] * X[n,ci,d-1+kd,h,w]
 *     (the 3x1x1 temporal convolution whose output channels are the nine spatial taps);
 *   optionally G is rounded to the activation dtype (round_g != 0), the page's first rounding;
 *   y[n,co,d,h,w] = E( b[co] + sum_{ky,kx} G[n,d,h+ky-1,w+kx-1,(ky*3+kx)*C_out+co] ),
 *     G zero outside the plane (the spatial zero padding).
 * Without rounding this equals oracle_conv3d at stride 1 (the algebra of the split); with it,
 * it models the page's value path in fp64.  g_out (optional) receives G as an
 * (N, D, H, W, 9*C_out) channels-last fp64 array.  x and y use `layout`.
 * ------------------------------------------------------------------------------------------- */
int oracle_head_split(const uint16_t *x, const uint16_t *w, const uint16_t *b, double *y,
                      double *g_out, int N, int C_in, int C_out, int D, int H, int W, int dtype,
                      int epi, int layout, int round_g) {
    if (check_enums(1, dtype, epi, layout) || N < 0 || C_in < 1 || C_out < 1 || D < 1 || H < 1 ||
        W < 1)
        return -1;
    double *tab = make_table(dtype);
    if (!tab) return -2;
    const int GC = 9 * C_out;
    const int64_t gsz = (int64_t)N * D * H * W * GC;
    double *G = g_out ? g_out : (double *)malloc((size_t)gsz * sizeof(double));
    if (!G) {
        free(tab);
        return -2;
    }
#pragma omp parallel for collapse(3) schedule(dynamic)
    for (int n = 0; n < N; ++n)
        for (int d = 0; d < D; ++d)
            for (int h = 0; h < H; ++h)
                for (int ww = 0; ww < W; ++ww)
                    for (int ky = 0; ky < 3; ++ky)
                        for (int kx = 0; kx < 3; ++kx)
                            for (int co = 0; co < C_out; ++co) {
                                double acc = 0.0;
                                for (int kd = 0; kd < 3; ++kd) {
                                    const int id = d - 1 + kd;
                                    if (id < 0 || id >= D) continue;
                                    for (int ci = 0; ci < C_in; ++ci)
                                        acc += tab[w[((((int64_t)co * C_in + ci) * 3 + kd) * 3 + ky) * 3 + kx]] *
                                               tab[x[offset5(layout, n, ci, id, h, ww, C_in, D, H, W)]];
                                }
                                if (round_g) acc = tab[oracle_encode_one(acc, dtype)];
                                G[((((int64_t)n * D + d) * H + h) * W + ww) * GC + (ky * 3 + kx) * C_out + co] = acc;
                            }
#pragma omp parallel for collapse(3) schedule(dynamic)
    for (int n = 0; n < N; ++n)
        for (int d = 0; d < D; ++d)
            for (int h = 0; h < H; ++h)
                for (int ww = 0; ww < W; ++ww)
                    for (int co = 0; co < C_out; ++co) {
                        double acc = b ? tab[b[co]] : 0.0;
                        for (int ky = 0; ky < 3; ++ky) {
                            const int hh = h + ky - 1;
                            if (hh < 0 || hh >= H) continue;
                            for (int kx = 0; kx < 3; ++kx) {
                                const int w2 = ww + kx - 1;
                                if (w2 < 0 || w2 >= W) continue;
                                acc += G[((((int64_t)n * D + d) * H + hh) * W + w2) * GC + (ky * 3 + kx) * C_out + co];
                            }
                        }
                        y[offset5(layout, n, co, d, h, ww, C_out, D, H, W)] = epilogue(acc, epi);
                    }
    if (!g_out) free(G);
    free(tab);
    return 0;
}

/* ---------------------------------------------------------------------------------------------
 * Thread count of the OpenMP loops above (no arithmetic): the CPU-baseline timing reports how
 * many threads the oracle used and times a single-threaded pass as well.
 * ------------------------------------------------------------------------------------------- */
#include <omp.h>

int oracle_max_threads(void) { return omp_get_max_threads(); }

void oracle_set_threads(int n) {
    if (n > 0) omp_set_num_threads(n);
}
