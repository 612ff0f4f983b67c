/* Host sanitizer driver for the CPU oracle (test infrastructure): calls every entry point of
 * conv_oracle.c on tiny inputs and with invalid arguments, so AddressSanitizer and
 * UndefinedBehaviorSanitizer see every loop and every early return.  Exits 0 when every call
 * returned what it should; the sanitizers abort on their own findings. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_conv2d(const uint16_t *x, const uint16_t *w, const uint16_t *b, double *y, int N,
                  int C_in, int C_out, int H, int W, int stride, int dtype, int epi, int layout);
int oracle_conv3d(const uint16_t *x, const uint16_t *w, const uint16_t *b, double *y, int N,
                  int C_in, int C_out, int D, int H, int W, int stride, int dtype, int epi,
                  int layout);
int oracle_conv3d_points(const uint16_t *x, const uint16_t *w, const uint16_t *b,
                         const int32_t *pts, int64_t npts, double *y_pts, int N, int C_in,
                         int C_out, int D, int H, int W, int stride, int dtype, int epi,
                         int layout);
int oracle_conv2d_points(const uint16_t *x, const uint16_t *w, const uint16_t *b,
                         const int32_t *pts, int64_t npts, double *y_pts, int N, int C_in,
                         int C_out, int H, int W, int stride, int dtype, int epi, int layout);
int oracle_head_split(const uint16_t *x, const uint16_t *w, const uint16_t *b, double *y,
                      double *g_out, int N, int C_in, int C_out, int D, int H, int W, int dtype,
                      int epi, int layout, int round_g);
double oracle_decode_one(uint16_t bits, int dtype);
uint16_t oracle_encode_one(double v, int dtype);
void oracle_decode(const uint16_t *in, double *out, int64_t n, int dtype);
void oracle_encode(const double *in, uint16_t *out, int64_t n, int dtype);
int oracle_out_size(int in, int stride);

static int fails = 0;
#define EXPECT(c)                                                   \
    do {                                                            \
        if (!(c)) {                                                 \
            fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #c); \
            ++fails;                                                \
        }                                                           \
    } while (0)

static uint16_t *bits(size_t n, unsigned seed) {
    uint16_t *p = (uint16_t *)malloc(n * sizeof(uint16_t));
    for (size_t i = 0; i < n; ++i) {
        seed = seed * 1103515245u + 12345u;
        p[i] = (uint16_t)(0x3C00u ^ ((seed >> 16) & 0x83FFu));   /* finite values near +-1 */
    }
    return p;
}

int main(void) {
    for (int dtype = 0; dtype < 2; ++dtype) {
        for (unsigned v = 0; v < 65536; ++v) {
            const double d = oracle_decode_one((uint16_t)v, dtype);
            (void)oracle_encode_one(d, dtype);
        }
        const int N = 2, Ci = 3, Co = 4, D = 3, H = 5, W = 6;
        uint16_t *x = bits((size_t)N * Ci * D * H * W, 1u + dtype), *w = bits((size_t)Co * Ci * 27, 7u),
                 *b = bits(Co, 9u);
        double *y = (double *)malloc(sizeof(double) * N * Co * D * H * W);
        double *g = (double *)malloc(sizeof(double) * N * D * H * W * 9 * Co);
        uint16_t *enc = (uint16_t *)malloc(sizeof(uint16_t) * N * Co * D * H * W);
        for (int layout = 0; layout < 2; ++layout)
            for (int stride = 1; stride <= 2; ++stride)
                for (int epi = 0; epi < 3; ++epi) {
                    EXPECT(oracle_conv2d(x, w, b, y, N, Ci, Co, H, W, stride, dtype, epi, layout) == 0);
                    EXPECT(oracle_conv2d(x, w, NULL, y, N, Ci, Co, H, W, stride, dtype, epi, layout) == 0);
                    EXPECT(oracle_conv3d(x, w, b, y, N, Ci, Co, D, H, W, stride, dtype, epi, layout) == 0);
                }
        oracle_encode(y, enc, (int64_t)N * Co * D * H * W, dtype);
        oracle_decode(enc, y, (int64_t)N * Co * D * H * W, dtype);
        const int32_t p3[] = {0, 0, 0, 0, 1, 2, 4, 5, 1, 1, 2, 3};
        const int32_t p2[] = {0, 0, 0, 1, 4, 5, 1, 2, 3};
        EXPECT(oracle_conv3d_points(x, w, b, p3, 3, y, N, Ci, Co, D, H, W, 1, dtype, 2, 1) == 0);
        EXPECT(oracle_conv2d_points(x, w, b, p2, 3, y, N, Ci, Co, H, W, 1, dtype, 1, 0) == 0);
        for (int round_g = 0; round_g < 2; ++round_g) {
            EXPECT(oracle_head_split(x, w, b, y, g, N, Ci, Co, D, H, W, dtype, 2, 1, round_g) == 0);
            EXPECT(oracle_head_split(x, w, b, y, NULL, N, Ci, Co, D, H, W, dtype, 2, 0, round_g) == 0);
        }
        /* invalid arguments return an error before touching any buffer */
        const int32_t bad3[] = {0, 3, 0, 0};
        const int32_t bad2[] = {2, 0, 0};
        EXPECT(oracle_conv3d_points(x, w, b, bad3, 1, y, N, Ci, Co, D, H, W, 1, dtype, 0, 1) != 0);
        EXPECT(oracle_conv2d_points(x, w, b, bad2, 1, y, N, Ci, Co, H, W, 1, dtype, 0, 0) != 0);
        EXPECT(oracle_conv2d(x, w, b, y, N, Ci, Co, H, W, 3, dtype, 0, 0) != 0);
        EXPECT(oracle_conv3d(x, w, b, y, N, 0, Co, D, H, W, 1, dtype, 0, 1) != 0);
        EXPECT(oracle_conv3d(x, w, b, y, N, Ci, Co, D, H, W, 1, 5, 0, 1) != 0);
        EXPECT(oracle_head_split(x, w, b, y, g, N, Ci, Co, D, H, W, dtype, 7, 1, 0) != 0);
        EXPECT(oracle_out_size(255, 2) == 128 && oracle_out_size(1, 1) == 1);
        free(x), free(w), free(b), free(y), free(g), free(enc);
    }
    if (fails) return 1;
    puts("oracle driver ok");
    return 0;
}
