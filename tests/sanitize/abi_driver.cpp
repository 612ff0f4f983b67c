// Host sanitizer driver for the C ABI's host code (test infrastructure): every call below is a
// request that validation rejects, or a pure host query (sizes, algorithm choice, regions), so
// nothing reaches a device and no GPU is needed.  AddressSanitizer and UndefinedBehaviorSanitizer
// watch the argument checks, the size arithmetic and the error messages.  Exits 0 when every call
// returned what it should.
#include <cstdio>
#include <cstring>

#include "conv3x3.h"

static int fails = 0;
#define EXPECT(c)                                                                  \
    do {                                                                           \
        if (!(c)) {                                                                \
            std::fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #c);  \
            ++fails;                                                               \
        }                                                                          \
    } while (0)

int main() {
    void *const A = reinterpret_cast<void *>(1ull << 20);
    void *const B = reinterpret_cast<void *>(1ull << 30);
    void *const Y = reinterpret_cast<void *>((1ull << 20) + (1ull << 28));
    EXPECT(conv_abi_version() == CONV_ABI_VERSION);
    for (int st = -6; st <= 1; ++st) EXPECT(conv_status_str(st) != nullptr);
    for (int n = -1; n < 300; ++n)
        for (int s = 0; s <= 3; ++s) (void)conv_out_size(n, s);
    // 2D rejections
    EXPECT(conv3x3_fwd(nullptr, B, nullptr, Y, 1, 16, 16, 8, 8, 1, 0, 0, 1, 0, nullptr) == CONV_E_INVAL);
    EXPECT(conv3x3_fwd(A, B, nullptr, Y, 1, 16, 16, 8, 8, 3, 0, 0, 1, 0, nullptr) == CONV_E_INVAL);
    EXPECT(conv3x3_fwd(A, B, nullptr, Y, 1, 16, 16, 8, 8, 1, 0, 9, 1, 0, nullptr) == CONV_E_INVAL);
    EXPECT(conv3x3_fwd(A, B, nullptr, Y, 1, 16, 16, 8, 8, 1, 0, 0, 7, 0, nullptr) == CONV_E_INVAL);
    EXPECT(conv3x3_fwd(A, B, nullptr, A, 1, 16, 16, 8, 8, 1, 0, 0, 1, 0, nullptr) == CONV_E_INVAL);
    EXPECT(conv3x3_fwd(A, B, nullptr, Y, 1, 12, 16, 8, 8, 1, 1, 0, 1, 0, nullptr) == CONV_E_UNSUPPORTED);
    EXPECT(conv3x3_fwd(A, B, nullptr, Y, 1, 16, 16, 8, 8, 1, 0, 0, 1, CONV_ALGO_SPLIT_HEAD, nullptr) == CONV_E_UNSUPPORTED);
    EXPECT(std::strlen(conv_last_error()) > 0);
    EXPECT(conv3x3_is_supported(8, 64, 64, 256, 256, 2, 0, 0, 1, 0) == CONV_OK);
    EXPECT(conv3x3_select_algo(8, 64, 64, 256, 256, 1, 0, 0, 0) == CONV_ALGO_MFMA);
    EXPECT(conv3x3_fwd(nullptr, nullptr, nullptr, nullptr, 0, 16, 16, 8, 8, 1, 0, 0, 1, 0, nullptr) == CONV_OK);
    // 3D rejections and queries
    EXPECT(conv3x3x3_fwd(nullptr, B, nullptr, Y, 1, 32, 12, 2, 8, 8, 1, 1, 1, 2, 0, nullptr, 0, nullptr) == CONV_E_INVAL);
    EXPECT(conv3x3x3_fwd(A, B, nullptr, Y, 1, 20, 12, 2, 8, 8, 1, 1, 1, 2, 0, nullptr, 0, nullptr) == CONV_E_UNSUPPORTED);
    EXPECT(conv3x3x3_fwd(A, B, nullptr, Y, 1, 32, 12, 2, 8, 8, 1, 0, 1, 2, 0, nullptr, 0, nullptr) == CONV_E_UNSUPPORTED);
    EXPECT(conv3x3x3_fwd(A, B, nullptr, Y, 1, 32, 12, 2, 8, 8, 1, 1, 1, 2, CONV_ALGO_SPLIT_HEAD, nullptr, 0, nullptr) == CONV_E_WORKSPACE);
    const int shapes[][6] = {{1, 256, 12, 16, 352, 624}, {1, 256, 256, 16, 176, 312}, {1, 512, 512, 4, 44, 78},
                             {1, 512, 512, 1, 44, 78}, {2, 40, 20, 3, 9, 13}, {1, 8, 1, 1, 1, 1}};
    for (const auto &s : shapes)
        for (int stride = 1; stride <= 2; ++stride)
            for (int algo = 0; algo <= 5; ++algo) {
                (void)conv3x3x3_select_algo(s[0], s[1], s[2], s[3], s[4], s[5], stride, 1, 1, algo);
                (void)conv3x3x3_workspace_bytes(s[0], s[1], s[2], s[3], s[4], s[5], stride, 1, 1, algo);
                (void)conv3x3x3_packed_weight_bytes(s[0], s[1], s[2], s[3], s[4], s[5], stride, 1, 1, algo);
                (void)conv3x3x3_is_supported(s[0], s[1], s[2], s[3], s[4], s[5], stride, 1, 1, 2, algo);
            }
    EXPECT(conv3x3x3_pack_weights(nullptr, B, 1, 32, 12, 2, 8, 8, 1, 1, 1, 0, nullptr) == CONV_E_INVAL);
    EXPECT(conv3x3x3_fwd_region(A, B, nullptr, Y, 1, 32, 12, 6, 8, 8, 4, 6, 1, 1, 3, 6, 0, 8, 1, 1, 2,
                                CONV_ALGO_FUSED_HEAD, nullptr, 0, nullptr) == CONV_E_UNSUPPORTED);
    EXPECT(conv3x3x3_fwd_region(A, B, nullptr, Y, 1, 32, 12, 6, 8, 8, 4, 6, 1, 1, 0, 7, 0, 8, 1, 1, 2,
                                CONV_ALGO_FUSED_HEAD, nullptr, 0, nullptr) == CONV_E_INVAL);
    EXPECT(conv_head_temporal(nullptr, B, Y, 1, 32, 12, 2, 8, 8, 1, nullptr) == CONV_E_INVAL);
    EXPECT(conv_head_stencil(A, nullptr, Y, 1, 2, 8, 8, 13, 1, 2, nullptr) == CONV_E_UNSUPPORTED);
    EXPECT(conv_video_rgb8(A, Y, 1, 2, 4, 8, 11, 1, nullptr) == CONV_E_UNSUPPORTED);
    EXPECT(conv3x3x3_head_rgb8(nullptr, B, nullptr, Y, 1, 32, 2, 8, 8, 1, 2, nullptr) == CONV_E_INVAL);
    // region helpers
    int f[4];
    for (int Hg = 1; Hg < 40; ++Hg)
        for (int lo = 0; lo <= Hg; ++lo)
            for (int rows = 0; lo + rows <= Hg; rows += 3)
                for (int g = 0; g < 3; ++g) EXPECT(conv_band_region(lo, rows, g, Hg, &f[0], &f[1], &f[2], &f[3]) == CONV_OK);
    EXPECT(conv_band_region(0, 4, 1, 10, nullptr, &f[1], &f[2], &f[3]) == CONV_E_INVAL);
    EXPECT(conv_band_region(8, 4, 1, 10, &f[0], &f[1], &f[2], &f[3]) == CONV_E_INVAL);
    EXPECT(conv_band_region(0, 2147483647, 2, 2147483647, &f[0], &f[1], &f[2], &f[3]) == CONV_E_INVAL);
    for (int d = 0; d < 20; ++d)
        for (int c = -1; c <= 3; ++c) (void)conv_causal_region(d, c, &f[0], &f[1], &f[2], &f[3]);
    EXPECT(conv_causal_region(2147483647, 2, &f[0], &f[1], &f[2], &f[3]) == CONV_E_INVAL);
    EXPECT(conv_calib_mfma_bf16(nullptr, 1, 1, nullptr) == CONV_E_INVAL);
    if (fails) return 1;
    std::puts("abi driver ok");
    return 0;
}
