// Shared device-side helpers of the gfx950 convolution kernels: storage-type traits, the
// fp32 <-> fp16/bf16 conversions and the fused epilogue (bias is folded into the accumulator's
// initial value by each kernel; the epilogue is applied to the fp32 sum before the one
// round-to-nearest-even on the store).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cx {

typedef uint16_t u16;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

enum { EPI_NONE = 0, EPI_RELU = 1, EPI_CLAMP1 = 2 };

// bf16 is the upper half of an IEEE binary32.
__device__ __forceinline__ float bf16_bits_to_f32(u16 b) {
    return __uint_as_float((uint32_t)b << 16);
}
// v_cvt_pk_bf16_f32: round to nearest, ties to even (the kernels run in the default round mode
// with fp32 denormals kept), overflow gives infinity, NaN stays a quiet NaN.  Branch-free.
__device__ __forceinline__ u16 f32_to_bf16_bits(float f) {
    return __builtin_bit_cast(u16, (__bf16)f);
}
__device__ __forceinline__ float f16_bits_to_f32(u16 h) {
    return (float)__builtin_bit_cast(_Float16, h);
}
// v_cvt_f16_f32 rounds to nearest-even in the default mode; overflow gives infinity.
__device__ __forceinline__ u16 f32_to_f16_bits(float f) {
    return __builtin_bit_cast(u16, (_Float16)f);
}

// Storage-type traits: IS_BF16 selects the conversions and the matrix-core/dot instructions.
template <bool IS_BF16>
struct Elem;

template <>
struct Elem<false> {  // IEEE binary16
    typedef f16x8_t vec8;
    typedef f16x2_t vec2;
    static __device__ __forceinline__ float to_f32(u16 b) { return f16_bits_to_f32(b); }
    static __device__ __forceinline__ u16 from_f32(float f) { return f32_to_f16_bits(f); }
    static __device__ __forceinline__ f32x4_t mfma16x16x32(vec8 a, vec8 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x16_t mfma32x32x16(vec8 a, vec8 b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    // a.x*b.x + a.y*b.y + c with an fp32 accumulator
    static __device__ __forceinline__ float dot2(vec2 a, vec2 b, float c) {
        return __builtin_amdgcn_fdot2(a, b, c, false);
    }
};

template <>
struct Elem<true> {  // bfloat16
    typedef bf16x8_t vec8;
    typedef bf16x2_t vec2;
    static __device__ __forceinline__ float to_f32(u16 b) { return bf16_bits_to_f32(b); }
    static __device__ __forceinline__ u16 from_f32(float f) { return f32_to_bf16_bits(f); }
    static __device__ __forceinline__ f32x4_t mfma16x16x32(vec8 a, vec8 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x16_t mfma32x32x16(vec8 a, vec8 b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float dot2(vec2 a, vec2 b, float c) {
        return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
    }
};

// The fused epilogue on the fp32 sum (bias already included).  ReLU keeps NaN (the compare is
// false); the clamp is min(1, max(-1, v)).
template <int EPI>
__device__ __forceinline__ float epilogue(float v) {
    if constexpr (EPI == EPI_RELU) return v < 0.f ? 0.f : v;
    if constexpr (EPI == EPI_CLAMP1) return fminf(1.f, fmaxf(-1.f, v));
    return v;
}

// Remaps a linear workgroup id so that consecutive logical tiles run on the same XCD: the
// dispatcher hands workgroup i to XCD i % 8, and each XCD has its own L2.  Bijective on
// [0, total).
__device__ __forceinline__ uint32_t xcd_remap(uint32_t i, uint32_t total) {
    const uint32_t q = total / 8u, r = total % 8u;
    const uint32_t xcd = i % 8u, k = i / 8u;
    const uint32_t start = xcd < r ? xcd * (q + 1u) : r * (q + 1u) + (xcd - r) * q;
    return start + k;
}

// A value of the head's output as an 8-bit video code: clamp(RNE(127.5 * (v + 1)), 0, 255) of the
// exact value, NaN -> 0 ([-1, 1] onto [0, 255]).  For every fp16/bf16 value v (fp32 denormals
// kept) one fused multiply-add rounds the exact 127.5*v + 127.5 without moving it onto or across
// a half-integer, except for tiny v, where it lands on the tie 127.5 itself and the sign of v
// decides (checked over all 65536 patterns of both types).
__device__ __forceinline__ uint32_t rgb_code(float v) {
    const float t = __builtin_fmaf(v, 127.5f, 127.5f);
    float q = __builtin_rintf(t);
    if (v < 0.f && t == 127.5f) q = 127.f;
    q = __builtin_fmaxf(q, 0.f);     // also NaN -> 0
    q = __builtin_fminf(q, 255.f);
    return (uint32_t)q;
}

}  // namespace cx
