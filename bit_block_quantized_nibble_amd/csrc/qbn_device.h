// Device-side helpers shared by the qbn kernels (gfx950 only).
//
// Decoders here are the GPU's own: E2M1 pairs go through the gfx950 FP4
// conversion instructions, E4M3FN and E8M0 are decoded by building binary32
// bit patterns, fp16 by the hardware half->float conversion. None of this is
// shared with the CPU reference used by the tests.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qbn.h"

namespace qbn {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- E2M1
// Two E2M1 codes of byte SEL of `word` (low nibble first) -> two binary32.
// The conversion scale is 1.0, so the result is the bare codebook value
// (0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives, code 8 = -0).
template <int SEL>
__device__ __forceinline__ f32x2 e2m1x2_f32(uint32_t word) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, SEL);
}

template <int SEL>
__device__ __forceinline__ bf16x2 e2m1x2_bf16(uint32_t word) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, SEL);
}

// ---------------------------------------------------------------- E8M0
// Unbiased exponent of an E8M0 byte (valid for 0..254; 255 is NaN).
__device__ __forceinline__ int e8m0_exponent(uint32_t b) { return (int)(b & 0xFFu) - 127; }

// ---------------------------------------------------------------- E4M3FN
// E4M3FN byte -> binary32, exact for all 254 finite encodings, NaN for
// 0x7F / 0xFF. Exponent/fraction bits are placed in a binary32 pattern whose
// value is the E4M3 magnitude times 2^-120 (the E4M3 subnormals land on
// binary32 subnormals), then rescaled by the exact power 2^120.
__device__ __forceinline__ float e4m3fn_f32(uint32_t b) {
    uint32_t mag = (b & 0x7Fu) << 20;
    float v = __uint_as_float(mag) * 0x1p120f;
    v = __uint_as_float(__float_as_uint(v) | ((b & 0x80u) << 24));
    return ((b & 0x7Fu) == 0x7Fu) ? __uint_as_float(0x7FC00000u) : v;
}

// Same decode for callers that have validated the scales (no NaN select).
__device__ __forceinline__ float e4m3fn_f32_valid(uint32_t b) {
    uint32_t mag = (b & 0x7Fu) << 20;
    float v = __uint_as_float(mag) * 0x1p120f;
    return __uint_as_float(__float_as_uint(v) | ((b & 0x80u) << 24));
}

// ---------------------------------------------------------------- fp16 / bf16
__device__ __forceinline__ float f16_bits_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xFFFFu));
}

// binary32 -> bfloat16 bits, round to nearest even (gfx950 hardware convert).
__device__ __forceinline__ uint16_t bf16_bits_rne(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)bf16_bits_rne(lo) | ((uint32_t)bf16_bits_rne(hi) << 16);
}

// Reinterpret a 32-bit value as two bfloat16 / two fp16 (low half first).
// Takes the word by value: applying __builtin_bit_cast to an ext-vector
// element expression (v.y, v.z, ...) reads element 0 with this compiler.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }
__device__ __forceinline__ f16x2 as_f16x2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }

// ---------------------------------------------------------------- loads
__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ u32x2 ld8(const void *p) { return *reinterpret_cast<const u32x2 *>(p); }
__device__ __forceinline__ uint32_t ld4(const void *p) { return *reinterpret_cast<const uint32_t *>(p); }

// ---------------------------------------------------------------- DPP reductions
// Cross-lane sums with data-parallel-primitive moves (no LDS traffic). The
// disabled-row / out-of-range case reads the `old` operand, which is 0.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}

// Sum over groups of W consecutive lanes (W a power of two, 1..64). The
// group's sum is valid in its LAST lane (lane % W == W - 1); for W <= 16 every
// lane of the group holds it. Fixed order, hence deterministic.
template <int W>
__device__ __forceinline__ float group_sum_last(float v) {
    if (W >= 2) v += dpp_f32<0xB1>(v);          // quad_perm [1,0,3,2]
    if (W >= 4) v += dpp_f32<0x4E>(v);          // quad_perm [2,3,0,1]
    if (W >= 8) v += dpp_f32<0x141>(v);         // row_half_mirror
    if (W >= 16) v += dpp_f32<0x140>(v);        // row_mirror
    if (W >= 32) v += dpp_f32<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
    if (W >= 64) v += dpp_f32<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
    return v;
}

// ---------------------------------------------------------------- reductions
// Sum over groups of W consecutive lanes (W a power of two <= 64); every lane
// of a group ends with the group's sum. Fixed butterfly order: deterministic.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int off = W / 2; off > 0; off >>= 1)
        v += __shfl_xor(v, off, W);
    return v;
}

}  // namespace qbn
