// Encode side: the step before the hot path.
//   NVFP4 quantizer ("Why 4-Bit Quantization Is King" section 5:
//     x = q_E2M1 * s_block(E4M3) * s_global; the Muser chapter section 7.2
//     pins the E2M1 rounding to ModelOpt's ties-to-even midpoints; "Four
//     Bits, Three Contracts" section 2 uses the lowest code on a tie):
//     per block of 16, s = E4M3FN(amax / (6 scale2)), t = s * scale2,
//     code = E2M1(x / t) with the chosen tie rule, all in binary32.
//   Signed INT4 symmetric ("Why 4-Bit Quantization Is King" section 1):
//     s = amax / 7 per group, q = clip(round_half_even(w / s), -8, 7),
//     two's-complement nibbles, the earlier element in the low nibble.
//   b-bit packing ("Bit Packing Architecture", "The packing arithmetic" and
//     "Odd widths"): element i at bits [i b, i b + b) of a little-endian
//     stream of 32-bit words, straddling words when b does not divide 32;
//     or split into two planes (the low `lo` bits and the high b - lo bits,
//     each its own stream, as GGUF's Q6_K keeps 4 + 2).
// Every output is bit-exact with the definitions (IEEE binary32 division,
// correctly rounded); the lane kernels reach the same codes with a division
// only next to a rounding boundary (the bracket below).
#include <algorithm>

#include "qbn_device.h"
#include "qbn_launch.h"

namespace qbn {
namespace {

template <typename XT>
__device__ __forceinline__ float load_elem(const XT *p);
template <>
__device__ __forceinline__ float load_elem<float>(const float *p) {
    return *p;
}
template <>
__device__ __forceinline__ float load_elem<__bf16>(const __bf16 *p) {
    return __builtin_bit_cast(float, (uint32_t)*reinterpret_cast<const uint16_t *>(p) << 16);
}

// Division-free codes for the lane kernels. A code that depends on q =
// fl(v / d) through a non-decreasing map C (round half even then clip for
// INT4, the E2M1 code for NVFP4) is taken from x = fl(v * fl(1 / d)), which
// lies within 3 ulp of q: when C(fl(x * kBelow)) == C(fl(x * kAbove)), the
// two ends bracket q (the margin of 2^-20 relative is 16 ulp) and C(q) is
// that common value. Otherwise (INT4: that element; NVFP4: that pair), or
// for every element when 1 / d overflows, the code comes from the correctly
// rounded quotient. Exact ties (a quotient on a rounding boundary) always
// take that path; with bf16 weights they are common (a group whose amax has
// a mantissa divisible by 7 puts many weights on half-integers).
constexpr float kBelow = 1.0f - 0x1p-20f, kAbove = 1.0f + 0x1p-20f;

// Maximum over groups of L consecutive lanes (L a power of two <= 64), in
// every lane of the group: DPP moves inside a row of 16 (quad swaps, then
// the half-row and row mirrors), shuffles across rows. Max is exact, so the
// order does not matter. The lanes of a group are active together.
template <int L>
__device__ __forceinline__ float group_max(float a) {
    if (L >= 2) a = __builtin_fmaxf(a, dpp_f32<0xB1>(a));   // quad_perm [1,0,3,2]
    if (L >= 4) a = __builtin_fmaxf(a, dpp_f32<0x4E>(a));   // quad_perm [2,3,0,1]
    if (L >= 8) a = __builtin_fmaxf(a, dpp_f32<0x141>(a));  // row_half_mirror
    if (L >= 16) a = __builtin_fmaxf(a, dpp_f32<0x140>(a)); // row_mirror
    if (L >= 32) a = __builtin_fmaxf(a, __shfl_xor(a, 16, 64));
    if (L >= 64) a = __builtin_fmaxf(a, __shfl_xor(a, 32, 64));
    return a;
}

// Eight consecutive elements as binary32 from one (bf16) or two (f32) 16-byte
// loads; p must be 16-byte aligned. The weights are read once: non-temporal
// loads (the NVFP4 encoder 3% faster, the INT4 one 1%).
template <typename XT>
__device__ __forceinline__ void load8(const XT *p, float v[8]) {
    if constexpr (sizeof(XT) == 2) {
        const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = __builtin_bit_cast(float, q[j] << 16);
            v[2 * j + 1] = __builtin_bit_cast(float, q[j] & 0xFFFF0000u);
        }
    } else {
        const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
        const u32x4 b = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p + 4));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // through plain words: a bit cast taken of a vector element
            // itself reads element 0 whatever the index
            const uint32_t wa = a[j], wb = b[j];
            v[j] = __builtin_bit_cast(float, wa);
            v[4 + j] = __builtin_bit_cast(float, wb);
        }
    }
}

// E2M1 code of v: magnitude saturated at 6, then the number of grid
// midpoints (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5) below it; an exact
// midpoint between codes c and c + 1 goes up when TIE_EVEN and c + 1 is
// even, else stays at c (the lowest code). The sign bit follows v.
template <bool TIE_EVEN>
__device__ __forceinline__ uint32_t e2m1_code(float v) {
    const float a = __builtin_fminf(__builtin_fabsf(v), 6.0f);
    constexpr float mid[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < 7; ++i) c += (a > mid[i] || (TIE_EVEN && (i & 1) && a == mid[i])) ? 1u : 0u;
    return c | (__builtin_signbit(v) ? 8u : 0u);
}

// The 32-bit word of the E2M1 codes of q[0..7], element j at bits 4j. Ties
// to even through the hardware conversion (scale 1: nearest, ties to the
// even code, finite magnitudes past 6 saturate, the sign kept, also on a
// zero: the code e2m1_code<true> gives; byte b takes elements 2b and 2b + 1,
// low nibble first), else e2m1_code<false> per element.
template <bool TIE_EVEN, bool CLIP = true>
__device__ __forceinline__ uint32_t e2m1_word(const float q[8]) {
    uint32_t w = 0;
    if constexpr (TIE_EVEN) {
        // CLIP: magnitudes clipped at 6 first (the same code), so that an
        // infinite quotient saturates too; without it q must be finite
        float c[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = CLIP ? __builtin_copysignf(__builtin_fminf(__builtin_fabsf(q[j]), 6.0f), q[j]) : q[j];
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, c[0], c[1], 1.0f, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, c[2], c[3], 1.0f, 1);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, c[4], c[5], 1.0f, 2);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, c[6], c[7], 1.0f, 3);
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) w |= e2m1_code<false>(q[j]) << (4 * j);
    }
    return w;
}

// E4M3FN byte of q >= 0 (finite): nearest, ties to even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3fn_byte(float q) {
    typedef short v2s __attribute__((ext_vector_type(2)));
    v2s r = {0, 0};
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, __builtin_fminf(q, 448.0f), 0.0f, 1.0f, false);
    return (uint32_t)(uint16_t)r[0] & 0x7Fu;
}

// One thread per 16-element block.
template <typename XT, bool TIE_EVEN>
__global__ __launch_bounds__(256) void k_quantize_nvfp4(const XT *__restrict__ x, int64_t m, int64_t k, int64_t ldx,
                                                        float scale2, uint8_t *__restrict__ codes,
                                                        uint8_t *__restrict__ scales) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t nb = k / 16;
    if (t >= m * nb) return;
    const int64_t row = t / nb, b = t - row * nb;
    const XT *p = x + row * ldx + 16 * b;
    float v[16];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        v[j] = load_elem<XT>(p + j);
        amax = __builtin_fmaxf(amax, __builtin_fabsf(v[j]));
    }
    const float den = 6.0f * scale2;
    const uint32_t sb = e4m3fn_byte(amax / den);
    scales[t] = (uint8_t)sb;
    const float tt = e4m3fn_f32(sb) * scale2;
    uint32_t w[2] = {0u, 0u};
    if (tt != 0.0f) {
#pragma unroll
        for (int j = 0; j < 16; ++j) w[j / 8] |= e2m1_code<TIE_EVEN>(v[j] / tt) << (4 * (j % 8));
    }
    *reinterpret_cast<u32x2 *>(codes + row * (k / 2) + 8 * b) = u32x2{w[0], w[1]};
}

// Two lanes per 16-element block, eight elements per lane from 16-byte
// loads: the block amax is one DPP swap away, the even lane stores the
// scale byte and each lane the 32-bit word of its eight codes. The same
// scale bytes and codes as the one-thread-per-block kernel.
template <typename XT, bool TIE_EVEN, bool DENSE>
__global__ __launch_bounds__(256) void k_quantize_nvfp4_lanes(const XT *__restrict__ x, int64_t m, int64_t k,
                                                              int64_t ldx, float scale2, uint8_t *__restrict__ codes,
                                                              uint8_t *__restrict__ scales) {
    const int64_t per_row = k / 8, total = m * per_row, stride = (int64_t)gridDim.x * 256;
    // t counts 8-element pieces: code word at byte 4t, block t / 2 (both
    // lanes of a block iterate together: the stride is even)
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total; t += stride) {
        float v[8];
        if (DENSE) {
            load8(x + 8 * t, v);
        } else {
            const int64_t row = t / per_row;
            load8(x + row * ldx + 8 * (t - row * per_row), v);
        }
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[j]));
        amax = group_max<2>(amax);
        const float den = 6.0f * scale2;
        const uint32_t sb = e4m3fn_byte(amax / den);
        if ((t & 1) == 0) scales[t / 2] = (uint8_t)sb;
        const float tt = e4m3fn_f32(sb) * scale2;
        uint32_t word = 0;
        if (tt != 0.0f) {
            const float inv = 1.0f / tt;
            // uniform over the block: 1 / t overflows, or some bracket end
            // v * (1 / t) * (1 + 2^-20) would not be finite (|v| <= amax)
            const bool all_exact = !(amax * inv * kAbove < __builtin_huge_valf());
            float lo[8], hi[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float q = v[j] * inv;
                lo[j] = q * kBelow;
                hi[j] = q * kAbove;
            }
            word = e2m1_word<TIE_EVEN, false>(lo);
            const uint32_t diff = all_exact ? ~0u : word ^ e2m1_word<TIE_EVEN, false>(hi);
            if (diff != 0u) {  // some pair next to a code boundary: those pairs from the exact quotients
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    if ((diff >> (8 * b)) & 0xFFu) {
                        float q[8];
#pragma unroll
                        for (int j = 0; j < 8; ++j) q[j] = 0.0f;
                        q[2 * b] = v[2 * b] / tt;
                        q[2 * b + 1] = v[2 * b + 1] / tt;
                        const uint32_t e = e2m1_word<TIE_EVEN>(q);
                        word = (word & ~(0xFFu << (8 * b))) | (e & (0xFFu << (8 * b)));
                    }
                }
            }
        }
        __builtin_nontemporal_store(word, reinterpret_cast<uint32_t *>(codes) + t);  // one contiguous run per wave
    }
}

// One thread per group.
template <typename XT>
__global__ __launch_bounds__(256) void k_quantize_int4_sym(const XT *__restrict__ w, int64_t m, int64_t k,
                                                           int64_t ldw, int64_t group, uint8_t *__restrict__ codes,
                                                           float *__restrict__ scales) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t ng = k / group;
    if (t >= m * ng) return;
    const int64_t row = t / ng, g = t - row * ng;
    const XT *p = w + row * ldw + group * g;
    float amax = 0.0f;
    for (int64_t j = 0; j < group; ++j) amax = __builtin_fmaxf(amax, __builtin_fabsf(load_elem<XT>(p + j)));
    const float s = amax / 7.0f;
    scales[t] = s;
    uint8_t *out = codes + row * (k / 2) + (group * g) / 2;
    for (int64_t j = 0; j < group; j += 2) {
        uint32_t nib[2] = {0u, 0u};
        if (s != 0.0f) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float r = __builtin_rintf(load_elem<XT>(p + j + h) / s);
                nib[h] = (uint32_t)(int)__builtin_fminf(__builtin_fmaxf(r, -8.0f), 7.0f) & 15u;
            }
        }
        out[j / 2] = (uint8_t)(nib[0] | (nib[1] << 4));
    }
}

// L = group / 8 consecutive lanes per group (L a power of two <= 64, so a
// group never straddles a wave), eight consecutive elements per lane: the
// lanes load 16- or 32-byte pieces of the row side by side, take the group's
// amax across the L-lane segment (group_max), and each stores the 32-bit
// word of its eight nibbles. The same scales and codes as the one-thread-per-group kernel.
template <typename XT, int L, bool DENSE>
__global__ __launch_bounds__(256) void k_quantize_int4_sym_lanes(const XT *__restrict__ w, int64_t m, int64_t k,
                                                                 int64_t ldw, uint8_t *__restrict__ codes,
                                                                 float *__restrict__ scales) {
    const int64_t per_row = k / 8, total = m * per_row, stride = (int64_t)gridDim.x * 256;
    // t counts 8-element pieces; the code word of piece t sits at byte 4t and
    // its group is t / L (per_row is a multiple of L). The stride is a
    // multiple of L, so the L lanes of a group always iterate together.
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total; t += stride) {
        float v[8];
        if (DENSE) {
            load8(w + 8 * t, v);
        } else {
            const int64_t row = t / per_row;
            load8(w + row * ldw + 8 * (t - row * per_row), v);
        }
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[j]));
        amax = group_max<L>(amax);
        const float s = amax / 7.0f;
        if ((t & (L - 1)) == 0) scales[t / L] = s;
        uint32_t word = 0;
        if (s != 0.0f) {
            const float inv = 1.0f / s;
            const bool all_exact = !(inv < __builtin_huge_valf());  // uniform over the group
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float x = v[j] * inv;
                float r = __builtin_rintf(x * kBelow);
                if (all_exact || r != __builtin_rintf(x * kAbove)) r = __builtin_rintf(v[j] / s);
                word |= ((uint32_t)(int)__builtin_fminf(__builtin_fmaxf(r, -8.0f), 7.0f) & 15u) << (4 * j);
            }
        }
        __builtin_nontemporal_store(word, reinterpret_cast<uint32_t *>(codes) + t);  // one contiguous run per wave
    }
}

// One thread per 32 values, whose W-bit fields (shift..shift + W - 1 of each
// byte; shift + W <= 8) fill exactly the W whole words W t .. W t + W - 1 of
// the stream, so threads share no word. Values past `count` count as 0 (the
// unused high bits of the last word). VEC: the 32 bytes are read as two
// 16-byte loads (base 16-byte aligned, all 32 in range).
template <int W, bool VEC>
__global__ __launch_bounds__(256) void k_pack_bits(const uint8_t *__restrict__ src, int64_t count, int shift,
                                                   uint32_t *__restrict__ words, int64_t nwords) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t i0 = 32 * t;
    if (i0 >= count) return;
    uint32_t b[8];
    if (VEC && i0 + 32 <= count) {
        const u32x4 lo = ld16(src + i0), hi = ld16(src + i0 + 16);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            b[j] = lo[j];
            b[4 + j] = hi[j];
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) b[j] = 0u;
#pragma unroll
        for (int i = 0; i < 32; ++i)
            if (i0 + i < count) b[i / 4] |= (uint32_t)src[i0 + i] << (8 * (i % 4));
    }
    constexpr uint32_t mask = (1u << W) - 1u;
    uint32_t out[W];
#pragma unroll
    for (int j = 0; j < W; ++j) out[j] = 0u;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const uint32_t v = (b[i / 4] >> (8 * (i % 4) + shift)) & mask;
        const int pos = i * W, wd = pos / 32, off = pos % 32;
        out[wd] |= v << off;
        if (off + W > 32) out[wd + 1] |= v >> (32 - off);
    }
#pragma unroll
    for (int j = 0; j < W; ++j)
        if (W * t + j < nwords) words[W * t + j] = out[j];
}

// One thread per element: the lo-bit field of stream a and, when hi_width >
// 0, the hi_width-bit field of stream b above it.
__global__ __launch_bounds__(256) void k_unpack_bits(const uint32_t *__restrict__ a, const uint32_t *__restrict__ b,
                                                     int64_t count, int lo_width, int hi_width,
                                                     uint8_t *__restrict__ dst) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= count) return;
    auto field = [](const uint32_t *s, int64_t i, int width) {
        const int64_t pos = i * width;
        const int64_t w = pos / 32;
        const int off = (int)(pos % 32);
        uint32_t v = s[w] >> off;
        if (off + width > 32) v |= s[w + 1] << (32 - off);
        return v & ((1u << width) - 1u);
    };
    uint32_t v = field(a, i, lo_width);
    if (hi_width > 0) v |= field(b, i, hi_width) << lo_width;
    dst[i] = (uint8_t)v;
}

// Grid of the grid-stride lane kernels: enough 256-thread workgroups to fill
// every CU at full occupancy (8 per CU), fewer for a small input.
dim3 lane_grid(int64_t pieces) { return dim3((unsigned)std::min<int64_t>((pieces + 255) / 256, 256 * 8)); }

template <typename XT, bool DENSE>
void launch_int4_sym_lanes_d(int64_t lanes, hipStream_t s, const XT *w, int64_t m, int64_t k, int64_t ldw,
                             uint8_t *codes, float *scales) {
    const dim3 g = lane_grid(m * (k / 8));
#define QBN_I4L(L) \
    hipLaunchKernelGGL((k_quantize_int4_sym_lanes<XT, L, DENSE>), g, dim3(256), 0, s, w, m, k, ldw, codes, scales)
    switch (lanes) {
        case 1: QBN_I4L(1); break;
        case 2: QBN_I4L(2); break;
        case 4: QBN_I4L(4); break;
        case 8: QBN_I4L(8); break;
        case 16: QBN_I4L(16); break;
        case 32: QBN_I4L(32); break;
        default: QBN_I4L(64); break;
    }
#undef QBN_I4L
}

template <typename XT>
hipError_t launch_int4_sym_lanes(int64_t lanes, hipStream_t s, const XT *w, int64_t m, int64_t k, int64_t ldw,
                                 uint8_t *codes, float *scales) {
    if (ldw == k || m == 1)
        launch_int4_sym_lanes_d<XT, true>(lanes, s, w, m, k, ldw, codes, scales);
    else
        launch_int4_sym_lanes_d<XT, false>(lanes, s, w, m, k, ldw, codes, scales);
    return hipGetLastError();
}

template <typename XT>
void launch_nvfp4_lanes(bool dense, bool tie_even, hipStream_t s, const XT *x, int64_t m, int64_t k, int64_t ldx,
                        float scale2, uint8_t *c, uint8_t *sc) {
    const dim3 g = lane_grid(m * (k / 8));
#define QBN_NVL(T, D) hipLaunchKernelGGL((k_quantize_nvfp4_lanes<XT, T, D>), g, dim3(256), 0, s, x, m, k, ldx, scale2, c, sc)
    if (dense) {
        if (tie_even) QBN_NVL(true, true); else QBN_NVL(false, true);
    } else {
        if (tie_even) QBN_NVL(true, false); else QBN_NVL(false, false);
    }
#undef QBN_NVL
}

template <bool VEC>
void launch_pack_width(int width, dim3 g, hipStream_t s, const uint8_t *src, int64_t count, int shift,
                       uint32_t *words, int64_t nwords) {
#define QBN_PK(W) hipLaunchKernelGGL((k_pack_bits<W, VEC>), g, dim3(256), 0, s, src, count, shift, words, nwords)
    switch (width) {
        case 1: QBN_PK(1); break;
        case 2: QBN_PK(2); break;
        case 3: QBN_PK(3); break;
        case 4: QBN_PK(4); break;
        case 5: QBN_PK(5); break;
        case 6: QBN_PK(6); break;
        case 7: QBN_PK(7); break;
        default: QBN_PK(8); break;
    }
#undef QBN_PK
}

hipError_t pack_stream(const uint8_t *src, int64_t count, int shift, int width, uint32_t *words, hipStream_t s) {
    const int64_t nwords = (count * width + 31) / 32;
    const dim3 g((unsigned)(((count + 31) / 32 + 255) / 256));
    if (reinterpret_cast<uintptr_t>(src) % 16 == 0)
        launch_pack_width<true>(width, g, s, src, count, shift, words, nwords);
    else
        launch_pack_width<false>(width, g, s, src, count, shift, words, nwords);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_nvfp4(const void *x, int x_dtype, int64_t m, int64_t k, int64_t ldx, float scale2, int tie,
                                 void *codes, void *scales, hipStream_t s) {
    const int64_t blocks = m * (k / 16);
    uint8_t *c = (uint8_t *)codes, *sc = (uint8_t *)scales;
    const int eb = x_dtype == QBN_BF16 ? 2 : 4;
    if ((ldx * eb) % 16 == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0) {  // 16-byte rows and base
        const bool dense = ldx == k || m == 1;
        if (x_dtype == QBN_BF16)
            launch_nvfp4_lanes<__bf16>(dense, tie == 0, s, (const __bf16 *)x, m, k, ldx, scale2, c, sc);
        else
            launch_nvfp4_lanes<float>(dense, tie == 0, s, (const float *)x, m, k, ldx, scale2, c, sc);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((blocks + 255) / 256));
    if (x_dtype == QBN_BF16) {
        if (tie == 0)
            hipLaunchKernelGGL((k_quantize_nvfp4<__bf16, true>), grid, dim3(256), 0, s, (const __bf16 *)x, m, k, ldx,
                               scale2, c, sc);
        else
            hipLaunchKernelGGL((k_quantize_nvfp4<__bf16, false>), grid, dim3(256), 0, s, (const __bf16 *)x, m, k,
                               ldx, scale2, c, sc);
    } else {
        if (tie == 0)
            hipLaunchKernelGGL((k_quantize_nvfp4<float, true>), grid, dim3(256), 0, s, (const float *)x, m, k, ldx,
                               scale2, c, sc);
        else
            hipLaunchKernelGGL((k_quantize_nvfp4<float, false>), grid, dim3(256), 0, s, (const float *)x, m, k, ldx,
                               scale2, c, sc);
    }
    return hipGetLastError();
}

hipError_t launch_quantize_int4_sym(const void *w, int w_dtype, int64_t m, int64_t k, int64_t ldw, int64_t group,
                                    void *codes, float *scales, hipStream_t s) {
    const int64_t groups = m * (k / group);
    const int64_t lanes = group / 8;
    const int eb = w_dtype == QBN_BF16 ? 2 : 4;
    // the lane kernel: group = 8 L with L a power of two <= 64, 16-byte rows
    // and base (vector loads), 4-byte code rows (k % 8 == 0 follows)
    if (group % 8 == 0 && lanes <= 64 && (lanes & (lanes - 1)) == 0 && (ldw * eb) % 16 == 0 &&
        reinterpret_cast<uintptr_t>(w) % 16 == 0 && reinterpret_cast<uintptr_t>(codes) % 4 == 0) {
        if (w_dtype == QBN_BF16)
            return launch_int4_sym_lanes<__bf16>(lanes, s, (const __bf16 *)w, m, k, ldw, (uint8_t *)codes, scales);
        return launch_int4_sym_lanes<float>(lanes, s, (const float *)w, m, k, ldw, (uint8_t *)codes, scales);
    }
    const dim3 grid((unsigned)((groups + 255) / 256));
    if (w_dtype == QBN_BF16)
        hipLaunchKernelGGL(k_quantize_int4_sym<__bf16>, grid, dim3(256), 0, s, (const __bf16 *)w, m, k, ldw, group,
                           (uint8_t *)codes, scales);
    else
        hipLaunchKernelGGL(k_quantize_int4_sym<float>, grid, dim3(256), 0, s, (const float *)w, m, k, ldw, group,
                           (uint8_t *)codes, scales);
    return hipGetLastError();
}

hipError_t launch_pack_bits(const void *values, int64_t count, int bits, int lo, void *words_lo, void *words_hi,
                            hipStream_t s) {
    const uint8_t *v = (const uint8_t *)values;
    hipError_t e = pack_stream(v, count, 0, lo > 0 ? lo : bits, (uint32_t *)words_lo, s);
    if (e != hipSuccess || lo == 0) return e;
    return pack_stream(v, count, lo, bits - lo, (uint32_t *)words_hi, s);
}

hipError_t launch_unpack_bits(const void *words_lo, const void *words_hi, int64_t count, int bits, int lo,
                              void *values, hipStream_t s) {
    hipLaunchKernelGGL(k_unpack_bits, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s,
                       (const uint32_t *)words_lo, (const uint32_t *)words_hi, count, lo > 0 ? lo : bits,
                       lo > 0 ? bits - lo : 0, (uint8_t *)values);
    return hipGetLastError();
}

}  // namespace qbn
