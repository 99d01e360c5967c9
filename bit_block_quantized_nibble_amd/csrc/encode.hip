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
// correctly rounded).
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

// One thread per output word: the bits [32 w, 32 w + 32) of the stream of
// `width`-bit fields ((src[i] >> shift) & mask at bits i * width).
__global__ __launch_bounds__(256) void k_pack_bits(const uint8_t *__restrict__ src, int64_t count, int shift,
                                                   int width, uint32_t *__restrict__ words, int64_t nwords) {
    const int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (w >= nwords) return;
    const uint32_t mask = (1u << width) - 1u;
    const int64_t b0 = 32 * w;
    const int64_t i0 = b0 / width, i1 = min(count - 1, (b0 + 31) / width);
    uint32_t acc = 0;
    for (int64_t i = i0; i <= i1; ++i) {
        const uint32_t v = ((uint32_t)src[i] >> shift) & mask;
        const int64_t pos = i * width - b0;  // may be negative: the field started in the previous word
        acc |= pos >= 0 ? (v << pos) : (v >> (-pos));
    }
    words[w] = acc;
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

}  // namespace

hipError_t launch_quantize_nvfp4(const void *x, int x_dtype, int64_t m, int64_t k, int64_t ldx, float scale2, int tie,
                                 void *codes, void *scales, hipStream_t s) {
    const int64_t blocks = m * (k / 16);
    const dim3 grid((unsigned)((blocks + 255) / 256));
    uint8_t *c = (uint8_t *)codes, *sc = (uint8_t *)scales;
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
    const int w0 = lo > 0 ? lo : bits;
    const int64_t n0 = (count * w0 + 31) / 32;
    hipLaunchKernelGGL(k_pack_bits, dim3((unsigned)((n0 + 255) / 256)), dim3(256), 0, s, (const uint8_t *)values,
                       count, 0, w0, (uint32_t *)words_lo, n0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || lo == 0) return e;
    const int64_t n1 = (count * (bits - lo) + 31) / 32;
    hipLaunchKernelGGL(k_pack_bits, dim3((unsigned)((n1 + 255) / 256)), dim3(256), 0, s, (const uint8_t *)values,
                       count, lo, bits - lo, (uint32_t *)words_hi, n1);
    return hipGetLastError();
}

hipError_t launch_unpack_bits(const void *words_lo, const void *words_hi, int64_t count, int bits, int lo,
                              void *values, hipStream_t s) {
    hipLaunchKernelGGL(k_unpack_bits, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s,
                       (const uint32_t *)words_lo, (const uint32_t *)words_hi, count, lo > 0 ? lo : bits,
                       lo > 0 ? bits - lo : 0, (uint8_t *)values);
    return hipGetLastError();
}

}  // namespace qbn
