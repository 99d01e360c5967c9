// Bulk dequantization: materialize W_hat for all six formats, binary32 or
// bfloat16 (round to nearest even of the binary32 value), in [n][k] or
// [k][n] layout. Bit-exact with each format's rule, negative zero
// included; scale bytes that the validator rejects decode to NaN.
//
// Materializing gives back the bandwidth a fused kernel saves ("Why 4-Bit
// Quantization Is King", section 7), so this is the parity and conversion
// tool, not the GEMV route. Kernels are bandwidth-bound: each thread reads
// one natural unit of its format (a code dword, a Q4_K code dword, a Q4_0
// block, a GPTQ/AWQ word or four) and writes its outputs with the widest
// stores the layout allows; the thread -> unit mapping is chosen per output
// layout so that consecutive lanes write consecutive addresses.
#include "qbn_device.h"
#include "qbn_launch.h"

namespace qbn {
namespace {

constexpr int kBlock = 256;

// AWQ slot order: the slots of a word hold columns 0,2,4,6,1,3,5,7 of its
// group of eight ("Bit Packing Architecture", 'Real layouts compared'), so
// column c sits in slot awq_slot(c), at bit 4 * awq_slot(c).
__device__ __forceinline__ constexpr int awq_slot(int c) { return (c & 1) ? 4 + (c >> 1) : (c >> 1); }

template <bool BF16>
struct Out;
template <>
struct Out<false> {
    __device__ __forceinline__ static void put(void *out, int64_t idx, float v) { ((float *)out)[idx] = v; }
    // 4 consecutive values at idx (idx % 4 == 0)
    __device__ __forceinline__ static void put4(void *out, int64_t idx, float a, float b, float c, float d) {
        *reinterpret_cast<f32x4 *>((float *)out + idx) = f32x4{a, b, c, d};
    }
    // the same as a non-temporal store, for a wave whose lanes write one
    // contiguous run (full lines leave L2 without waiting to merge)
    __device__ __forceinline__ static void put4_nt(void *out, int64_t idx, float a, float b, float c, float d) {
        __builtin_nontemporal_store(f32x4{a, b, c, d}, reinterpret_cast<f32x4 *>((float *)out + idx));
    }
};
template <>
struct Out<true> {
    __device__ __forceinline__ static void put(void *out, int64_t idx, float v) { ((uint16_t *)out)[idx] = bf16_bits_rne(v); }
    __device__ __forceinline__ static void put4(void *out, int64_t idx, float a, float b, float c, float d) {
        *reinterpret_cast<u32x2 *>((uint16_t *)out + idx) = u32x2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
    }
    __device__ __forceinline__ static void put4_nt(void *out, int64_t idx, float a, float b, float c, float d) {
        __builtin_nontemporal_store(u32x2{pack_bf16x2(a, b), pack_bf16x2(c, d)},
                                    reinterpret_cast<u32x2 *>((uint16_t *)out + idx));
    }
};

__device__ __forceinline__ int64_t tid64() { return (int64_t)blockIdx.x * blockDim.x + threadIdx.x; }

// ------------------------------------------------------------------ MXFP4 / NVFP4
// One thread per code dword (8 elements, all in one scale group).
// LAYOUT 0: thread t -> dword t of the row-major code array, output [n][k].
// LAYOUT 1: thread t -> (row = t % n, dword column t / n), output [k][n].
template <int FMT, bool BF16, int LAYOUT>
__global__ __launch_bounds__(kBlock) void k_dequant_e2m1(const uint8_t *__restrict__ codes,
                                                          const uint8_t *__restrict__ scales, float scale2,
                                                          int64_t n, int64_t k, void *__restrict__ out) {
    const int64_t t = tid64();
    const int64_t dpr = k / 8;  // dwords per row
    if (t >= n * dpr) return;
    int64_t row, cd;
    if (LAYOUT == 0) {
        row = t / dpr;
        cd = t - row * dpr;
    } else {
        cd = t / n;
        row = t - cd * n;
    }
    const uint32_t w = ld4(codes + row * (k / 2) + 4 * cd);
    const int64_t col = 8 * cd;
    float v[8];
    const f32x2 p0 = e2m1x2_f32<0>(w), p1 = e2m1x2_f32<1>(w), p2 = e2m1x2_f32<2>(w), p3 = e2m1x2_f32<3>(w);
    v[0] = p0.x; v[1] = p0.y; v[2] = p1.x; v[3] = p1.y; v[4] = p2.x; v[5] = p2.y; v[6] = p3.x; v[7] = p3.y;
    if (FMT == QBN_MXFP4) {
        const uint32_t b = scales[row * (k / 32) + col / 32];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            v[i] = (b == 0xFFu) ? __uint_as_float(0x7FC00000u) : __builtin_amdgcn_ldexpf(v[i], e8m0_exponent(b));
    } else {
        const float s = e4m3fn_f32(scales[row * (k / 16) + col / 16]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float local = v[i] * s;  // exact: at most 6 significant bits
            v[i] = local * scale2;         // the single rounding, after the block scale
        }
    }
    if (LAYOUT == 0) {
        const int64_t o = row * k + col;
        Out<BF16>::put4(out, o, v[0], v[1], v[2], v[3]);
        Out<BF16>::put4(out, o + 4, v[4], v[5], v[6], v[7]);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) Out<BF16>::put(out, (col + i) * n + row, v[i]);
    }
}

// ------------------------------------------------------------------ Q4_K
// Scale/min pair j of the 12 metadata bytes ("Four Bits, Three Contracts",
// section 6), from the header words h.y = B[0..3], h.z = B[4..7], h.w = B[8..11].
__device__ __forceinline__ void q4k_sm(const u32x4 &h, int j, uint32_t &s, uint32_t &m) {
    if (j < 4) {
        s = (h.y >> (8 * j)) & 63u;
        m = (h.z >> (8 * j)) & 63u;
    } else {
        const int jj = j - 4;
        s = ((h.w >> (8 * jj)) & 15u) | (((h.y >> (8 * jj + 6)) & 3u) << 4);
        m = ((h.w >> (8 * jj + 4)) & 15u) | (((h.z >> (8 * jj + 6)) & 3u) << 4);
    }
}

// One thread per code dword of a super-block: dword tt (0..31) is code bytes
// 4tt..4tt+3 = 32c + l0 + {0..3} with c = tt/8, l0 = 4(tt%8); low nibbles go
// to outputs 64c + l0 + i (sub-block 2c), high nibbles to 64c + 32 + l0 + i
// (sub-block 2c+1).
// LAYOUT 0: t -> (block = t / 32, tt = t % 32); LAYOUT 1: t -> (row = t % n, rest).
template <bool BF16, int LAYOUT>
__global__ __launch_bounds__(kBlock) void k_dequant_q4k(const uint8_t *__restrict__ blocks, int64_t n, int64_t k,
                                                         void *__restrict__ out) {
    const int64_t t = tid64();
    const int64_t nb = k / 256;
    if (t >= n * nb * 32) return;
    int64_t row, b, tt;
    if (LAYOUT == 0) {
        const int64_t blk = t / 32;
        tt = t - blk * 32;
        row = blk / nb;
        b = blk - row * nb;
    } else {
        row = t % n;
        const int64_t rest = t / n;  // = b * 32 + tt
        b = rest / 32;
        tt = rest - b * 32;
    }
    const uint8_t *bp = blocks + (row * nb + b) * 144;
    const u32x4 h = ld16(bp);
    const uint32_t q = ld4(bp + 16 + 4 * tt);
    const int c = (int)(tt / 8);
    const int l0 = 4 * (int)(tt % 8);
    const float d = f16_bits_f32(h.x & 0xFFFFu);
    const float dmin = f16_bits_f32(h.x >> 16);
    uint32_t s_lo, m_lo, s_hi, m_hi;
    q4k_sm(h, 2 * c, s_lo, m_lo);
    q4k_sm(h, 2 * c + 1, s_hi, m_hi);
    const float step_lo = d * (float)s_lo, off_lo = dmin * (float)m_lo;  // exact products
    const float step_hi = d * (float)s_hi, off_hi = dmin * (float)m_hi;
    float lo[4], hi[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t byte = (q >> (8 * i)) & 0xFFu;
        lo[i] = __builtin_fmaf(step_lo, (float)(byte & 15u), -off_lo);
        hi[i] = __builtin_fmaf(step_hi, (float)(byte >> 4), -off_hi);
    }
    const int64_t col = 256 * b + 64 * c + l0;
    if (LAYOUT == 0) {
        Out<BF16>::put4(out, row * k + col, lo[0], lo[1], lo[2], lo[3]);
        Out<BF16>::put4(out, row * k + col + 32, hi[0], hi[1], hi[2], hi[3]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            Out<BF16>::put(out, (col + i) * n + row, lo[i]);
            Out<BF16>::put(out, (col + 32 + i) * n + row, hi[i]);
        }
    }
}

// ------------------------------------------------------------------ Q4_0
// One thread per 18-byte block: fp16 d, byte j = element j (low) | j+16 (high),
// w = d * (q - 8) ("Bit Packing Architecture", 'Real layouts compared').
template <bool BF16, int LAYOUT>
__global__ __launch_bounds__(kBlock) void k_dequant_q4_0(const uint8_t *__restrict__ blocks, int64_t n, int64_t k,
                                                          void *__restrict__ out) {
    const int64_t t = tid64();
    const int64_t nb = k / 32;
    if (t >= n * nb) return;
    int64_t row, b;
    if (LAYOUT == 0) {
        row = t / nb;
        b = t - row * nb;
    } else {
        row = t % n;
        b = t / n;
    }
    const uint16_t *bp = reinterpret_cast<const uint16_t *>(blocks + (row * nb + b) * 18);
    const float d = f16_bits_f32(bp[0]);
    float v[32];
#pragma unroll
    for (int h = 0; h < 8; ++h) {
        const uint32_t pair = bp[1 + h];  // bytes 2h and 2h+1 of the code area
        v[2 * h] = d * (float)((int)(pair & 15u) - 8);
        v[2 * h + 16] = d * (float)((int)((pair >> 4) & 15u) - 8);
        v[2 * h + 1] = d * (float)((int)((pair >> 8) & 15u) - 8);
        v[2 * h + 17] = d * (float)((int)((pair >> 12) & 15u) - 8);
    }
    const int64_t col = 32 * b;
    if (LAYOUT == 0) {
#pragma unroll
        for (int i = 0; i < 32; i += 4) Out<BF16>::put4(out, row * k + col + i, v[i], v[i + 1], v[i + 2], v[i + 3]);
    } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) Out<BF16>::put(out, (col + i) * n + row, v[i]);
    }
}

// ------------------------------------------------------------------ GPTQ / AWQ
// GPTQ word (r, c) holds rows 8r..8r+7 of column c; AWQ word (kk, g) holds
// columns 8g..8g+7 of row kk in slot order. w = s * (q - z), exact.
// GPTQ: a thread takes VEC adjacent words of one word-row (VEC columns).
template <bool BF16, int LAYOUT, int VEC>
__global__ __launch_bounds__(kBlock) void k_dequant_gptq(const uint32_t *__restrict__ qw,
                                                          const uint16_t *__restrict__ scales,
                                                          const uint8_t *__restrict__ zeros, int64_t n, int64_t k,
                                                          int64_t group, void *__restrict__ out) {
    const int64_t t = tid64();
    const int64_t nv = n / VEC;
    if (t >= (k / 8) * nv) return;
    const int64_t r = t / nv;
    const int64_t c0 = (t - r * nv) * VEC;
    const int64_t gi = (8 * r) / group;  // all 8 rows share a group (group % 8 == 0)
    uint32_t wd[VEC];
    float s[VEC], z[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
        wd[v] = qw[r * n + c0 + v];
        s[v] = f16_bits_f32(scales[gi * n + c0 + v]);
        z[v] = (float)zeros[gi * n + c0 + v];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float o[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) o[v] = s[v] * ((float)((wd[v] >> (4 * j)) & 15u) - z[v]);
        const int64_t kk = 8 * r + j;
        if (LAYOUT == 1) {
            if (VEC == 4) {
                // lanes hold neighbouring column quads: each store is one
                // contiguous run (23.3 -> 18.4 us for 4096 x 11008 to bf16)
                Out<BF16>::put4_nt(out, kk * n + c0, o[0], o[1], o[2], o[3]);
            } else {
#pragma unroll
                for (int v = 0; v < VEC; ++v) Out<BF16>::put(out, kk * n + c0 + v, o[v]);
            }
        } else {
#pragma unroll
            for (int v = 0; v < VEC; ++v) Out<BF16>::put(out, (c0 + v) * k + kk, o[v]);
        }
    }
}

template <bool BF16, int LAYOUT>
__global__ __launch_bounds__(kBlock) void k_dequant_awq(const uint32_t *__restrict__ qw,
                                                         const uint16_t *__restrict__ scales,
                                                         const uint8_t *__restrict__ zeros, int64_t n, int64_t k,
                                                         int64_t group, void *__restrict__ out) {
    const int64_t t = tid64();
    const int64_t ng = n / 8;
    if (t >= k * ng) return;
    const int64_t kk = t / ng;
    const int64_t g = t - kk * ng;
    const uint32_t wd = qw[kk * ng + g];
    const int64_t gi = kk / group;
    float o[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int64_t col = 8 * g + c;
        const float s = f16_bits_f32(scales[gi * n + col]);
        const float z = (float)zeros[gi * n + col];
        o[c] = s * ((float)((wd >> (4 * awq_slot(c))) & 15u) - z);
    }
    if (LAYOUT == 1) {
        Out<BF16>::put4(out, kk * n + 8 * g, o[0], o[1], o[2], o[3]);
        Out<BF16>::put4(out, kk * n + 8 * g + 4, o[4], o[5], o[6], o[7]);
    } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) Out<BF16>::put(out, (8 * g + c) * k + kk, o[c]);
    }
}

template <typename K, typename... A>
hipError_t launch1d(K kern, int64_t threads, hipStream_t s, A... args) {
    if (threads <= 0) return hipSuccess;
    const int64_t grid = (threads + kBlock - 1) / kBlock;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kBlock), 0, s, args...);
    return hipGetLastError();
}

template <bool BF16, int LAYOUT>
hipError_t dequant_typed(const qbn_tensor &w, void *out, hipStream_t s) {
    const uint8_t *d8 = (const uint8_t *)w.data;
    switch (w.format) {
    case QBN_MXFP4:
        return launch1d(k_dequant_e2m1<QBN_MXFP4, BF16, LAYOUT>, w.n * (w.k / 8), s, d8, (const uint8_t *)w.scales,
                        w.scale2, w.n, w.k, out);
    case QBN_NVFP4:
        return launch1d(k_dequant_e2m1<QBN_NVFP4, BF16, LAYOUT>, w.n * (w.k / 8), s, d8, (const uint8_t *)w.scales,
                        w.scale2, w.n, w.k, out);
    case QBN_Q4_K:
        return launch1d(k_dequant_q4k<BF16, LAYOUT>, w.n * (w.k / 256) * 32, s, d8, w.n, w.k, out);
    case QBN_Q4_0:
        return launch1d(k_dequant_q4_0<BF16, LAYOUT>, w.n * (w.k / 32), s, d8, w.n, w.k, out);
    case QBN_GPTQ4: {
        const bool vec4 = (w.n % 4 == 0) && LAYOUT == 1;
        if (vec4)
            return launch1d(k_dequant_gptq<BF16, LAYOUT, 4>, (w.k / 8) * (w.n / 4), s, (const uint32_t *)w.data,
                            (const uint16_t *)w.scales, (const uint8_t *)w.zeros, w.n, w.k, (int64_t)w.group, out);
        return launch1d(k_dequant_gptq<BF16, LAYOUT, 1>, (w.k / 8) * w.n, s, (const uint32_t *)w.data,
                        (const uint16_t *)w.scales, (const uint8_t *)w.zeros, w.n, w.k, (int64_t)w.group, out);
    }
    case QBN_AWQ4:
        return launch1d(k_dequant_awq<BF16, LAYOUT>, w.k * (w.n / 8), s, (const uint32_t *)w.data,
                        (const uint16_t *)w.scales, (const uint8_t *)w.zeros, w.n, w.k, (int64_t)w.group, out);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_dequant(const qbn_tensor &w, void *out, int out_dtype, int out_layout, hipStream_t s) {
    const bool bf = (out_dtype == QBN_BF16);
    if (out_layout == 0) return bf ? dequant_typed<true, 0>(w, out, s) : dequant_typed<false, 0>(w, out, s);
    return bf ? dequant_typed<true, 1>(w, out, s) : dequant_typed<false, 1>(w, out, s);
}

}  // namespace qbn
