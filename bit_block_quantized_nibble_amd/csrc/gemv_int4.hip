// Decode GEMV straight from the integer int4 layouts ("Bit Packing
// Architecture", "Real layouts compared"; the GPTQ / AWQ / Q4_0 rows of the
// adjacent-formats list):
//   GPTQ4 / AWQ4: y[c] = sum_k s[k/g][c] * (q[k][c] - z[k/g][c]) * x[k], the
//     weight stored input-major (K x N logical matrix; GPTQ packs 8 k per
//     int32 word of one column, AWQ 8 columns per word of one k, in the slot
//     order 0,2,4,6,1,3,5,7);
//   Q4_0: y[r] = sum_b d_b * sum_j (q_j - 8) * x[32 b + j], rows of 18-byte
//     blocks (fp16 d, byte j = element j low | element j + 16 high).
// The integer difference q - z (or q - 8) is exact in binary32; the group
// scale multiplies each group's partial sum once. Reductions run in a fixed
// order (DPP / shuffles / LDS), so results are deterministic.
#include "qbn_device.h"
#include "qbn_launch.h"

namespace qbn {
namespace {

template <typename XT>
struct X8;  // eight consecutive activations as binary32
template <>
struct X8<float> {
    __device__ __forceinline__ static void at(const float *x, int64_t k, float (&v)[8]) {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(x + k);
        const f32x4 b = *reinterpret_cast<const f32x4 *>(x + k + 4);
        v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
    }
};
template <>
struct X8<__bf16> {
    __device__ __forceinline__ static void at(const __bf16 *x, int64_t k, float (&v)[8]) {
        const u32x4 w = ld16(x + k);
        const uint32_t p[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __builtin_bit_cast(float, p[i] << 16);
            v[2 * i + 1] = __builtin_bit_cast(float, p[i] & 0xFFFF0000u);
        }
    }
};

// Byte B of a word as binary32 (one v_cvt_f32_ubyteB).
template <int B>
__device__ __forceinline__ float ubyte(uint32_t w) {
    return (float)((w >> (8 * B)) & 0xFFu);
}

// The eight 4-bit codes of a word as binary32, in nibble order.
__device__ __forceinline__ void nibbles_f32(uint32_t w, float (&q)[8]) {
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    q[0] = ubyte<0>(lo);
    q[1] = ubyte<0>(hi);
    q[2] = ubyte<1>(lo);
    q[3] = ubyte<1>(hi);
    q[4] = ubyte<2>(lo);
    q[5] = ubyte<2>(hi);
    q[6] = ubyte<3>(lo);
    q[7] = ubyte<3>(hi);
}

// ------------------------------------------------------------------ GPTQ / AWQ
// A workgroup covers 32 columns (4 lanes x 8 columns) and all of K, split
// into 64 slices of whole 8-row steps; each lane keeps 8 column sums.
constexpr int kAffCW = 4, kAffSL = 64;

// VEC: the 8 columns of a lane are loaded as 16-byte (codes, scales) and
// 8-byte (zeros) vectors; needs n % 8 == 0 and 16-byte aligned data and
// scales. Otherwise element loads with columns past n clamped (not stored).
template <int FMT, typename XT, bool VEC>
__global__ __launch_bounds__(256) void k_gemv_affine(const uint32_t *__restrict__ qw, const uint16_t *__restrict__ sc,
                                                     const uint8_t *__restrict__ zp, const XT *__restrict__ x,
                                                     float *__restrict__ y, int64_t n, int64_t k, int64_t group) {
    __shared__ float red[4][kAffCW][8];
    const int t = threadIdx.x;
    const int cw = t % kAffCW, sl = t / kAffCW;
    const int64_t c0 = (int64_t)blockIdx.x * (8 * kAffCW) + 8 * cw;
    const int64_t nsteps = k / 8, per = (nsteps + kAffSL - 1) / kAffSL;
    const int64_t j0 = sl * per, j1 = min(nsteps, j0 + per);
    int64_t cc[8];  // clamped columns (element loads)
#pragma unroll
    for (int i = 0; i < 8; ++i) cc[i] = min(c0 + i, n - 1);
    const bool live = c0 < n;

    float tot[8], acc[8], zf[8], sf[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) tot[i] = acc[i] = zf[i] = sf[i] = 0.0f;
    int64_t cur = -1;
    for (int64_t j = live ? j0 : j1; j < j1; ++j) {
        const int64_t gi = (8 * j) / group;
        if (gi != cur) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                tot[i] = fmaf(sf[i], acc[i], tot[i]);
                acc[i] = 0.0f;
            }
            cur = gi;
            if (VEC) {
                const u32x4 s4 = ld16(sc + gi * n + c0);
                const u32x2 z2 = ld8(zp + gi * n + c0);
                const uint32_t sw[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sf[2 * i] = f16_bits_f32(sw[i] & 0xFFFFu);
                    sf[2 * i + 1] = f16_bits_f32(sw[i] >> 16);
                }
                zf[0] = ubyte<0>(z2.x);
                zf[1] = ubyte<1>(z2.x);
                zf[2] = ubyte<2>(z2.x);
                zf[3] = ubyte<3>(z2.x);
                zf[4] = ubyte<0>(z2.y);
                zf[5] = ubyte<1>(z2.y);
                zf[6] = ubyte<2>(z2.y);
                zf[7] = ubyte<3>(z2.y);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    sf[i] = f16_bits_f32(sc[gi * n + cc[i]]);
                    zf[i] = (float)zp[gi * n + cc[i]];
                }
            }
        }
        float xv[8];
        X8<XT>::at(x, 8 * j, xv);
        if (FMT == QBN_GPTQ4) {
            // word i holds rows 8j .. 8j+7 of column c0 + i, row 8j + e at bits 4e
            uint32_t w[8];
            if (VEC) {
                const u32x4 a = ld16(qw + j * n + c0), b = ld16(qw + j * n + c0 + 4);
                w[0] = a.x, w[1] = a.y, w[2] = a.z, w[3] = a.w, w[4] = b.x, w[5] = b.y, w[6] = b.z, w[7] = b.w;
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) w[i] = qw[j * n + cc[i]];
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float q[8];
                nibbles_f32(w[i], q);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[i] = fmaf(q[e] - zf[i], xv[e], acc[i]);
            }
        } else {
            // word e holds columns c0 .. c0+7 of row 8j + e; slot t is column
            // 0,2,4,6,1,3,5,7 [t]
            const int64_t nw = n / 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float q[8];
                nibbles_f32(qw[(8 * j + e) * nw + c0 / 8], q);
                constexpr int col[8] = {0, 2, 4, 6, 1, 3, 5, 7};
#pragma unroll
                for (int tt = 0; tt < 8; ++tt) acc[col[tt]] = fmaf(q[tt] - zf[col[tt]], xv[e], acc[col[tt]]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) tot[i] = fmaf(sf[i], acc[i], tot[i]);

    // slices: 16 per wave (lane bits 2..5), then the four waves in order
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float v = tot[i];
        v += __shfl_xor(v, 4, 64);
        v += __shfl_xor(v, 8, 64);
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        tot[i] = v;
    }
    const int lane = t % 64, wave = t / 64;
    if (lane < kAffCW) {
#pragma unroll
        for (int i = 0; i < 8; ++i) red[wave][lane][i] = tot[i];
    }
    __syncthreads();
    if (wave == 0 && lane < kAffCW && live) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float v = ((red[0][lane][i] + red[1][lane][i]) + red[2][lane][i]) + red[3][lane][i];
            if (c0 + i < n) y[c0 + i] = v;
        }
    }
}

// ------------------------------------------------------------------ Q4_0
// One wave per R rows; lanes stride over the rows' blocks and load each
// block's activations once for all R rows.
struct __attribute__((packed, aligned(2))) Q40 {
    uint16_t d;
    uint32_t c[4];
};

template <typename XT>
struct X32;  // the 32 activations of a block as binary32
template <>
struct X32<float> {
    __device__ __forceinline__ static void at(const float *x, int64_t k, float (&v)[32]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const f32x4 a = *reinterpret_cast<const f32x4 *>(x + k + 4 * i);
            v[4 * i] = a.x, v[4 * i + 1] = a.y, v[4 * i + 2] = a.z, v[4 * i + 3] = a.w;
        }
    }
};
template <>
struct X32<__bf16> {
    __device__ __forceinline__ static void at(const __bf16 *x, int64_t k, float (&v)[32]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4 w = ld16(x + k + 8 * i);
            const uint32_t p[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                v[8 * i + 2 * h] = __builtin_bit_cast(float, p[h] << 16);
                v[8 * i + 2 * h + 1] = __builtin_bit_cast(float, p[h] & 0xFFFF0000u);
            }
        }
    }
};

template <typename XT, int R>
__global__ __launch_bounds__(256) void k_gemv_q4_0(const uint8_t *__restrict__ blocks, const XT *__restrict__ x,
                                                   float *__restrict__ y, int64_t n, int64_t k) {
    const int lane = threadIdx.x % kWave;
    const int64_t r0 = ((int64_t)blockIdx.x * (256 / kWave) + threadIdx.x / kWave) * R;
    if (r0 >= n) return;  // whole waves only; no barrier follows
    const int64_t nb = k / 32;
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0f;
    for (int64_t b = lane; b < nb; b += kWave) {
        float xv[32];
        X32<XT>::at(x, 32 * b, xv);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t row = min(r0 + r, n - 1);
            const Q40 blk = *reinterpret_cast<const Q40 *>(blocks + (row * nb + b) * 18);
            float part = 0.0f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                // byte 4w + i holds elements 4w + i (low) and 16 + 4w + i (high)
                float q[8];
                nibbles_f32(blk.c[w], q);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    part = fmaf(q[2 * i] - 8.0f, xv[4 * w + i], part);
                    part = fmaf(q[2 * i + 1] - 8.0f, xv[16 + 4 * w + i], part);
                }
            }
            acc[r] = fmaf(f16_bits_f32(blk.d), part, acc[r]);
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = group_sum_last<64>(acc[r]);
    if (lane == kWave - 1) {
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (r0 + r < n) y[r0 + r] = acc[r];
    }
}

template <int FMT, typename XT>
hipError_t run_affine(const qbn_tensor &w, const XT *x, float *y, hipStream_t s) {
    const unsigned grid = (unsigned)((w.n + 8 * kAffCW - 1) / (8 * kAffCW));
    const bool vec = (w.n % 8) == 0 && ((uintptr_t)w.data % 16) == 0 && ((uintptr_t)w.scales % 16) == 0 &&
                     ((uintptr_t)w.zeros % 8) == 0;
    if (vec)
        hipLaunchKernelGGL((k_gemv_affine<FMT, XT, true>), dim3(grid), dim3(256), 0, s, (const uint32_t *)w.data,
                           (const uint16_t *)w.scales, (const uint8_t *)w.zeros, x, y, w.n, w.k, (int64_t)w.group);
    else
        hipLaunchKernelGGL((k_gemv_affine<FMT, XT, false>), dim3(grid), dim3(256), 0, s, (const uint32_t *)w.data,
                           (const uint16_t *)w.scales, (const uint8_t *)w.zeros, x, y, w.n, w.k, (int64_t)w.group);
    return hipGetLastError();
}

template <typename XT>
hipError_t run_q4_0(const qbn_tensor &w, const XT *x, float *y, hipStream_t s) {
    constexpr int R = 8;
    const int64_t waves = (w.n + R - 1) / R;
    hipLaunchKernelGGL((k_gemv_q4_0<XT, R>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s,
                       (const uint8_t *)w.data, x, y, w.n, w.k);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_int4(const qbn_tensor &w, const void *x, int x_dtype, float *y, hipStream_t s) {
    const bool bf = (x_dtype == QBN_BF16);
    switch (w.format) {
    case QBN_GPTQ4:
        return bf ? run_affine<QBN_GPTQ4, __bf16>(w, (const __bf16 *)x, y, s)
                  : run_affine<QBN_GPTQ4, float>(w, (const float *)x, y, s);
    case QBN_AWQ4:
        return bf ? run_affine<QBN_AWQ4, __bf16>(w, (const __bf16 *)x, y, s)
                  : run_affine<QBN_AWQ4, float>(w, (const float *)x, y, s);
    case QBN_Q4_0:
        return bf ? run_q4_0<__bf16>(w, (const __bf16 *)x, y, s) : run_q4_0<float>(w, (const float *)x, y, s);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace qbn
