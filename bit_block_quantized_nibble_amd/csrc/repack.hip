// Bit-exact int4 layout repacks between GPTQ, AWQ and GGUF Q4_0.
//
// "Bit Packing Architecture", 'Repacking between formats': the safe method
// goes through the logical matrix -- unpack the source codes to a plain
// [K][N] u8 matrix with the source's axis, order and sign handling, then
// pack with the target's axis and order -- and never reinterprets words.
// Here the logical matrix exists one tile at a time, in LDS: a workgroup
// unpacks a KT x NT tile of the source into LDS (u8 per code, [k][n]) with
// loads that are contiguous across the workgroup, synchronizes, and packs
// the tile into the target layout with stores that are contiguous as well.
//
// Layouts ("Bit Packing Architecture", 'Real layouts compared'):
//  GPTQ int32 [K/8][N]: row 8r+j of column n at bits 4j of word [r][n];
//  AWQ  int32 [K][N/8]: slot t of word [k][g] holds column 8g + {0,2,4,6,1,3,5,7}[t];
//  Q4_0 [N][K/32] x 18 bytes: fp16 d, then byte j = element j | element j+16 << 4,
//       blocks running along k inside output column n.
// Codes are moved unchanged (shifts are logical, so a top-slot code >= 8 that
// makes the int32 negative round-trips). A Q4_0 block's d is the bit
// pattern of the source group's fp16 scale; in the other direction the
// group scale is the d of the group's first block and the zero point is 8.
#include "qbn_device.h"
#include "qbn_launch.h"

namespace qbn {
namespace {

constexpr int KT = 256;            // tile rows (k)
constexpr int NT = 64;             // tile columns (n)
constexpr int LDP = NT + 4;        // LDS row pitch in bytes (breaks bank alignment of rows)
constexpr int kThreads = 256;

// AWQ slot s holds column awq_col(s) of its group of eight: 0,2,4,6,1,3,5,7.
__device__ __forceinline__ constexpr int awq_col(int s) { return s < 4 ? 2 * s : 2 * (s - 4) + 1; }

struct Tile {
    uint8_t q[KT * LDP];
};

__device__ __forceinline__ uint32_t lds_dword(const Tile &t, int k, int c) {
    return *reinterpret_cast<const uint32_t *>(&t.q[k * LDP + c]);
}
__device__ __forceinline__ void lds_put_dword(Tile &t, int k, int c, uint32_t v) {
    *reinterpret_cast<uint32_t *>(&t.q[k * LDP + c]) = v;
}

// ------------------------------------------------------------------ unpack into LDS
// GPTQ: thread -> column quad cq (4 columns), word rows r = t/16 + 16*i.
__device__ void load_gptq(Tile &t, const uint32_t *__restrict__ qw, int64_t N, int64_t K, int64_t k0, int64_t n0) {
    const int cq = threadIdx.x % (NT / 4);
    const int rr = threadIdx.x / (NT / 4);
    for (int r = rr; r < KT / 8; r += kThreads / (NT / 4)) {
        const int64_t kr = k0 / 8 + r;
        uint32_t w[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int64_t n = n0 + 4 * cq + c;
            w[c] = (8 * kr < K && n < N) ? qw[kr * N + n] : 0u;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t v = 0;
#pragma unroll
            for (int c = 0; c < 4; ++c) v |= ((w[c] >> (4 * j)) & 15u) << (8 * c);
            lds_put_dword(t, 8 * r + j, 4 * cq, v);
        }
    }
}

// AWQ: thread -> word column g (8 codes), rows k = t/8 + 32*i.
__device__ void load_awq(Tile &t, const uint32_t *__restrict__ qw, int64_t N, int64_t K, int64_t k0, int64_t n0) {
    const int g = threadIdx.x % (NT / 8);
    const int kk = threadIdx.x / (NT / 8);
    const int64_t ng = N / 8;
    for (int k = kk; k < KT; k += kThreads / (NT / 8)) {
        const int64_t kg = k0 + k;
        const int64_t gg = n0 / 8 + g;
        const uint32_t w = (kg < K && gg < ng) ? qw[kg * ng + gg] : 0u;
        uint32_t col[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) col[awq_col(s)] = (w >> (4 * s)) & 15u;
        lds_put_dword(t, k, 8 * g, col[0] | (col[1] << 8) | (col[2] << 16) | (col[3] << 24));
        lds_put_dword(t, k, 8 * g + 4, col[4] | (col[5] << 8) | (col[6] << 16) | (col[7] << 24));
    }
}

// Q4_0: thread -> (column quad cq, block b); reads the 4 blocks (cq's columns, b).
__device__ void load_q4_0(Tile &t, const uint8_t *__restrict__ blocks, int64_t N, int64_t K, int64_t k0,
                          int64_t n0) {
    const int cq = threadIdx.x % (NT / 4);
    const int b = threadIdx.x / (NT / 4);
    if (b >= KT / 32) return;
    const int64_t nbr = K / 32;  // blocks per output column
    const int64_t bg = k0 / 32 + b;
    uint32_t codes[4][4];        // [column][code dword]
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int64_t n = n0 + 4 * cq + c;
        const bool ok = (bg < nbr) && (n < N);
        const uint16_t *bp = reinterpret_cast<const uint16_t *>(blocks + (n * nbr + bg) * 18);
        uint16_t h[9];
#pragma unroll
        for (int i = 1; i < 9; ++i) h[i] = ok ? bp[i] : (uint16_t)0;
#pragma unroll
        for (int i = 0; i < 4; ++i) codes[c][i] = (uint32_t)h[1 + 2 * i] | ((uint32_t)h[2 + 2 * i] << 16);
    }
    // byte j of the 16 code bytes: element j (low), element j+16 (high)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t byte = (codes[c][j / 4] >> (8 * (j % 4))) & 0xFFu;
            lo |= (byte & 15u) << (8 * c);
            hi |= (byte >> 4) << (8 * c);
        }
        lds_put_dword(t, 32 * b + j, 4 * cq, lo);
        lds_put_dword(t, 32 * b + j + 16, 4 * cq, hi);
    }
}

// ------------------------------------------------------------------ pack from LDS
__device__ void store_gptq(const Tile &t, uint32_t *__restrict__ qw, int64_t N, int64_t K, int64_t k0, int64_t n0) {
    const int cq = threadIdx.x % (NT / 4);
    const int rr = threadIdx.x / (NT / 4);
    for (int r = rr; r < KT / 8; r += kThreads / (NT / 4)) {
        const int64_t kr = k0 / 8 + r;
        if (8 * kr >= K) break;
        uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t v = lds_dword(t, 8 * r + j, 4 * cq);
#pragma unroll
            for (int c = 0; c < 4; ++c) w[c] |= ((v >> (8 * c)) & 15u) << (4 * j);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int64_t n = n0 + 4 * cq + c;
            if (n < N) qw[kr * N + n] = w[c];
        }
    }
}

__device__ void store_awq(const Tile &t, uint32_t *__restrict__ qw, int64_t N, int64_t K, int64_t k0, int64_t n0) {
    const int g = threadIdx.x % (NT / 8);
    const int kk = threadIdx.x / (NT / 8);
    const int64_t ng = N / 8;
    for (int k = kk; k < KT; k += kThreads / (NT / 8)) {
        const int64_t kg = k0 + k;
        const int64_t gg = n0 / 8 + g;
        if (kg >= K || gg >= ng) continue;
        const uint32_t a = lds_dword(t, k, 8 * g), b = lds_dword(t, k, 8 * g + 4);
        uint32_t col[8];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            col[c] = (a >> (8 * c)) & 15u;
            col[4 + c] = (b >> (8 * c)) & 15u;
        }
        uint32_t w = 0;
#pragma unroll
        for (int s = 0; s < 8; ++s) w |= col[awq_col(s)] << (4 * s);
        qw[kg * ng + gg] = w;
    }
}

// Q4_0 destination: d of block (n, b) = fp16 bits of scale[(32b)/group][n].
__device__ void store_q4_0(const Tile &t, uint8_t *__restrict__ blocks, const uint16_t *__restrict__ scales,
                           int64_t group, int64_t N, int64_t K, int64_t k0, int64_t n0) {
    const int cq = threadIdx.x % (NT / 4);
    const int b = threadIdx.x / (NT / 4);
    if (b >= KT / 32) return;
    const int64_t nbr = K / 32;
    const int64_t bg = k0 / 32 + b;
    if (bg >= nbr) return;
    uint32_t lo[16], hi[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        lo[j] = lds_dword(t, 32 * b + j, 4 * cq);
        hi[j] = lds_dword(t, 32 * b + j + 16, 4 * cq);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int64_t n = n0 + 4 * cq + c;
        if (n >= N) break;
        uint16_t *bp = reinterpret_cast<uint16_t *>(blocks + (n * nbr + bg) * 18);
        bp[0] = scales[((32 * bg) / group) * N + n];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t b0 = ((lo[2 * i] >> (8 * c)) & 15u) | (((hi[2 * i] >> (8 * c)) & 15u) << 4);
            const uint32_t b1 = ((lo[2 * i + 1] >> (8 * c)) & 15u) | (((hi[2 * i + 1] >> (8 * c)) & 15u) << 4);
            bp[1 + i] = (uint16_t)(b0 | (b1 << 8));
        }
    }
}

template <int SRC, int DST>
__global__ __launch_bounds__(kThreads) void k_repack(const void *__restrict__ src, const uint16_t *__restrict__ src_scales,
                                                     int64_t group, void *__restrict__ dst, int64_t N, int64_t K) {
    __shared__ Tile tile;
    const int64_t ntiles_n = (N + NT - 1) / NT;
    const int64_t k0 = (int64_t)(blockIdx.x / ntiles_n) * KT;
    const int64_t n0 = (int64_t)(blockIdx.x % ntiles_n) * NT;
    if (SRC == QBN_GPTQ4) load_gptq(tile, (const uint32_t *)src, N, K, k0, n0);
    if (SRC == QBN_AWQ4) load_awq(tile, (const uint32_t *)src, N, K, k0, n0);
    if (SRC == QBN_Q4_0) load_q4_0(tile, (const uint8_t *)src, N, K, k0, n0);
    __syncthreads();
    if (DST == QBN_GPTQ4) store_gptq(tile, (uint32_t *)dst, N, K, k0, n0);
    if (DST == QBN_AWQ4) store_awq(tile, (uint32_t *)dst, N, K, k0, n0);
    if (DST == QBN_Q4_0) store_q4_0(tile, (uint8_t *)dst, src_scales, group, N, K, k0, n0);
}

// Q4_0 -> GPTQ/AWQ companions: scale[gi][n] = d of block (n, gi*group/32), zero = 8.
__global__ __launch_bounds__(256) void k_q4_0_group_scales(const uint8_t *__restrict__ blocks, int64_t N, int64_t K,
                                                           int64_t group, uint16_t *__restrict__ scales,
                                                           uint8_t *__restrict__ zeros) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t G = K / group;
    if (i >= G * N) return;
    const int64_t gi = i / N, n = i - gi * N;
    const int64_t b = gi * (group / 32);
    scales[i] = *reinterpret_cast<const uint16_t *>(blocks + (n * (K / 32) + b) * 18);
    zeros[i] = 8;
}

template <int SRC, int DST>
hipError_t run(const qbn_tensor &s, int64_t group, void *dst, hipStream_t st) {
    const int64_t N = s.n, K = s.k;
    const int64_t tiles = ((K + KT - 1) / KT) * ((N + NT - 1) / NT);
    hipLaunchKernelGGL((k_repack<SRC, DST>), dim3((unsigned)tiles), dim3(kThreads), 0, st, s.data,
                       (const uint16_t *)s.scales, group, dst, N, K);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_repack(const qbn_tensor &src, int dst_format, int dst_group, void *dst_data, void *dst_scales,
                         void *dst_zeros, hipStream_t s) {
    const int64_t N = src.n, K = src.k;
    hipError_t e = hipErrorInvalidValue;
    const int sf = src.format;
    if (sf == QBN_GPTQ4 && dst_format == QBN_AWQ4) e = run<QBN_GPTQ4, QBN_AWQ4>(src, src.group, dst_data, s);
    else if (sf == QBN_AWQ4 && dst_format == QBN_GPTQ4) e = run<QBN_AWQ4, QBN_GPTQ4>(src, src.group, dst_data, s);
    else if (sf == QBN_GPTQ4 && dst_format == QBN_Q4_0) e = run<QBN_GPTQ4, QBN_Q4_0>(src, src.group, dst_data, s);
    else if (sf == QBN_AWQ4 && dst_format == QBN_Q4_0) e = run<QBN_AWQ4, QBN_Q4_0>(src, src.group, dst_data, s);
    else if (sf == QBN_Q4_0 && dst_format == QBN_GPTQ4) e = run<QBN_Q4_0, QBN_GPTQ4>(src, dst_group, dst_data, s);
    else if (sf == QBN_Q4_0 && dst_format == QBN_AWQ4) e = run<QBN_Q4_0, QBN_AWQ4>(src, dst_group, dst_data, s);
    if (e != hipSuccess) return e;
    if (sf == QBN_Q4_0) {
        const int64_t cnt = (K / dst_group) * N;
        if (cnt > 0) {
            hipLaunchKernelGGL(k_q4_0_group_scales, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, s,
                               (const uint8_t *)src.data, N, K, (int64_t)dst_group, (uint16_t *)dst_scales,
                               (uint8_t *)dst_zeros);
            e = hipGetLastError();
        }
    } else if (dst_format != QBN_Q4_0) {
        // GPTQ <-> AWQ: scales and zero points keep their [K/group][N] layout
        const int64_t cnt = (K / src.group) * N;
        if (dst_scales && dst_scales != src.scales && cnt > 0)
            e = hipMemcpyAsync(dst_scales, src.scales, 2 * cnt, hipMemcpyDeviceToDevice, s);
        if (e == hipSuccess && dst_zeros && dst_zeros != src.zeros && cnt > 0)
            e = hipMemcpyAsync(dst_zeros, src.zeros, cnt, hipMemcpyDeviceToDevice, s);
    }
    return e;
}

}  // namespace qbn
