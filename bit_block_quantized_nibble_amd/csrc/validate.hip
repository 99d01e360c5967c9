// Load-time fail-closed scan ("Chapter 7 - NVFP4: the native lane", section
// 7.3: a NaN scale byte or an inconsistent companion refuses the load;
// "Four Bits, Three Contracts", section 7: reject rather than misread).
// The hot-path kernels trust validated scales and do not re-check them.
//
// The result is the smallest offending index, found with a 64-bit atomic
// minimum (order-independent, so the answer is deterministic), then turned
// into -1 when nothing was found. The three steps are kernels on the
// caller's stream; no memset node is used.
#include "qbn_device.h"
#include "qbn_launch.h"

namespace qbn {
namespace {

constexpr int kBlock = 256;
constexpr unsigned long long kNone = 0x7FFFFFFFFFFFFFFFull;

__global__ void k_set(unsigned long long *p, unsigned long long v) {
    if (threadIdx.x == 0 && blockIdx.x == 0) *p = v;
}

__global__ void k_finish(unsigned long long *p) {
    if (threadIdx.x == 0 && blockIdx.x == 0 && *p == kNone) *p = ~0ull;  // -1 as int64
}

__device__ __forceinline__ bool f16_nonfinite(uint32_t h) { return ((h >> 10) & 31u) == 31u; }

// kind 0: E8M0 scale bytes (0xFF is NaN); kind 1: E4M3FN (0x7F / 0xFF).
template <int KIND>
__global__ __launch_bounds__(kBlock) void k_scan_bytes(const uint8_t *__restrict__ p, int64_t count,
                                                        unsigned long long *first) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
        const uint32_t b = p[i];
        const bool bad = (KIND == 0) ? (b == 0xFFu) : ((b & 0x7Fu) == 0x7Fu);
        if (bad) atomicMin(first, (unsigned long long)i);
    }
}

// CKE split-half NVFP4 blocks: subscale i (logical order, row-major over
// [n][k/16]) is byte i % 4 of block i / 4; E4M3FN NaN is 0x7F / 0xFF.
__global__ __launch_bounds__(kBlock) void k_scan_cke(const uint8_t *__restrict__ blocks, int64_t count,
                                                      unsigned long long *first) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
        const uint32_t b = blocks[36 * (i / 4) + (i % 4)];
        if ((b & 0x7Fu) == 0x7Fu) atomicMin(first, (unsigned long long)i);
    }
}

// Q4_K blocks: d or dmin not finite.
__global__ __launch_bounds__(kBlock) void k_scan_q4k(const uint8_t *__restrict__ blocks, int64_t nblocks,
                                                      unsigned long long *first) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nblocks; i += stride) {
        const uint32_t h = ld4(blocks + 144 * i);
        if (f16_nonfinite(h & 0xFFFFu) || f16_nonfinite(h >> 16)) atomicMin(first, (unsigned long long)i);
    }
}

// Q4_0 blocks [n][k/32]: d not finite, or (bpg > 1) d differs from the first
// block of its group of bpg blocks along k.
__global__ __launch_bounds__(kBlock) void k_scan_q4_0(const uint8_t *__restrict__ blocks, int64_t nblocks,
                                                       int64_t bpr, int64_t bpg, unsigned long long *first) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nblocks; i += stride) {
        const uint32_t d = *reinterpret_cast<const uint16_t *>(blocks + 18 * i);
        bool bad = f16_nonfinite(d);
        if (bpg > 1) {
            const int64_t b = i % bpr;
            const int64_t lead = i - (b % bpg);
            bad = bad || (*reinterpret_cast<const uint16_t *>(blocks + 18 * lead) != d);
        }
        if (bad) atomicMin(first, (unsigned long long)i);
    }
}

// Refusal scans of the Q4_0 repacks. Exactly QBN_REPACK_SCAN_PARTS
// workgroups stride over the elements; workgroup g writes the smallest
// offending index it saw (or kNone) to parts[g]. Every word is written on
// every call, so nothing has to be cleared first; the repack kernel that
// follows takes the minimum of the parts.
// The repack refusal scans: exactly QBN_REPACK_SCAN_PARTS workgroups of
// kScanThreads, each writing the lowest offending index it saw (kNone if
// none) to parts[blockIdx.x]; the repack kernels reduce the parts. Every
// thread issues all of its loads before it compares anything, so a scan
// costs about one memory round trip rather than one per loop trip.
constexpr int kScanThreads = 1024;

__device__ __forceinline__ void part_min_store(unsigned long long mine, unsigned long long *parts) {
    __shared__ unsigned long long red[kScanThreads / 64];
    for (int off = 32; off > 0; off >>= 1) {
        const unsigned long long o = __shfl_xor(mine, off, 64);
        mine = o < mine ? o : mine;
    }
    if ((threadIdx.x & 63) == 0) red[threadIdx.x / 64] = mine;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned long long m = red[0];
        for (int w = 1; w < kScanThreads / 64; ++w) m = red[w] < m ? red[w] : m;
        parts[blockIdx.x] = m;
    }
}

__device__ __forceinline__ unsigned long long umin64(unsigned long long a, unsigned long long b) {
    return b < a ? b : a;
}

// Zero points that Q4_0 cannot hold: every one must be 8. The bytes before
// the first 16-byte boundary and after the last are checked one by one, the
// rest 16 at a time, four pieces per thread in flight.
__global__ __launch_bounds__(kScanThreads) void k_part_zero8(const uint8_t *__restrict__ zeros, int64_t count,
                                                              unsigned long long *parts) {
    unsigned long long mine = kNone;
    const int64_t t = (int64_t)blockIdx.x * kScanThreads + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * kScanThreads;
    int64_t head = (int64_t)((16u - (unsigned)(reinterpret_cast<uintptr_t>(zeros) & 15u)) & 15u);
    if (head > count) head = count;
    const int64_t pieces = (count - head) / 16;
    if (t < head && zeros[t] != 8u) mine = (unsigned long long)t;
    const u32x4 *al = reinterpret_cast<const u32x4 *>(zeros + head);
    for (int64_t p0 = t; p0 < pieces; p0 += 4 * stride) {
        u32x4 v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t p = p0 + j * stride;
            v[j] = p < pieces ? al[p] : u32x4{0x08080808u, 0x08080808u, 0x08080808u, 0x08080808u};
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t x = w[q] ^ 0x08080808u;  // nonzero bytes are zero points other than 8
                if (x != 0u)
                    mine = umin64(mine, (unsigned long long)(head + 16 * (p0 + j * stride) + 4 * q +
                                                             (__builtin_ctz(x) >> 3)));
            }
        }
    }
    for (int64_t i = head + 16 * pieces + t; i < count; i += stride)
        if (zeros[i] != 8u) mine = umin64(mine, (unsigned long long)i);
    part_min_store(mine, parts);
}

// Q4_0 blocks [n][k/32] whose d differs from the first block of their group
// of bpg blocks along k; eight blocks per thread in flight.
__global__ __launch_bounds__(kScanThreads) void k_part_q4_0_groups(const uint8_t *__restrict__ blocks,
                                                                    int64_t nblocks, int64_t bpr, int64_t bpg,
                                                                    unsigned long long *parts) {
    unsigned long long mine = kNone;
    const int64_t t = (int64_t)blockIdx.x * kScanThreads + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * kScanThreads;
    for (int64_t i0 = t; i0 < nblocks; i0 += 8 * stride) {
        uint16_t d[8], lead_d[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t i = i0 + j * stride;
            const int64_t ic = i < nblocks ? i : i0;
            const int64_t lead = ic - ((ic % bpr) % bpg);
            d[j] = *reinterpret_cast<const uint16_t *>(blocks + 18 * ic);
            lead_d[j] = *reinterpret_cast<const uint16_t *>(blocks + 18 * lead);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t i = i0 + j * stride;
            if (i < nblocks && d[j] != lead_d[j]) mine = umin64(mine, (unsigned long long)i);
        }
    }
    part_min_store(mine, parts);
}

// GPTQ / AWQ companions: scale not finite or logical zero point above 15.
__global__ __launch_bounds__(kBlock) void k_scan_affine(const uint16_t *__restrict__ scales,
                                                         const uint8_t *__restrict__ zeros, int64_t count,
                                                         unsigned long long *first) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
        if (f16_nonfinite(scales[i]) || zeros[i] > 15u) atomicMin(first, (unsigned long long)i);
    }
}

int64_t scan_grid(int64_t count) {
    int64_t g = (count + kBlock - 1) / kBlock;
    if (g > 4096) g = 4096;
    return g < 1 ? 1 : g;
}

__global__ void k_fill_zero(uint32_t *p, int64_t words) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += stride) p[i] = 0u;
}

__global__ void k_fill_zero_bytes(uint8_t *p, int64_t bytes) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < bytes; i += stride) p[i] = 0u;
}

// Zero the logical [rows][cols] region of a 2-byte matrix with leading
// dimension ld (padding columns are left untouched).
__global__ void k_fill_zero_2d_u16(uint16_t *p, int64_t rows, int64_t cols, int64_t ld) {
    const int64_t total = rows * cols;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int64_t r = i / cols;
        p[r * ld + (i - r * cols)] = 0;
    }
}

}  // namespace

hipError_t launch_fill_zero_2d_u16(void *out, int64_t rows, int64_t cols, int64_t ld, hipStream_t s) {
    if (rows <= 0 || cols <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_zero_2d_u16, dim3((unsigned)scan_grid(rows * cols)), dim3(kBlock), 0, s,
                       (uint16_t *)out, rows, cols, ld);
    return hipGetLastError();
}

hipError_t launch_validate(const qbn_tensor &w, int64_t *first_bad, hipStream_t s) {
    unsigned long long *f = reinterpret_cast<unsigned long long *>(first_bad);
    hipLaunchKernelGGL(k_set, dim3(1), dim3(64), 0, s, f, kNone);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = w.n, k = w.k;
    int64_t count = 0;
    switch (w.format) {
    case QBN_MXFP4:
        count = n * (k / 32);
        if (count > 0)
            hipLaunchKernelGGL(k_scan_bytes<0>, dim3((unsigned)scan_grid(count)), dim3(kBlock), 0, s,
                               (const uint8_t *)w.scales, count, f);
        break;
    case QBN_NVFP4:
        count = n * (k / 16);
        if (count > 0)
            hipLaunchKernelGGL(k_scan_bytes<1>, dim3((unsigned)scan_grid(count)), dim3(kBlock), 0, s,
                               (const uint8_t *)w.scales, count, f);
        break;
    case QBN_NVFP4_CKE:
        count = n * (k / 16);
        if (count > 0)
            hipLaunchKernelGGL(k_scan_cke, dim3((unsigned)scan_grid(count)), dim3(kBlock), 0, s,
                               (const uint8_t *)w.data, count, f);
        break;
    case QBN_Q4_K:
        count = n * (k / 256);
        if (count > 0)
            hipLaunchKernelGGL(k_scan_q4k, dim3((unsigned)scan_grid(count)), dim3(kBlock), 0, s,
                               (const uint8_t *)w.data, count, f);
        break;
    case QBN_Q4_0: {
        count = n * (k / 32);
        const int64_t bpg = (w.group > 0) ? (int64_t)w.group / 32 : 1;
        if (count > 0)
            hipLaunchKernelGGL(k_scan_q4_0, dim3((unsigned)scan_grid(count)), dim3(kBlock), 0, s,
                               (const uint8_t *)w.data, count, k / 32, bpg, f);
        break;
    }
    case QBN_GPTQ4:
    case QBN_AWQ4:
        count = (k / w.group) * n;
        if (count > 0)
            hipLaunchKernelGGL(k_scan_affine, dim3((unsigned)scan_grid(count)), dim3(kBlock), 0, s,
                               (const uint16_t *)w.scales, (const uint8_t *)w.zeros, count, f);
        break;
    default:
        return hipErrorInvalidValue;
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_finish, dim3(1), dim3(64), 0, s, f);
    return hipGetLastError();
}

hipError_t launch_fill_i64(int64_t *p, int64_t v, int64_t count, hipStream_t s) {
    for (int64_t i = 0; i < count; ++i)
        hipLaunchKernelGGL(k_set, dim3(1), dim3(64), 0, s, reinterpret_cast<unsigned long long *>(p + i),
                           (unsigned long long)v);
    return hipGetLastError();
}

hipError_t launch_scan_zero_points(const uint8_t *zeros, int64_t count, int64_t *parts, hipStream_t s) {
    hipLaunchKernelGGL(k_part_zero8, dim3(QBN_REPACK_SCAN_PARTS), dim3(kScanThreads), 0, s, zeros, count,
                       reinterpret_cast<unsigned long long *>(parts));
    return hipGetLastError();
}

hipError_t launch_scan_q4_0_groups(const uint8_t *blocks, int64_t n, int64_t k, int64_t group, int64_t *parts,
                                   hipStream_t s) {
    hipLaunchKernelGGL(k_part_q4_0_groups, dim3(QBN_REPACK_SCAN_PARTS), dim3(kScanThreads), 0, s, blocks,
                       n * (k / 32),
                       k / 32, group / 32, reinterpret_cast<unsigned long long *>(parts));
    return hipGetLastError();
}

hipError_t launch_fill_zero(void *out, int64_t bytes, hipStream_t s) {
    if (bytes <= 0) return hipSuccess;
    if (((uintptr_t)out % 4 == 0) && (bytes % 4 == 0)) {
        const int64_t words = bytes / 4;
        hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)scan_grid(words)), dim3(kBlock), 0, s, (uint32_t *)out, words);
    } else {
        hipLaunchKernelGGL(k_fill_zero_bytes, dim3((unsigned)scan_grid(bytes)), dim3(kBlock), 0, s, (uint8_t *)out,
                           bytes);
    }
    return hipGetLastError();
}

}  // namespace qbn
