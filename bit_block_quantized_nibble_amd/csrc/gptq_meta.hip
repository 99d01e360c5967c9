// GPTQ metadata conversions ("Bit Packing Architecture", "Real layouts
// compared" and "Repacking between formats", steps 2 and 3):
//   qzeros: int32 [G][N/8], a 4-bit stream along the output dimension
//     (column 8c + j at bits 4j of word c); version 1 stores z - 1, version
//     2 stores z. Converted to / from the logical zero points u8 [G][N].
//   act-order: g_idx[k] names the group of input row k. Resolving it orders
//     the rows by group (original order inside a group), permutes the packed
//     rows of qweight to match, and returns the permutation, which the
//     caller applies to the activations (qbn_permute) so that every output
//     is unchanged.
// All integer work, bit-exact.
#include "qbn_device.h"
#include "qbn_launch.h"

namespace qbn {
namespace {

// One thread per qzeros word: to_logical unpacks it into 8 zero points,
// otherwise packs 8 zero points into it.
__global__ __launch_bounds__(256) void k_qzeros(const void *__restrict__ src, void *__restrict__ dst, int64_t words,
                                                int version, int to_logical) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= words) return;
    const uint32_t off = version == 1 ? 1u : 0u;
    if (to_logical) {
        const uint32_t w = reinterpret_cast<const uint32_t *>(src)[t];
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            lo |= (((w >> (4 * j)) & 15u) + off) << (8 * j);
            hi |= (((w >> (4 * j + 16)) & 15u) + off) << (8 * j);
        }
        reinterpret_cast<u32x2 *>(dst)[t] = u32x2{lo, hi};
    } else {
        const u32x2 z = reinterpret_cast<const u32x2 *>(src)[t];
        uint32_t w = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            w |= (((z.x >> (8 * j)) - off) & 15u) << (4 * j);
            w |= (((z.y >> (8 * j)) - off) & 15u) << (4 * j + 16);
        }
        reinterpret_cast<uint32_t *>(dst)[t] = w;
    }
}

// One workgroup. Counts the rows of each group (LDS), checks every group
// holds exactly `group` rows, then places rows chunk by chunk: a row's slot
// is its group's base, plus the rows of that group in earlier chunks, plus
// those before it in its chunk. On a bad g_idx it writes the identity (so
// that the row permutation that follows stays in bounds) and status -1 (a
// value outside 0..G-1) or -2 (a group of the wrong size); else status 0.
constexpr int kMaxGroups = 8192;

__global__ __launch_bounds__(256) void k_resolve_g_idx(const int32_t *__restrict__ g_idx, int64_t K, int64_t group,
                                                       int32_t *__restrict__ perm, int32_t *__restrict__ status) {
    __shared__ int cnt[kMaxGroups];
    __shared__ int gbuf[256];
    __shared__ int bad;
    const int t = threadIdx.x;
    const int64_t G = K / group;
    for (int64_t g = t; g < G; g += 256) cnt[g] = 0;
    if (t == 0) bad = 0;
    __syncthreads();
    for (int64_t k = t; k < K; k += 256) {
        const int g = g_idx[k];
        if (g < 0 || g >= G)
            atomicOr(&bad, 1);
        else
            atomicAdd(&cnt[g], 1);
    }
    __syncthreads();
    if (bad == 0)
        for (int64_t g = t; g < G; g += 256)
            if (cnt[g] != group) atomicOr(&bad, 2);
    __syncthreads();
    if (bad) {
        for (int64_t k = t; k < K; k += 256) perm[k] = (int32_t)k;
        if (t == 0) status[0] = (bad & 1) ? -1 : -2;
        return;
    }
    for (int64_t g = t; g < G; g += 256) cnt[g] = 0;
    __syncthreads();
    for (int64_t c = 0; c < K; c += 256) {
        const int64_t k = c + t;
        const int g = k < K ? g_idx[k] : -1;
        gbuf[t] = g;
        __syncthreads();
        if (k < K) {
            int rank = 0;
            for (int u = 0; u < t; ++u) rank += gbuf[u] == g;
            perm[(int64_t)g * group + cnt[g] + rank] = (int32_t)k;
        }
        __syncthreads();
        if (k < K) atomicAdd(&cnt[g], 1);
        __syncthreads();
    }
    if (t == 0) status[0] = 0;
}

// One thread per output word (r, n): row 8r + j of the result is source row
// perm[8r + j], whose nibble sits at bits 4 (p % 8) of source word (p / 8, n).
__global__ __launch_bounds__(256) void k_permute_gptq(const uint32_t *__restrict__ qw, const int32_t *__restrict__ perm,
                                                      int64_t K, int64_t N, uint32_t *__restrict__ out) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= (K / 8) * N) return;
    const int64_t r = t / N, n = t - r * N;
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int64_t p = perm[8 * r + j];
        w |= ((qw[(p / 8) * N + n] >> (4 * (p % 8))) & 15u) << (4 * j);
    }
    out[t] = w;
}

template <typename T>
__global__ __launch_bounds__(256) void k_permute(const T *__restrict__ src, const int32_t *__restrict__ perm,
                                                 int64_t count, T *__restrict__ dst) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t < count) dst[t] = src[perm[t]];
}

}  // namespace

hipError_t launch_gptq_qzeros(const void *src, void *dst, int64_t groups, int64_t n, int version, int to_logical,
                              hipStream_t s) {
    const int64_t words = groups * (n / 8);
    hipLaunchKernelGGL(k_qzeros, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s, src, dst, words, version,
                       to_logical);
    return hipGetLastError();
}

hipError_t launch_gptq_resolve_g_idx(const void *qweight, const int32_t *g_idx, int64_t k, int64_t n, int64_t group,
                                     void *qweight_out, int32_t *perm, int32_t *status, hipStream_t s) {
    hipLaunchKernelGGL(k_resolve_g_idx, dim3(1), dim3(256), 0, s, g_idx, k, group, perm, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || n == 0) return e;
    const int64_t words = (k / 8) * n;
    hipLaunchKernelGGL(k_permute_gptq, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s,
                       (const uint32_t *)qweight, perm, k, n, (uint32_t *)qweight_out);
    return hipGetLastError();
}

hipError_t launch_permute(const void *src, const int32_t *perm, int64_t count, int elem_bytes, void *dst,
                          hipStream_t s) {
    const unsigned grid = (unsigned)((count + 255) / 256);
    if (elem_bytes == 4)
        hipLaunchKernelGGL(k_permute<uint32_t>, dim3(grid), dim3(256), 0, s, (const uint32_t *)src, perm, count,
                           (uint32_t *)dst);
    else
        hipLaunchKernelGGL(k_permute<uint16_t>, dim3(grid), dim3(256), 0, s, (const uint16_t *)src, perm, count,
                           (uint16_t *)dst);
    return hipGetLastError();
}

bool gptq_groups_fit(int64_t k, int64_t group) { return k / group <= kMaxGroups; }

}  // namespace qbn
