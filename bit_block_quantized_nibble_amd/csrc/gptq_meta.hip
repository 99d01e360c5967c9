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

// Lanes of one wave whose group index equals this lane's: one ballot per bit
// of the index (nbits covers 0..G-1), starting from the lanes in range.
__device__ __forceinline__ uint64_t same_group_lanes(bool in, int g, int nbits) {
    uint64_t same = __ballot(in);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (g >> b) & 1;
        const uint64_t v = __ballot(bit);
        same &= bit ? v : ~v;
    }
    return same;
}

// One workgroup of 1024 threads (16 waves). Counts the rows of each group
// (LDS), checks every group holds exactly `group` rows, then gives each row
// its slot: its group's base, plus the rows of its group before it. Each
// wave owns one contiguous share of the rows (`span`, a multiple of 64) and
// walks it 64 rows at a time; the lanes holding the same group index find
// each other with ballots (same_group_lanes), so the rank inside a 64-row
// piece is a popcount. With G * 16 counters in LDS (G <= kPrefixGroups) the
// waves count their shares, an exclusive prefix over the waves (a shuffle
// scan across 16 lanes per group) gives each wave its starting offset per
// group, and the waves then place their rows
// independently, reading g_idx from an LDS copy made while counting when K
// <= kStageRows. Beyond that the waves take turns, one 64-row piece each per
// turn, on one shared counter per group. Either way each group keeps the
// original row order. On a bad g_idx it writes the identity (so that the
// row permutation that follows stays in bounds) and status -1 (a value
// outside 0..G-1) or -2 (a group of the wrong size); else status 0.
constexpr int kMaxGroups = 8192;
constexpr int kPrefixGroups = 512;
constexpr int kResolveThreads = 1024;
constexpr int kResolveWaves = kResolveThreads / 64;
constexpr int kStageRows = 16384;  // g_idx kept in LDS for the placement passes up to this K

__global__ __launch_bounds__(kResolveThreads) void k_resolve_g_idx(const int32_t *__restrict__ g_idx, int64_t K,
                                                                   int64_t group, int32_t *__restrict__ perm,
                                                                   int32_t *__restrict__ status) {
    __shared__ int cnt[kMaxGroups];  // also kResolveWaves x kPrefixGroups per-wave counters
    __shared__ int staged[kStageRows];
    __shared__ int bad;
    const int t = threadIdx.x;
    const int64_t G = K / group;
    const bool stage = K <= kStageRows;
    for (int64_t g = t; g < G; g += kResolveThreads) cnt[g] = 0;
    if (t == 0) bad = 0;
    __syncthreads();
    if (stage) {
        // all of a thread's (at most 16) loads in flight before the first use
        int gv[kStageRows / kResolveThreads];
#pragma unroll
        for (int i = 0; i < kStageRows / kResolveThreads; ++i) {
            const int64_t k = t + (int64_t)i * kResolveThreads;
            gv[i] = k < K ? g_idx[k] : 0;
        }
#pragma unroll
        for (int i = 0; i < kStageRows / kResolveThreads; ++i) {
            const int64_t k = t + (int64_t)i * kResolveThreads;
            if (k < K) {
                const int g = gv[i];
                staged[k] = g;
                if (g < 0 || g >= G)
                    atomicOr(&bad, 1);
                else
                    atomicAdd(&cnt[g], 1);
            }
        }
    } else {
        for (int64_t k = t; k < K; k += kResolveThreads) {
            const int g = g_idx[k];
            if (g < 0 || g >= G)
                atomicOr(&bad, 1);
            else
                atomicAdd(&cnt[g], 1);
        }
    }
    __syncthreads();
    if (bad == 0)
        for (int64_t g = t; g < G; g += kResolveThreads)
            if (cnt[g] != group) atomicOr(&bad, 2);
    __syncthreads();
    if (bad) {
        for (int64_t k = t; k < K; k += kResolveThreads) perm[k] = (int32_t)k;
        if (t == 0) status[0] = (bad & 1) ? -1 : -2;
        return;
    }
    const int lane = t & 63, wave = t >> 6;
    const int nbits = G > 1 ? 32 - __builtin_clz((unsigned)(G - 1)) : 0;
    const uint64_t below = (1ull << lane) - 1ull, above = ~(below | (1ull << lane));
    if (G <= kPrefixGroups) {
        int *cw = cnt + wave * kPrefixGroups;  // this wave's counters
        const int32_t *gsrc = stage ? staged : g_idx;
        const int64_t span = ((K + kResolveThreads - 1) / kResolveThreads) * 64;
        const int64_t k0 = wave * span, k1 = min(K, k0 + span);
        __syncthreads();
        for (int64_t g = lane; g < G; g += 64) cw[g] = 0;
        for (int64_t c = k0; c < k1; c += 64) {
            const int64_t k = c + lane;
            const bool in = k < k1;
            const int g = in ? gsrc[k] : 0;
            const uint64_t same = same_group_lanes(in, g, nbits);
            if (in && (same & above) == 0) cw[g] += __popcll(same);  // the last lane of its set
        }
        __syncthreads();
        // exclusive prefix over the 16 waves, per group: 16 neighbouring lanes
        // hold one group's 16 counts and scan them with shuffles; 64 groups
        // per pass (each count is read and written by its own thread)
        for (int64_t g0 = 0; g0 < G; g0 += kResolveThreads / kResolveWaves) {
            const int64_t g = g0 + t / kResolveWaves;
            const int w = t % kResolveWaves;
            const int c = g < G ? cnt[w * kPrefixGroups + g] : 0;
            int incl = c;
#pragma unroll
            for (int o = 1; o < kResolveWaves; o <<= 1) {
                const int n = __shfl_up(incl, o, kResolveWaves);
                if (w >= o) incl += n;
            }
            if (g < G) cnt[w * kPrefixGroups + g] = (int)(g * group) + incl - c;
        }
        __syncthreads();
        for (int64_t c = k0; c < k1; c += 64) {
            const int64_t k = c + lane;
            const bool in = k < k1;
            const int g = in ? gsrc[k] : 0;
            const uint64_t same = same_group_lanes(in, g, nbits);
            if (in) {
                const int base = cw[g];
                perm[base + __popcll(same & below)] = (int32_t)k;
                if ((same & above) == 0) cw[g] = base + __popcll(same);
            }
        }
    } else {
        for (int64_t g = t; g < G; g += kResolveThreads) cnt[g] = 0;
        __syncthreads();
        for (int64_t c = 0; c < K; c += kResolveThreads) {
            const int64_t k = c + t;
            const bool in = k < K;
            const int g = in ? g_idx[k] : 0;
            const uint64_t same = same_group_lanes(in, g, nbits);
            for (int w = 0; w < kResolveWaves; ++w) {
                if (wave == w && in) {
                    const int base = cnt[g];
                    perm[(int64_t)g * group + base + __popcll(same & below)] = (int32_t)k;
                    if ((same & above) == 0) cnt[g] = base + __popcll(same);
                }
                __syncthreads();
            }
        }
    }
    if (t == 0) status[0] = 0;
}

// One thread per output word (r, n), or per four neighbouring words (r, 4n ..
// 4n + 3) with 16-byte accesses when V4: row 8r + j of the result is source
// row p = perm[8r + j], whose nibble sits at bits 4 (p % 8) of source word
// (p / 8, n). A workgroup covers 256 (or 1024) neighbouring columns of one
// row r, so the eight source rows it gathers are read in runs of 1 (or 4)
// KB.
template <bool V4>
__global__ __launch_bounds__(256) void k_permute_gptq(const uint32_t *__restrict__ qw, const int32_t *__restrict__ perm,
                                                      int64_t K, int64_t N, uint32_t *__restrict__ out) {
    // tiles of 256 threads: (row r, column tile c), taken column-tile-major
    // and dealt in contiguous shares to the 8 XCDs (workgroup b runs on XCD
    // b % 8), so one XCD gathers from one column slab while it lasts in L2
    constexpr int64_t cols = V4 ? 1024 : 256;
    const int64_t rows = K / 8, ctiles = (N + cols - 1) / cols, B = rows * ctiles, b = blockIdx.x;
    const int64_t xcd = b % 8, idx = xcd * (B / 8) + (xcd < B % 8 ? xcd : B % 8) + b / 8;
    const int64_t r = idx % rows, n = (idx / rows) * cols + (int64_t)threadIdx.x * (V4 ? 4 : 1);
    if (n >= N) return;
    if constexpr (V4) {
        u32x4 w = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t p = perm[8 * r + j];
            const u32x4 src = ld16(qw + (p / 8) * N + n);
            const uint32_t sh = 4 * (uint32_t)(p % 8);
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] |= ((src[i] >> sh) & 15u) << (4 * j);
        }
        *reinterpret_cast<u32x4 *>(out + r * N + n) = w;
    } else {
        uint32_t w = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t p = perm[8 * r + j];
            w |= ((qw[(p / 8) * N + n] >> (4 * (p % 8))) & 15u) << (4 * j);
        }
        out[r * N + n] = w;
    }
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
    hipLaunchKernelGGL(k_resolve_g_idx, dim3(1), dim3(kResolveThreads), 0, s, g_idx, k, group, perm, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || n == 0 || k == 0) return e;
    const bool v4 = n % 4 == 0 && reinterpret_cast<uintptr_t>(qweight) % 16 == 0 &&
                    reinterpret_cast<uintptr_t>(qweight_out) % 16 == 0;
    const int64_t cols = v4 ? 1024 : 256;
    const dim3 grid((unsigned)((k / 8) * ((n + cols - 1) / cols)));
    if (v4)
        hipLaunchKernelGGL(k_permute_gptq<true>, grid, dim3(256), 0, s, (const uint32_t *)qweight, perm, k, n,
                           (uint32_t *)qweight_out);
    else
        hipLaunchKernelGGL(k_permute_gptq<false>, grid, dim3(256), 0, s, (const uint32_t *)qweight, perm, k, n,
                           (uint32_t *)qweight_out);
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
