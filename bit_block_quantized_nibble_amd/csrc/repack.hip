// Bit-exact int4 layout repacks between GPTQ, AWQ and GGUF Q4_0.
//
// "Bit Packing Architecture", 'Repacking between formats': the safe method
// goes through the logical matrix -- unpack the source codes to a plain
// [K][N] u8 matrix with the source's axis, order and sign handling, then
// pack with the target's axis and order -- and never reinterprets words.
// GPTQ <-> AWQ: a thread holds the logical 8 x 8 block of codes (8 rows x 8
// columns) that one group of 8 GPTQ words and one group of 8 AWQ words both
// cover, as eight 32-bit words, and transposes it in registers (a three-
// stage butterfly: 16-bit halves, bytes, nibbles), with AWQ's slot order
// applied by renaming the words. Loads and stores are contiguous across
// consecutive threads.
// Q4_0 <-> GPTQ / AWQ: one Q4_0 block (32 consecutive k of one column) is
// four GPTQ words of that column, or column slot s of 32 AWQ words after
// four of the 8 x 8 transposes above; its 16 code bytes pair k = j with
// k = j + 16, a nibble zip of those words. Q4_0 is column-major, so a
// workgroup stages its tile's runs (8 consecutive blocks of each of its
// columns) in LDS and moves each run with contiguous 4- or 2-byte accesses;
// the GPTQ / AWQ side is read or written straight from registers, contiguous
// across consecutive threads.
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
#include <mutex>

#include "qbn_device.h"
#include "qbn_launch.h"

namespace qbn {
namespace {

// AWQ slot s holds column awq_col(s) of its group of eight: 0,2,4,6,1,3,5,7.
__device__ __forceinline__ constexpr int awq_col(int s) { return s < 4 ? 2 * s : 2 * (s - 4) + 1; }

// ------------------------------------------------------------------ 8 x 8 nibble transpose
// x[s] nibble j -> x[j] nibble s (a three-stage butterfly).
// __builtin_amdgcn_perm(a, b, sel): byte i of the result is byte sel_i of the
// 8-byte value a:b (b = bytes 0..3, a = bytes 4..7).
__device__ __forceinline__ void nib_transpose8(uint32_t *x) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {  // 16-bit halves, distance 4
        const uint32_t a = x[s], b = x[s + 4];
        x[s] = __builtin_amdgcn_perm(b, a, 0x05040100u);
        x[s + 4] = __builtin_amdgcn_perm(b, a, 0x07060302u);
    }
#pragma unroll
    for (int g = 0; g < 8; g += 4)
#pragma unroll
        for (int s = g; s < g + 2; ++s) {  // bytes, distance 2
            const uint32_t a = x[s], b = x[s + 2];
            x[s] = __builtin_amdgcn_perm(b, a, 0x06020400u);
            x[s + 2] = __builtin_amdgcn_perm(b, a, 0x07030501u);
        }
#pragma unroll
    for (int s = 0; s < 8; s += 2) {  // nibbles, distance 1
        const uint32_t a = x[s], b = x[s + 1];
        x[s] = (a & 0x0F0F0F0Fu) | ((b << 4) & 0xF0F0F0F0u);
        x[s + 1] = ((a >> 4) & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);
    }
}

// ------------------------------------------------------------------ GPTQ <-> AWQ in registers
// One thread per (GPTQ word row r, column group g of 8): GPTQ words
// [r][8g .. 8g+7] <-> AWQ words [8r + j][g], j < 8. R = K/8, G = N/8.
// VEC: the 8 GPTQ words are read / written as two 16-byte accesses.
template <bool VEC>
__global__ __launch_bounds__(256) void k_gptq_to_awq(const uint32_t *__restrict__ src, uint32_t *__restrict__ dst,
                                                     int64_t R, int64_t G) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= R * G) return;
    const int64_t r = i / G, g = i - r * G;
    const uint32_t *sp = src + r * (8 * G) + 8 * g;
    uint32_t a[8];
    if (VEC) {
        // read once: non-temporal (2.8% faster a step; the stores below too)
        const u32x4 lo = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(sp));
        const u32x4 hi = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(sp) + 1);
        a[0] = lo.x; a[1] = lo.y; a[2] = lo.z; a[3] = lo.w;
        a[4] = hi.x; a[5] = hi.y; a[6] = hi.z; a[7] = hi.w;
    } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) a[c] = sp[c];
    }
    // word s of the block = column awq_col(s); the transpose turns the
    // columns' row nibbles into the rows' slot nibbles
    uint32_t x[8];
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) x[s2] = a[awq_col(s2)];
    nib_transpose8(x);
#pragma unroll
    // non-temporal: lanes hold neighbouring words, so each store is one
    // contiguous run (11.1 -> 9.7 us for 4096 x 11008)
    for (int j = 0; j < 8; ++j) __builtin_nontemporal_store(x[j], dst + (8 * r + j) * G + g);
}

template <bool VEC>
__global__ __launch_bounds__(256) void k_awq_to_gptq(const uint32_t *__restrict__ src, uint32_t *__restrict__ dst,
                                                     int64_t R, int64_t G) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= R * G) return;
    const int64_t r = i / G, g = i - r * G;
    uint32_t x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = src[(8 * r + j) * G + g];
    nib_transpose8(x);  // x[s] = column awq_col(s), nibble j = row 8r + j
    uint32_t a[8];
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) a[awq_col(s2)] = x[s2];
    uint32_t *dp = dst + r * (8 * G) + 8 * g;
    if (VEC) {
        reinterpret_cast<u32x4 *>(dp)[0] = u32x4{a[0], a[1], a[2], a[3]};
        reinterpret_cast<u32x4 *>(dp)[1] = u32x4{a[4], a[5], a[6], a[7]};
    } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) dp[c] = a[c];
    }
}

// ------------------------------------------------------------------ Q4_0 blocks
// A column's 32 codes of one block as four words T[q] (nibble j = k 8q + j,
// the GPTQ word order) <-> the block's 16 code bytes as four words D[m]
// (byte i of D[m] = code 4m + i | code 4m + i + 16 << 4).
__device__ __forceinline__ uint32_t nib_spread(uint32_t x) {  // 4 nibbles -> low nibbles of 4 bytes
    x &= 0xFFFFu;
    x = (x | (x << 8)) & 0x00FF00FFu;
    return (x | (x << 4)) & 0x0F0F0F0Fu;
}
__device__ __forceinline__ uint32_t nib_compress(uint32_t x) {  // low nibbles of 4 bytes -> 16 bits
    x &= 0x0F0F0F0Fu;
    x = (x | (x >> 4)) & 0x00FF00FFu;
    return (x | (x >> 8)) & 0x0000FFFFu;
}
__device__ __forceinline__ void block_zip(const uint32_t *T, uint32_t *D) {
    D[0] = nib_spread(T[0]) | (nib_spread(T[2]) << 4);
    D[1] = nib_spread(T[0] >> 16) | (nib_spread(T[2] >> 16) << 4);
    D[2] = nib_spread(T[1]) | (nib_spread(T[3]) << 4);
    D[3] = nib_spread(T[1] >> 16) | (nib_spread(T[3] >> 16) << 4);
}
__device__ __forceinline__ void block_unzip(const uint32_t *D, uint32_t *T) {
    T[0] = nib_compress(D[0]) | (nib_compress(D[1]) << 16);
    T[2] = nib_compress(D[0] >> 4) | (nib_compress(D[1] >> 4) << 16);
    T[1] = nib_compress(D[2]) | (nib_compress(D[3]) << 16);
    T[3] = nib_compress(D[2] >> 4) | (nib_compress(D[3] >> 4) << 16);
}

// LDS staging of Q4_0 runs: run r (up to RB blocks of one column) at
// r * RS bytes; RS is an odd number of words, so consecutive lanes writing
// consecutive runs hit different banks.
constexpr int RB = 8;
constexpr int RS = RB * 18 + 4;

__device__ __forceinline__ void put_block(uint8_t *run, int b, uint16_t d, const uint32_t *D) {
    uint16_t *p = reinterpret_cast<uint16_t *>(run + 18 * b);
    p[0] = d;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        p[1 + 2 * m] = (uint16_t)D[m];
        p[2 + 2 * m] = (uint16_t)(D[m] >> 16);
    }
}
__device__ __forceinline__ void get_block(const uint8_t *run, int b, uint32_t *D) {
    const uint16_t *p = reinterpret_cast<const uint16_t *>(run + 18 * b);
#pragma unroll
    for (int m = 0; m < 4; ++m) D[m] = (uint32_t)p[1 + 2 * m] | ((uint32_t)p[2 + 2 * m] << 16);
}

// Moves NR staged runs between LDS and global memory; run r belongs to
// column col(r) (skipped when col(r) >= N) and holds blocks b0 .. b0+nb-1 of
// it, contiguous at (col * nbr + b0) * 18. Wave w moves runs w, w + 4, ...,
// BATCH runs at a time with all of a batch's loads issued before its stores.
// MODE 2: every run is a whole RB = 8 blocks (144 bytes, nine 16-byte
// pieces) starting on a 16-byte boundary (k % 256 == 0, 16-byte aligned
// base): lane l moves piece l % 9 of run l / 9, so one instruction moves 7
// runs; all of a wave's loads are issued before its stores. MODE 1 (WORDS):
// every run starts on a 4-byte boundary and has an even block count (a run
// is then at most 36 words, one per lane); MODE 0: 2-byte units.
struct alignas(4) Piece16 {  // 16 bytes at a 4-byte aligned LDS address (runs sit RS apart)
    uint32_t v[4];
};

template <bool TO_LDS, int NR, typename ColOf>
__device__ __forceinline__ void move_runs(uint8_t *lds, uint8_t *__restrict__ blocks, ColOf col, int64_t N,
                                          int64_t nbr, int64_t b0, int nb, int mode) {
    constexpr int PER_WAVE = NR / 4;
    constexpr int BATCH = PER_WAVE < 16 ? PER_WAVE : 16;
    static_assert(NR % (4 * BATCH) == 0, "whole batches");
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
    if (mode == 2) {
        constexpr int IT = (NR + 27) / 28;  // 4 waves x 7 runs per step
        const int j = lane / 9, pc = lane % 9;
        u32x4 v[IT];
        bool ok[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int r = 28 * it + 7 * wave + j;
            ok[it] = j < 7 && r < NR && col(r < NR ? r : 0) < N;
            if (ok[it]) {
                if (TO_LDS) {
                    v[it] = reinterpret_cast<const u32x4 *>(blocks + (col(r) * nbr + b0) * 18)[pc];
                } else {
                    const Piece16 q = *reinterpret_cast<const Piece16 *>(lds + r * RS + 16 * pc);
                    v[it] = u32x4{q.v[0], q.v[1], q.v[2], q.v[3]};
                }
            }
        }
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int r = 28 * it + 7 * wave + j;
            if (ok[it]) {
                if (TO_LDS) {
                    Piece16 q;
                    q.v[0] = v[it].x, q.v[1] = v[it].y, q.v[2] = v[it].z, q.v[3] = v[it].w;
                    *reinterpret_cast<Piece16 *>(lds + r * RS + 16 * pc) = q;
                } else {
                    // non-temporal: the 144-byte runs are written once (AWQ -> Q4_0
                    // 21.9 -> 21.4 us a step)
                    __builtin_nontemporal_store(v[it], reinterpret_cast<u32x4 *>(blocks + (col(r) * nbr + b0) * 18) + pc);
                }
            }
        }
        return;
    }
    const bool words = mode != 0;
    const int L = nb * 18;
    for (int r0 = wave; r0 < NR; r0 += 4 * BATCH) {
        if (words) {
            uint32_t v[BATCH];
            uint32_t *gp[BATCH];
            bool ok[BATCH];
#pragma unroll
            for (int i = 0; i < BATCH; ++i) {
                const int r = r0 + 4 * i;
                const int64_t n = col(r);
                ok[i] = n < N && lane < L / 4;
                gp[i] = reinterpret_cast<uint32_t *>(blocks + (n * nbr + b0) * 18) + lane;
                uint32_t *lp = reinterpret_cast<uint32_t *>(lds + r * RS) + lane;
                v[i] = ok[i] ? (TO_LDS ? *gp[i] : *lp) : 0u;
            }
#pragma unroll
            for (int i = 0; i < BATCH; ++i) {
                uint32_t *lp = reinterpret_cast<uint32_t *>(lds + (r0 + 4 * i) * RS) + lane;
                if (ok[i]) {
                    if (TO_LDS) *lp = v[i];
                    else __builtin_nontemporal_store(v[i], gp[i]);
                }
            }
        } else {
#pragma unroll
            for (int h = 0; h < 2; ++h) {  // a run is at most 72 halfwords
                const int u = lane + 64 * h;
                uint16_t v[BATCH];
                uint16_t *gp[BATCH];
                bool ok[BATCH];
#pragma unroll
                for (int i = 0; i < BATCH; ++i) {
                    const int r = r0 + 4 * i;
                    const int64_t n = col(r);
                    ok[i] = n < N && u < L / 2;
                    gp[i] = reinterpret_cast<uint16_t *>(blocks + (n * nbr + b0) * 18) + u;
                    uint16_t *lp = reinterpret_cast<uint16_t *>(lds + r * RS) + u;
                    v[i] = ok[i] ? (TO_LDS ? *gp[i] : *lp) : (uint16_t)0;
                }
#pragma unroll
                for (int i = 0; i < BATCH; ++i) {
                    uint16_t *lp = reinterpret_cast<uint16_t *>(lds + (r0 + 4 * i) * RS) + u;
                    if (ok[i]) {
                        if (TO_LDS) *lp = v[i];
                        else __builtin_nontemporal_store(v[i], gp[i]);
                    }
                }
            }
        }
    }
}

// The Q4_0 kernels run after a refusal scan that has left its partial minima
// in parts[0 .. QBN_REPACK_SCAN_PARTS - 1] (kNone where nothing was found).
// Every workgroup takes their minimum (the same for all, so the whole grid
// agrees), workgroup 0 publishes it as *result (-1 for none), and on a
// refusal every workgroup leaves before writing anything.
constexpr unsigned long long kNone = 0x7FFFFFFFFFFFFFFFull;

// The scan's minimum: one part per lane (there are as many parts as lanes),
// then a butterfly minimum across the wave, so every lane of every wave
// holds it.
static_assert(QBN_REPACK_SCAN_PARTS == kWave, "one refusal-scan part per lane");
__device__ __forceinline__ unsigned long long refusal_min(const int64_t *parts) {
    unsigned long long m = (unsigned long long)parts[threadIdx.x & (kWave - 1)];
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
        const unsigned long long o = __shfl_xor(m, off, kWave);
        m = o < m ? o : m;
    }
    return m;
}

// Workgroup 0 publishes the scan's result; true means refused. The kernels
// read the parts first and ask this just before their first global store,
// so the parts' latency overlaps their own loads; nothing is stored on a
// refusal.
__device__ __forceinline__ bool refused(unsigned long long m, int64_t *result) {
    if (blockIdx.x == 0 && threadIdx.x == 0) *result = (m == kNone) ? -1 : (int64_t)m;
    return m != kNone;
}

// Workgroup tiles: RB consecutive blocks (RB * 32 k) of 64 columns (GPTQ
// side) or of 256 columns = 32 AWQ word columns (AWQ side); blockIdx.x runs
// fastest along k so the runs of one column are completed together.
// GPTQ tile: thread (c = t % 64, i = t / 64) handles blocks i and i + 4.
__global__ __launch_bounds__(256) void k_gptq_to_q4_0(const uint32_t *__restrict__ src,
                                                      const uint16_t *__restrict__ scales, int64_t group,
                                                      uint8_t *__restrict__ dst, int64_t N, int64_t K, int words,
                                                      const int64_t *__restrict__ parts, int64_t *__restrict__ result) {
    const unsigned long long rm = refusal_min(parts);
    __shared__ __attribute__((aligned(16))) uint8_t runs[64 * RS];
    const int64_t nbr = K / 32, nbt = (nbr + RB - 1) / RB;
    const int64_t b0 = (int64_t)(blockIdx.x % nbt) * RB, n0 = (int64_t)(blockIdx.x / nbt) * 64;
    const int nb = (int)((nbr - b0) < RB ? (nbr - b0) : RB);
    const int c = threadIdx.x % 64;
    const int64_t n = n0 + c;
    if (n < N) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int b = threadIdx.x / 64 + 4 * h;
            if (b >= nb) continue;
            const int64_t bg = b0 + b;
            uint32_t T[4], D[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) T[q] = src[(4 * bg + q) * N + n];
            block_zip(T, D);
            put_block(runs + c * RS, b, scales[((32 * bg) / group) * N + n], D);
        }
    }
    if (refused(rm, result)) return;  // the whole grid leaves: nothing is written
    __syncthreads();
    move_runs<false, 64>(runs, dst, [&](int r) { return n0 + r; }, N, nbr, b0, nb, words);
}

// Q4_0 -> GPTQ / AWQ also write the companions of the target: for every
// group (group / 32 consecutive blocks of a column) the scale is the bit
// pattern of its first block's d and the zero point is 8.
__global__ __launch_bounds__(256) void k_q4_0_to_gptq(const uint8_t *__restrict__ src, uint32_t *__restrict__ dst,
                                                      uint16_t *__restrict__ gscales, uint8_t *__restrict__ gzeros,
                                                      int64_t group, int64_t N, int64_t K, int words,
                                                      const int64_t *__restrict__ parts, int64_t *__restrict__ result) {
    const unsigned long long rm = refusal_min(parts);
    __shared__ __attribute__((aligned(16))) uint8_t runs[64 * RS];
    const int64_t nbr = K / 32, nbt = (nbr + RB - 1) / RB;
    const int64_t b0 = (int64_t)(blockIdx.x % nbt) * RB, n0 = (int64_t)(blockIdx.x / nbt) * 64;
    const int nb = (int)((nbr - b0) < RB ? (nbr - b0) : RB);
    move_runs<true, 64>(runs, const_cast<uint8_t *>(src), [&](int r) { return n0 + r; }, N, nbr, b0, nb,
                        words);
    __syncthreads();
    if (refused(rm, result)) return;
    const int c = threadIdx.x % 64;
    const int64_t n = n0 + c;
    if (n >= N) return;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int b = threadIdx.x / 64 + 4 * h;
        if (b >= nb) continue;
        const int64_t bg = b0 + b;
        uint32_t T[4], D[4];
        get_block(runs + c * RS, b, D);
        block_unzip(D, T);
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[(4 * bg + q) * N + n] = T[q];
        if ((32 * bg) % group == 0) {
            const int64_t gi = (32 * bg) / group;
            gscales[gi * N + n] = *reinterpret_cast<const uint16_t *>(runs + c * RS + 18 * b);
            gzeros[gi * N + n] = 8;
        }
    }
}

// AWQ tile: thread (g = t % 32, b = t / 32) reads the 32 AWQ words of block
// b of word column g0 + g; run 32 s + g holds column 8 (g0 + g) + awq_col(s).
__global__ __launch_bounds__(256) void k_awq_to_q4_0(const uint32_t *__restrict__ src,
                                                     const uint16_t *__restrict__ scales, int64_t group,
                                                     uint8_t *__restrict__ dst, int64_t N, int64_t K, int words,
                                                     const int64_t *__restrict__ parts, int64_t *__restrict__ result) {
    const unsigned long long rm = refusal_min(parts);
    __shared__ __attribute__((aligned(16))) uint8_t runs[256 * RS];
    const int64_t G = N / 8, nbr = K / 32, nbt = (nbr + RB - 1) / RB;
    const int64_t b0 = (int64_t)(blockIdx.x % nbt) * RB, g0 = (int64_t)(blockIdx.x / nbt) * 32;
    const int nb = (int)((nbr - b0) < RB ? (nbr - b0) : RB);
    const int g = threadIdx.x % 32, b = threadIdx.x / 32;
    if (g0 + g < G && b < nb) {
        const int64_t bg = b0 + b;
        uint32_t x[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) x[j] = src[(32 * bg + j) * G + g0 + g];
        // rows 8q .. 8q+7 -> T[q][s] = column awq_col(s), nibble j = row 8q + j
#pragma unroll
        for (int q = 0; q < 4; ++q) nib_transpose8(x + 8 * q);
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) {
            const int64_t n = 8 * (g0 + g) + awq_col(s2);
            const uint32_t T[4] = {x[s2], x[8 + s2], x[16 + s2], x[24 + s2]};
            uint32_t D[4];
            block_zip(T, D);
            put_block(runs + (32 * s2 + g) * RS, b, scales[((32 * bg) / group) * N + n], D);
        }
    }
    if (refused(rm, result)) return;
    __syncthreads();
    move_runs<false, 256>(runs, dst, [&](int r) { return 8 * (g0 + r % 32) + awq_col(r / 32); }, N, nbr, b0, nb,
                          words);
}

__global__ __launch_bounds__(256) void k_q4_0_to_awq(const uint8_t *__restrict__ src, uint32_t *__restrict__ dst,
                                                     uint16_t *__restrict__ gscales, uint8_t *__restrict__ gzeros,
                                                     int64_t group, int64_t N, int64_t K, int words,
                                                     const int64_t *__restrict__ parts, int64_t *__restrict__ result) {
    const unsigned long long rm = refusal_min(parts);
    __shared__ __attribute__((aligned(16))) uint8_t runs[256 * RS];
    const int64_t G = N / 8, nbr = K / 32, nbt = (nbr + RB - 1) / RB;
    const int64_t b0 = (int64_t)(blockIdx.x % nbt) * RB, g0 = (int64_t)(blockIdx.x / nbt) * 32;
    const int nb = (int)((nbr - b0) < RB ? (nbr - b0) : RB);
    move_runs<true, 256>(runs, const_cast<uint8_t *>(src),
                         [&](int r) { return 8 * (g0 + r % 32) + awq_col(r / 32); }, N, nbr, b0, nb, words);
    __syncthreads();
    if (refused(rm, result)) return;
    const int g = threadIdx.x % 32, b = threadIdx.x / 32;
    if (g0 + g >= G || b >= nb) return;
    const int64_t bg = b0 + b;
    uint32_t x[32];
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) {
        uint32_t D[4], T[4];
        get_block(runs + (32 * s2 + g) * RS, b, D);
        block_unzip(D, T);
#pragma unroll
        for (int q = 0; q < 4; ++q) x[8 * q + s2] = T[q];
    }
    if ((32 * bg) % group == 0) {
        const int64_t gi = (32 * bg) / group;
#pragma unroll
        for (int c = 0; c < 8; ++c) {  // column 8 (g0 + g) + c sits in slot awq_slot(c)
            const int sl = (c % 2 == 0) ? c / 2 : 4 + c / 2;
            gscales[gi * N + 8 * (g0 + g) + c] = *reinterpret_cast<const uint16_t *>(runs + (32 * sl + g) * RS + 18 * b);
            gzeros[gi * N + 8 * (g0 + g) + c] = 8;
        }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) nib_transpose8(x + 8 * q);  // x[8q + j] = AWQ word of row 8q + j
#pragma unroll
    for (int j = 0; j < 32; ++j) dst[(32 * bg + j) * G + g0 + g] = x[j];
}

}  // namespace

// Scratch of the allocation-free repack (qbn_repack_noalloc): the partial
// results of the refusal scan, one copy per GPU in file-scope device memory,
// held until the process ends. The scan writes every word on every call, so
// nothing in it has to be cleared; calls that overlap on one GPU race on it.
static __device__ __align__(256) int64_t scratch[QBN_REPACK_SCAN_PARTS];

hipError_t repack_scratch(int64_t **parts) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static int64_t *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        // the symbol's address on the current device; the host-side name
        // `scratch` is never passed to a kernel
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = static_cast<int64_t *>(p);
    }
    *parts = addr[dev];
    return hipSuccess;
}

hipError_t launch_repack(const qbn_tensor &src, const qbn_tensor &dst, int64_t *parts, int64_t *result,
                         hipStream_t s) {
    const int64_t N = src.n, K = src.k;
    const int sf = src.format, df = dst.format;
    void *const dst_data = const_cast<void *>(dst.data);
    const dim3 blk(256);
    if ((sf == QBN_GPTQ4 && df == QBN_AWQ4) || (sf == QBN_AWQ4 && df == QBN_GPTQ4)) {
        // one thread per 8 x 8 block of codes
        const int64_t R = K / 8, G = N / 8, cnt = R * G;
        if (cnt > 0) {
            const void *gp = sf == QBN_GPTQ4 ? src.data : dst_data;  // the GPTQ side
            const bool vec = (reinterpret_cast<uintptr_t>(gp) % 16) == 0;
            const dim3 grid((unsigned)((cnt + 255) / 256));
            const uint32_t *sp = (const uint32_t *)src.data;
            uint32_t *dp = (uint32_t *)dst_data;
            if (sf == QBN_GPTQ4) {
                if (vec) hipLaunchKernelGGL(k_gptq_to_awq<true>, grid, blk, 0, s, sp, dp, R, G);
                else hipLaunchKernelGGL(k_gptq_to_awq<false>, grid, blk, 0, s, sp, dp, R, G);
            } else {
                if (vec) hipLaunchKernelGGL(k_awq_to_gptq<true>, grid, blk, 0, s, sp, dp, R, G);
                else hipLaunchKernelGGL(k_awq_to_gptq<false>, grid, blk, 0, s, sp, dp, R, G);
            }
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        // scales and zero points keep their [K/group][N] layout
        const int64_t gcnt = (K / src.group) * N;
        hipError_t e = hipSuccess;
        if (dst.scales != src.scales && gcnt > 0)
            e = hipMemcpyAsync(const_cast<void *>(dst.scales), src.scales, 2 * gcnt, hipMemcpyDeviceToDevice, s);
        if (e == hipSuccess && dst.zeros != src.zeros && gcnt > 0)
            e = hipMemcpyAsync(const_cast<void *>(dst.zeros), src.zeros, gcnt, hipMemcpyDeviceToDevice, s);
        return e;
    }
    const bool to_q4 = df == QBN_Q4_0;
    if (!(to_q4 ? (sf == QBN_GPTQ4 || sf == QBN_AWQ4) : (sf == QBN_Q4_0 && (df == QBN_GPTQ4 || df == QBN_AWQ4))))
        return hipErrorInvalidValue;
    // refusal scan: every zero point must be 8 (to Q4_0), or every block of a
    // target group must carry the same d (from Q4_0)
    hipError_t e = to_q4 ? launch_scan_zero_points((const uint8_t *)src.zeros, (K / src.group) * N, parts, s)
                         : launch_scan_q4_0_groups((const uint8_t *)src.data, N, K, dst.group, parts, s);
    if (e != hipSuccess) return e;
    const int64_t nbr = K / 32, nbt = (nbr + RB - 1) / RB;
    // Q4_0 runs move as 4-byte words when every run starts and ends on a
    // word: an even block count per column (then every tile's count is even
    // too) and a word-aligned base.
    const void *q4 = to_q4 ? dst_data : src.data;
    // 16-byte pieces (mode 2) when every run is 8 whole blocks on a 16-byte
    // boundary: (n nbr + b0) * 18 is a multiple of 144 when nbr % 8 == 0
    const int words = ((nbr % RB == 0) && (reinterpret_cast<uintptr_t>(q4) % 16 == 0)) ? 2
                      : ((nbr % 2 == 0) && (reinterpret_cast<uintptr_t>(q4) % 4 == 0)) ? 1
                                                                                        : 0;
    const bool awq = (sf == QBN_AWQ4) || (df == QBN_AWQ4);
    const int64_t ntile = awq ? (N / 8 + 31) / 32 : (N + 63) / 64;
    const int64_t tiles = nbt * ntile;
    if (tiles > 0) {
        const dim3 grid((unsigned)tiles);
        uint16_t *const gs = (uint16_t *)const_cast<void *>(dst.scales);
        uint8_t *const gz = (uint8_t *)const_cast<void *>(dst.zeros);
        if (sf == QBN_GPTQ4)
            hipLaunchKernelGGL(k_gptq_to_q4_0, grid, blk, 0, s, (const uint32_t *)src.data,
                               (const uint16_t *)src.scales, (int64_t)src.group, (uint8_t *)dst_data, N, K, words,
                               parts, result);
        else if (sf == QBN_AWQ4)
            hipLaunchKernelGGL(k_awq_to_q4_0, grid, blk, 0, s, (const uint32_t *)src.data,
                               (const uint16_t *)src.scales, (int64_t)src.group, (uint8_t *)dst_data, N, K, words,
                               parts, result);
        else if (df == QBN_GPTQ4)
            hipLaunchKernelGGL(k_q4_0_to_gptq, grid, blk, 0, s, (const uint8_t *)src.data, (uint32_t *)dst_data, gs,
                               gz, (int64_t)dst.group, N, K, words, parts, result);
        else
            hipLaunchKernelGGL(k_q4_0_to_awq, grid, blk, 0, s, (const uint8_t *)src.data, (uint32_t *)dst_data, gs,
                               gz, (int64_t)dst.group, N, K, words, parts, result);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace qbn
