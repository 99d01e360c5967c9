// Prefill GEMM straight from the integer int4 layouts ("Bit Packing
// Architecture", 'Real layouts compared'; "Why 4-Bit Quantization Is King",
// section 7: a weight-only W4 kernel keeps B packed, decodes each tile,
// applies the scales and accumulates in a wider type):
//   Y[m][n] = sum_k X[m][k] * W_hat[k][n],  X bf16 [M][ldx], Y bf16 or f32,
//   GPTQ4 / AWQ4: W_hat = s[k/g][n] * (q - z[k/g][n]);
//   Q4_0:         W_hat = d[n][k/32] * (q - 8).
//
// s * (q - z) is exact in binary32 but not in bf16 (an fp16 scale has 11
// significant bits), so the scale stays out of the matrix core: each tile of
// codes is decoded once per workgroup into LDS as bf16 (q - z), a small
// integer and exact, and v_mfma_f32_32x32x16_bf16 sums X (q - z) over each
// 32-long sub-block of k into a partial accumulator. At the end of every
// group whose size is a multiple of 64, and otherwise at the end of every
// 32-k sub-block (Q4_0, groups of 32, 96, ...), the partial is multiplied by
// its column's scale and added to the running total, so every product is
// exact and each output sees k/16 MFMA steps plus k/group (or k/32) scaled
// additions in binary32.
//
// Tiling: workgroup 128 x 128 of Y, four waves in 2 x 2, each 64 x 64 (2 x 2
// MFMA tiles); k advances 64 at a time. The next tile's X, codes, zero points
// and scales are loaded into registers while the current one is multiplied
// from LDS (two buffers, one barrier per k-tile). Columns of a 32-k sub-block
// take their scale from LDS, written by the thread that loaded it.
//
// Codes decode with the binary16-subnormal trick: masked bits read as fp16
// are q * 2^-24 (or 16 q * 2^-24 for the upper nibble of a byte), and one
// mixed fma per code returns q - z exactly in binary32; the upper halves of
// two such values are their bf16 encodings.
#include "qbn_device.h"
#include "qbn_launch.h"

namespace qbn {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kThreads = 256;
constexpr int LDK = BK + 8;  // LDS row pitch in bf16 (16 bytes of padding against bank conflicts)

struct alignas(16) Smem {
    alignas(16) uint16_t a[2][BM * LDK];  // X tile, [m][k]
    alignas(16) uint16_t b[2][BN * LDK];  // decoded codes (q - z) as bf16, [n][k]
    alignas(16) float s[2][2][BN];        // scale of each column for the tile's two 32-k sub-blocks
};

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t *p) { return *reinterpret_cast<const bf16x8 *>(p); }

// bf16 encodings of two exactly representable binary32 values, lo first.
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// q_m - z[m] for the eight nibbles of a word (bits 4m .. 4m+3), exact.
__device__ __forceinline__ void nibbles_minus(uint32_t v, const float (&z)[8], float (&w)[8]) {
    const uint32_t v8 = v >> 8;
    const f16x2 p0 = __builtin_bit_cast(f16x2, v & 0x000F000Fu);   // nibbles 0, 4
    const f16x2 p1 = __builtin_bit_cast(f16x2, v8 & 0x000F000Fu);  // nibbles 2, 6
    const f16x2 p2 = __builtin_bit_cast(f16x2, v & 0x00F000F0u);   // 16 x nibbles 1, 5
    const f16x2 p3 = __builtin_bit_cast(f16x2, v8 & 0x00F000F0u);  // 16 x nibbles 3, 7
    w[0] = __builtin_fmaf((float)p0.x, 0x1p24f, -z[0]);
    w[4] = __builtin_fmaf((float)p0.y, 0x1p24f, -z[4]);
    w[2] = __builtin_fmaf((float)p1.x, 0x1p24f, -z[2]);
    w[6] = __builtin_fmaf((float)p1.y, 0x1p24f, -z[6]);
    w[1] = __builtin_fmaf((float)p2.x, 0x1p20f, -z[1]);
    w[5] = __builtin_fmaf((float)p2.y, 0x1p20f, -z[5]);
    w[3] = __builtin_fmaf((float)p3.x, 0x1p20f, -z[3]);
    w[7] = __builtin_fmaf((float)p3.y, 0x1p20f, -z[7]);
}

__device__ __forceinline__ float f16_to_f32(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }

// An 18-byte Q4_0 block (2-byte aligned; its dwords are read unaligned).
struct __attribute__((packed, aligned(2))) Q40B {
    uint16_t d;
    uint32_t c[4];
};

// ------------------------------------------------------------------ stage
// X: thread t loads rows t/8 + 32i (i < 4), 16 bytes at k chunk t % 8.
// Codes (per format):
//   GPTQ4: word row r = t%8 (k = 8r .. 8r+7 of the tile), 4 columns 4(t/8) .. +3
//          (lanes step along the word rows first: the 16-byte LDS stores of
//          a wave then cover all 16 bank slots);
//   AWQ4:  k rows 4(t%16) .. +3, word column t / 16 (columns 8(t/16) .. +7):
//          consecutive lanes step along k, so the 8-byte LDS stores of a wave
//          fill 256 distinct bytes (with lanes stepping along n instead, the
//          1152-byte column stride folded them onto two bank offsets);
//   Q4_0:  block t % 2 (k = 32(t%2) .. +31) of column t / 2.
// Scales for LDS: GPTQ4 / AWQ4 thread t writes column t % 128 of sub-block
// t / 128; Q4_0 its own block's d.
template <int FMT>
struct Stage {
    u32x4 a[4];
    uint32_t w[4];  // GPTQ4 / AWQ4 words; Q4_0: the 16 code bytes
    uint32_t zb[2]; // GPTQ4: 4 zero points (bytes); AWQ4: 8 (two words)
    float s;        // scale destined for LDS
};

struct Args {
    const uint16_t *X;
    int64_t ldx;
    const uint8_t *data;
    const uint16_t *scales;
    const uint8_t *zeros;
    int64_t group;
    void *Y;
    int64_t ldy;
    int64_t M, N, K;
};

// Group of element k0 + off (0 <= off < 64) of a k-tile whose first element
// lies in group g0 at offset rem0 (a multiple of 32, at most group - 32): the
// tile crosses at most two group boundaries, so two compares replace a
// division.
__device__ __forceinline__ int64_t group_of(int64_t g0, int64_t rem0, int64_t group, int off) {
    const int64_t r = rem0 + off;
    return g0 + (r >= group ? 1 : 0) + (r >= 2 * group ? 1 : 0);
}

// Every load below reads a valid address: an index outside the operand is
// replaced by 0 and the loaded value by 0 (selects, not branches).
// VEC (n % 8 == 0, 16-byte aligned codes, 8-byte aligned zero points): GPTQ
// reads its four words in one 16-byte load and its four zero points in one
// dword; AWQ its eight zero points in one 8-byte load.
template <int FMT, bool VEC, bool XB = false>
__device__ __forceinline__ void stage_load(Stage<FMT> &st, const Args &p, int64_t m0, int64_t n0, int64_t k0,
                                           int64_t g0, int64_t rem0, const uint32_t (&xo)[4],
                                           __amdgpu_buffer_rsrc_t rx) {
    const int t = threadIdx.x;
    if constexpr (XB) {  // k % 64 == 0: X through its descriptor, rows past m read as 0
#pragma unroll
        for (int i = 0; i < 4; ++i)
            st.a[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, xo[i], (int)(k0 * 2), 0));
    } else {
        const int c16 = t % 8;
        const int64_t k = k0 + 8 * c16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t m = m0 + t / 8 + 32 * i;
            const bool ok = m < p.M && k < p.K;
            const u32x4 v = ld16(p.X + (ok ? m * p.ldx + k : 0));
            st.a[i] = ok ? v : u32x4{0u, 0u, 0u, 0u};
        }
    }
    if (FMT == QBN_GPTQ4) {
        const int r = t % 8;
        const int64_t kk = k0 + 8 * r;
        const int64_t n = n0 + 4 * (t / 8);
        const bool kok = kk < p.K;
        const int64_t g = kok ? group_of(g0, rem0, p.group, 8 * r) : 0;
        const uint32_t *src = reinterpret_cast<const uint32_t *>(p.data);
        if (VEC) {  // n % 4 == 0 here, so the four columns are all in or all out
            const bool ok = kok && n < p.N;
            const u32x4 w = *reinterpret_cast<const u32x4 *>(src + (ok ? (kk / 8) * p.N + n : 0));
            const uint32_t z = *reinterpret_cast<const uint32_t *>(p.zeros + (ok ? g * p.N + n : 0));
            st.w[0] = ok ? w.x : 0u;
            st.w[1] = ok ? w.y : 0u;
            st.w[2] = ok ? w.z : 0u;
            st.w[3] = ok ? w.w : 0u;
            st.zb[0] = ok ? z : 0u;
        } else {
            uint32_t zz = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = kok && (n + i < p.N);
                const uint32_t w = src[ok ? (kk / 8) * p.N + n + i : 0];
                const uint32_t z = p.zeros[ok ? g * p.N + n + i : 0];
                st.w[i] = ok ? w : 0u;
                zz |= (ok ? z : 0u) << (8 * i);
            }
            st.zb[0] = zz;
        }
    } else if (FMT == QBN_AWQ4) {
        const int h = t % 16, c = t / 16;
        const int64_t n = n0 + 8 * c;
        const int64_t kk = k0 + 4 * h;
        const bool nok = n < p.N;
        const int64_t g = kk < p.K ? group_of(g0, rem0, p.group, 4 * h) : 0;
        const uint32_t *src = reinterpret_cast<const uint32_t *>(p.data);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = nok && kk + i < p.K;
            const uint32_t w = src[ok ? (kk + i) * (p.N / 8) + n / 8 : 0];
            st.w[i] = ok ? w : 0u;
        }
        const uint8_t *zp = p.zeros + (nok ? g * p.N + n : 0);
        uint32_t z0 = 0, z1 = 0;
        if (VEC) {
            const u32x2 z = *reinterpret_cast<const u32x2 *>(zp);
            z0 = z.x;
            z1 = z.y;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                z0 |= (uint32_t)zp[j] << (8 * j);
                z1 |= (uint32_t)zp[4 + j] << (8 * j);
            }
        }
        st.zb[0] = nok ? z0 : 0u;
        st.zb[1] = nok ? z1 : 0u;
    } else {  // Q4_0
        const int64_t n = n0 + t / 2;
        const int64_t b = k0 / 32 + (t % 2);
        const bool ok = n < p.N && 32 * b < p.K;
        const Q40B blk = *reinterpret_cast<const Q40B *>(p.data + (ok ? (n * (p.K / 32) + b) * 18 : 0));
#pragma unroll
        for (int i = 0; i < 4; ++i) st.w[i] = ok ? blk.c[i] : 0u;
        st.s = ok ? f16_to_f32(blk.d) : 0.0f;
    }
    if (FMT != QBN_Q4_0) {
        const int sb = t / 128;
        const int64_t n = n0 + t % 128;
        const int64_t kk = k0 + 32 * sb;
        const bool ok = n < p.N && kk < p.K;
        const float v = f16_to_f32(p.scales[ok ? group_of(g0, rem0, p.group, 32 * sb) * p.N + n : 0]);
        st.s = ok ? v : 0.0f;
    }
}

// Buffer-resource path (k % 64 == 0; GPTQ4 / AWQ4 in the VEC layout, or
// Q4_0 with dword-aligned blocks; every operand under 2 GiB). Each lane's
// byte offsets into X, the codes, the zero points and the scales are fixed
// for the whole k loop; a k-tile only moves the uniform offset (k0 and its
// group), which the buffer loads take in a scalar register. With groups that
// are not a multiple of 64 a tile spans two groups, and a lane whose rows lie
// in the second adds one group row to its zero-point and scale offsets. No
// guards: k % 64 == 0, rows past m lie beyond the X descriptor's range and
// read as 0, and columns past n feed only outputs that are never stored.
struct BufOffsets {
    uint32_t x[4];  // X row t/8 + 32i of the tile, chunk t % 8
    uint32_t w;     // GPTQ: word row t % 8, columns 4(t/8)..; AWQ: rows 4(t%16).., word column t/16
    uint32_t z;     // zero points of this thread's columns, group 0
    uint32_t sc;    // scale of column t % 128, group 0
};

constexpr int32_t kRsrcWord3 = 0x00020000;  // raw buffer descriptor, gfx9 family

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, kRsrcWord3);
}

// The range check of a buffer load covers the lane's offset but not the
// uniform one, which carries the k-tile and the group; so lanes whose
// columns lie past n take the offsets of the last valid columns (their
// outputs are never stored) rather than reading past the end of the codes,
// zero points or scales on the last k-tile or group.
template <int FMT>
__device__ __forceinline__ BufOffsets buf_offsets(const Args &p, int64_t m0, int64_t n0) {
    const int t = threadIdx.x;
    BufOffsets o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o.x[i] = (uint32_t)(((m0 + t / 8 + 32 * i) * p.ldx + 8 * (t % 8)) * 2);
    if (FMT == QBN_GPTQ4) {
        const int64_t n = min(n0 + 4 * (t / 8), p.N - 4);  // n % 8 == 0 on this path
        o.w = (uint32_t)(((t % 8) * p.N + n) * 4);
        o.z = (uint32_t)n;
    } else if (FMT == QBN_Q4_0) {
        // block (column n0 + t/2, t % 2) of the first k-tile; with k % 64 == 0 a
        // block starts 2 bytes past a dword boundary exactly when t is odd, so
        // the dword-aligned read starts at the block (t even) or 2 bytes before it
        const int64_t n = min(n0 + t / 2, p.N - 1);
        o.w = (uint32_t)((n * (p.K / 32) + (t % 2)) * 18 - 2 * (t % 2));
        o.z = 0;
    } else {
        const int64_t n = min(n0 + 8 * (t / 16), p.N - 8);
        o.w = (uint32_t)(((4 * (t % 16)) * (p.N / 8) + n / 8) * 4);
        o.z = (uint32_t)n;
    }
    o.sc = (uint32_t)(min(n0 + t % 128, p.N - 1) * 2);
    return o;
}

template <int FMT, bool PG>
__device__ __forceinline__ void stage_load_buf(Stage<FMT> &st, const Args &p, const BufOffsets &o,
                                               __amdgpu_buffer_rsrc_t rx, __amdgpu_buffer_rsrc_t rw,
                                               __amdgpu_buffer_rsrc_t rz, __amdgpu_buffer_rsrc_t rs, int64_t k0,
                                               int64_t g, int64_t rem0) {
    // PG (group % 64 == 0): the whole tile lies in group g. Otherwise
    // rem0 + off < 2 group for every offset off < 64 of the tile (rem0 < group,
    // and rem0 == 0 when group == 32), so a lane's group is g or g + 1.
    const uint32_t t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        st.a[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, o.x[i], (int)(k0 * 2), 0));
    const int zoff = (int)(g * p.N);
    if (FMT == QBN_Q4_0) {
        // 20 dword-aligned bytes covering the 18-byte block (see buf_offsets)
        const int soff = (int)((k0 / 32) * 18);
        const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, o.w, soff, 0));
        const uint32_t e = __builtin_amdgcn_raw_buffer_load_b32(rw, o.w + 16, soff, 0);
        const bool odd = (t & 1) != 0;
        const uint32_t dw[5] = {a.x, a.y, a.z, a.w, e};
#pragma unroll
        for (int i = 0; i < 4; ++i)  // odd: codes start on dword 1; even: 2 bytes into dword 0
            st.w[i] = odd ? dw[i + 1] : __builtin_amdgcn_alignbyte(dw[i + 1], dw[i], 2);
        st.s = f16_to_f32(odd ? (a.x >> 16) : (a.x & 0xFFFFu));
        return;
    }
    if (FMT == QBN_GPTQ4) {
        const u32x4 w = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, o.w, (int)((k0 / 8) * p.N * 4), 0));
        st.w[0] = w.x;
        st.w[1] = w.y;
        st.w[2] = w.z;
        st.w[3] = w.w;
        const uint32_t dz = !PG && rem0 + 8 * (t % 8) >= p.group ? (uint32_t)p.N : 0u;
        st.zb[0] = __builtin_amdgcn_raw_buffer_load_b32(rz, o.z + dz, zoff, 0);
    } else {
        const int base = (int)(k0 * (p.N / 8) * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            st.w[i] = __builtin_amdgcn_raw_buffer_load_b32(rw, o.w + (uint32_t)(i * (p.N / 8) * 4), base, 0);
        const uint32_t dz = !PG && rem0 + 4 * (t % 16) >= p.group ? (uint32_t)p.N : 0u;
        const u32x2 z = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rz, o.z + dz, zoff, 0));
        st.zb[0] = z.x;
        st.zb[1] = z.y;
    }
    const uint32_t ds = !PG && rem0 + 32 * (t / 128) >= p.group ? 2 * (uint32_t)p.N : 0u;
    const uint32_t sv = __builtin_amdgcn_raw_buffer_load_b16(rs, o.sc + ds, zoff * 2, 0);
    st.s = f16_to_f32(sv);
}

// NARROW (AWQ4): each row pair of a column goes to LDS on its own (4-byte
// stores) as soon as it is decoded, instead of both pairs in one 8-byte
// store; fewer live registers, which the per-32-k rescale path needs.
template <int FMT, bool NARROW = false>
__device__ __forceinline__ void stage_store(const Stage<FMT> &st, Smem &sm, int buf) {
    const int t = threadIdx.x;
    {
        const int c16 = t % 8;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<u32x4 *>(&sm.a[buf][(t / 8 + 32 * i) * LDK + 8 * c16]) = st.a[i];
    }
    if (FMT == QBN_GPTQ4) {
        const int r = t % 8;
        const int c = 4 * (t / 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float z = (float)((st.zb[0] >> (8 * i)) & 0xFFu);
            const float zz[8] = {z, z, z, z, z, z, z, z};
            float v[8];
            nibbles_minus(st.w[i], zz, v);  // k = 8r + m
            *reinterpret_cast<u32x4 *>(&sm.b[buf][(c + i) * LDK + 8 * r]) =
                u32x4{bf16_pair(v[0], v[1]), bf16_pair(v[2], v[3]), bf16_pair(v[4], v[5]), bf16_pair(v[6], v[7])};
        }
        sm.s[buf][t / 128][t % 128] = st.s;
    } else if (FMT == QBN_AWQ4) {
        const int h = t % 16, c = t / 16;
        // slot tt of a word holds column 0,2,4,6,1,3,5,7 [tt] of its eight
        float zs[8];
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
            constexpr int col[8] = {0, 2, 4, 6, 1, 3, 5, 7};
            zs[tt] = (float)((st.zb[col[tt] / 4] >> (8 * (col[tt] % 4))) & 0xFFu);
        }
        if constexpr (NARROW) {
#pragma unroll
            for (int ih = 0; ih < 2; ++ih) {
                float v0[8], v1[8];
                nibbles_minus(st.w[2 * ih], zs, v0);  // v0[slot]: k = 4h + 2ih
                nibbles_minus(st.w[2 * ih + 1], zs, v1);
#pragma unroll
                for (int tt = 0; tt < 8; ++tt) {
                    constexpr int col[8] = {0, 2, 4, 6, 1, 3, 5, 7};
                    *reinterpret_cast<uint32_t *>(&sm.b[buf][(8 * c + col[tt]) * LDK + 4 * h + 2 * ih]) =
                        bf16_pair(v0[tt], v1[tt]);
                }
            }
        } else {
            // two rows at a time: pr[ih][tt] = bf16 pair of rows (2 ih, 2 ih + 1)
            // of the slot-tt column
            uint32_t pr[2][8];
#pragma unroll
            for (int ih = 0; ih < 2; ++ih) {
                float v0[8], v1[8];
                nibbles_minus(st.w[2 * ih], zs, v0);  // v0[slot]: k = 4h + 2ih
                nibbles_minus(st.w[2 * ih + 1], zs, v1);
#pragma unroll
                for (int tt = 0; tt < 8; ++tt) pr[ih][tt] = bf16_pair(v0[tt], v1[tt]);
            }
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) {
                constexpr int col[8] = {0, 2, 4, 6, 1, 3, 5, 7};
                *reinterpret_cast<u32x2 *>(&sm.b[buf][(8 * c + col[tt]) * LDK + 4 * h]) = u32x2{pr[0][tt], pr[1][tt]};
            }
        }
        sm.s[buf][t / 128][t % 128] = st.s;
    } else {
        // code dword d holds bytes 4d .. 4d+3: nibble 2j of it is element 4d + j,
        // nibble 2j + 1 element 16 + 4d + j
        const float z8[8] = {8.0f, 8.0f, 8.0f, 8.0f, 8.0f, 8.0f, 8.0f, 8.0f};
        uint16_t *dst = &sm.b[buf][(t / 2) * LDK + 32 * (t % 2)];
#pragma unroll
        for (int half = 0; half < 2; ++half) {  // code dwords 2 half, 2 half + 1: elements 8 half .. +7 and 16 + the same
            uint32_t lo[4], hi[4];
#pragma unroll
            for (int dd = 0; dd < 2; ++dd) {
                float v[8];
                nibbles_minus(st.w[2 * half + dd], z8, v);
                lo[2 * dd] = bf16_pair(v[0], v[2]);
                lo[2 * dd + 1] = bf16_pair(v[4], v[6]);
                hi[2 * dd] = bf16_pair(v[1], v[3]);
                hi[2 * dd + 1] = bf16_pair(v[5], v[7]);
            }
            *reinterpret_cast<u32x4 *>(dst + 8 * half) = u32x4{lo[0], lo[1], lo[2], lo[3]};
            *reinterpret_cast<u32x4 *>(dst + 16 + 8 * half) = u32x4{hi[0], hi[1], hi[2], hi[3]};
        }
        sm.s[buf][t % 2][t / 2] = st.s;
    }
}

// One k-tile's MFMA work on buffer buf: step ks (0..3) covers k = 16 ks ..
// 16 ks + 15 of the tile. FRESH starts the partial sums at zero (the
// matrix core's accumulator input is the constant 0).
template <bool FRESH>
__device__ __forceinline__ void mfma_step(const Smem &sm, int buf, int ks, int arow, int brow, int kofs,
                                          f32x16 (&part)[2][2]) {
    const bf16x8 a0 = lds_frag(&sm.a[buf][(arow)*LDK + 16 * ks + kofs]);
    const bf16x8 a1 = lds_frag(&sm.a[buf][(arow + 32) * LDK + 16 * ks + kofs]);
    const bf16x8 b0 = lds_frag(&sm.b[buf][(brow)*LDK + 16 * ks + kofs]);
    const bf16x8 b1 = lds_frag(&sm.b[buf][(brow + 32) * LDK + 16 * ks + kofs]);
    const f32x16 zero = {};
    part[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, FRESH ? zero : part[0][0], 0, 0, 0);
    part[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, FRESH ? zero : part[0][1], 0, 0, 0);
    part[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, FRESH ? zero : part[1][0], 0, 0, 0);
    part[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, FRESH ? zero : part[1][1], 0, 0, 0);
}

// tot += s (column scale) * part.
__device__ __forceinline__ void rescale(float s0, float s1, const f32x16 (&part)[2][2], f32x16 (&tot)[2][2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            tot[i][0][v] = __builtin_fmaf(s0, part[i][0][v], tot[i][0][v]);
            tot[i][1][v] = __builtin_fmaf(s1, part[i][1][v], tot[i][1][v]);
        }
}

// PER_GROUP (GPTQ4 / AWQ4 with group % 64 == 0): the partial sums run over a
// whole group (group / 64 k-tiles) before one rescale. Otherwise (Q4_0,
// groups of 32 or any odd multiple of 32) every 32-k sub-block is rescaled
// with its own scale; within a group that scale is the same, so both forms
// compute the same sum up to rounding.
// BUF: the buffer path for everything (k % 64 == 0; GPTQ4 / AWQ4 with VEC,
// or Q4_0); XB: X alone through its descriptor (k % 64 == 0), the weights
// through the general loader.
template <int FMT, bool YF32, bool PER_GROUP, bool VEC, bool BUF, bool XB = BUF>
__global__ __launch_bounds__(kThreads, 2) void k_gemm_int4(Args p) {
    __shared__ Smem sm;
    // Tile order: workgroups go to the 8 XCDs in turn (block b to XCD b % 8),
    // so XCD x is given a contiguous run of logical tiles (x q + min(x, r)
    // onwards, q, r = grid / 8, grid % 8); logical tiles walk groups of 8 row
    // tiles column by column. The ~64 workgroups an XCD runs at once then
    // cover about 8 x 8 tiles and share their X rows and weight columns in
    // that XCD's L2.
    const int64_t tiles_n = (p.N + BN - 1) / BN;
    const int64_t tiles_m = (p.M + BM - 1) / BM;
    const int64_t nblk = gridDim.x, q8 = nblk / 8, r8 = nblk % 8, xcd = blockIdx.x % 8;
    const int64_t lt = xcd * q8 + min(xcd, r8) + blockIdx.x / 8;
    constexpr int64_t GM = 8;
    const int64_t per_group = GM * tiles_n;
    const int64_t first_m = (lt / per_group) * GM;
    const int64_t gm = min(tiles_m - first_m, GM);
    const int64_t m0 = (first_m + (lt % per_group) % gm) * BM;
    const int64_t n0 = ((lt % per_group) / gm) * BN;
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int wm = wave / 2, wn = wave % 2;
    const int nk = (int)((p.K + BK - 1) / BK);
    const int tpg = PER_GROUP ? (int)(p.group / BK) : 1;  // k-tiles per group

    f32x16 part[2][2], tot[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            part[i][j] = f32x16{};
            tot[i][j] = f32x16{};
        }

    // group cursor of the next k-tile to load (uniform): its first element is
    // element lrem of group lg
    int64_t lg = 0, lrem = 0;
    Stage<FMT> st;
    BufOffsets bo = buf_offsets<FMT>(p, m0, n0);
    const __amdgpu_buffer_rsrc_t rx = rsrc(p.X, XB ? (uint32_t)(((p.M - 1) * p.ldx + p.K) * 2) : 0u);
    __amdgpu_buffer_rsrc_t rw, rz, rs;
    if constexpr (BUF) {
        if constexpr (FMT == QBN_Q4_0) {
            rw = rsrc(p.data, (uint32_t)(p.N * (p.K / 32) * 18));
            rz = rw;
            rs = rw;
        } else {
            rw = rsrc(p.data, (uint32_t)(p.K * p.N / 2));
            rz = rsrc(p.zeros, (uint32_t)((p.K / p.group) * p.N));
            rs = rsrc(p.scales, (uint32_t)((p.K / p.group) * p.N * 2));
        }
        stage_load_buf<FMT, PER_GROUP>(st, p, bo, rx, rw, rz, rs, 0, 0, 0);
    } else {
        stage_load<FMT, VEC, XB>(st, p, m0, n0, 0, lg, lrem, bo.x, rx);
    }
    stage_store<FMT, !PER_GROUP>(st, sm, 0);
    __syncthreads();

    const int arow = wm * 64 + (lane % 32);
    const int brow = wn * 64 + (lane % 32);
    const int kofs = 8 * (lane / 32);
    const int scol = wn * 64 + (lane % 32);  // lane holds column lane % 32 of each MFMA tile
    int tig = 0;                             // k-tile index inside its group
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) {
            lrem += BK;
            while (lrem >= p.group) {
                lrem -= p.group;
                ++lg;
            }
            if constexpr (BUF)
                stage_load_buf<FMT, PER_GROUP>(st, p, bo, rx, rw, rz, rs, (int64_t)(kt + 1) * BK, lg, lrem);
            else
                stage_load<FMT, VEC, XB>(st, p, m0, n0, (int64_t)(kt + 1) * BK, lg, lrem, bo.x, rx);
        }
        if (PER_GROUP) {
            if (tig == 0) {
                mfma_step<true>(sm, buf, 0, arow, brow, kofs, part);
            } else {
                mfma_step<false>(sm, buf, 0, arow, brow, kofs, part);
            }
            mfma_step<false>(sm, buf, 1, arow, brow, kofs, part);
            mfma_step<false>(sm, buf, 2, arow, brow, kofs, part);
            mfma_step<false>(sm, buf, 3, arow, brow, kofs, part);
            if (++tig == tpg) {
                tig = 0;
                rescale(sm.s[buf][1][scol], sm.s[buf][1][scol + 32], part, tot);
            }
        } else {
            mfma_step<true>(sm, buf, 0, arow, brow, kofs, part);
            mfma_step<false>(sm, buf, 1, arow, brow, kofs, part);
            rescale(sm.s[buf][0][scol], sm.s[buf][0][scol + 32], part, tot);
            // keep the second sub-block's work below the rescale, so that one
            // set of partial sums is live at a time (no spills)
            __builtin_amdgcn_sched_barrier(0);
            mfma_step<true>(sm, buf, 2, arow, brow, kofs, part);
            mfma_step<false>(sm, buf, 3, arow, brow, kofs, part);
            rescale(sm.s[buf][1][scol], sm.s[buf][1][scol + 32], part, tot);
        }
        if (kt + 1 < nk) stage_store<FMT, !PER_GROUP>(st, sm, buf ^ 1);
        __syncthreads();
    }

    // lane holds C[i][j] with j = lane % 32, i = 8(v/4) + 4(lane/32) + v%4
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t n = n0 + wn * 64 + 32 * j + (lane % 32);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t m = m0 + wm * 64 + 32 * i + 8 * (v / 4) + 4 * (lane / 32) + (v % 4);
                if (m < p.M && n < p.N) {
                    if (YF32)
                        ((float *)p.Y)[m * p.ldy + n] = tot[i][j][v];
                    else
                        ((uint16_t *)p.Y)[m * p.ldy + n] = bf16_bits_rne(tot[i][j][v]);
                }
            }
        }
}

template <int FMT, bool PER_GROUP, bool VEC, bool BUF = false, bool XB = BUF>
hipError_t run3(const Args &a, bool yf32, hipStream_t s) {
    const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    if (yf32)
        hipLaunchKernelGGL((k_gemm_int4<FMT, true, PER_GROUP, VEC, BUF, XB>), dim3((unsigned)tiles), dim3(kThreads), 0,
                           s, a);
    else
        hipLaunchKernelGGL((k_gemm_int4<FMT, false, PER_GROUP, VEC, BUF, XB>), dim3((unsigned)tiles), dim3(kThreads),
                           0, s, a);
    return hipGetLastError();
}

// X's byte offsets (rows of the last tile included) fit in 31 bits.
bool x_buf_fits(const Args &a) { return ((a.M + BM) * a.ldx + a.K) * 2 < ((int64_t)1 << 31); }

// Every byte offset of the buffer path fits in 31 bits.
bool buf_fits(const Args &a) {
    constexpr int64_t L = (int64_t)1 << 31;
    const int64_t xb = ((a.M + BM) * a.ldx + a.K) * 2;  // rows of the last tile included
    return xb < L && a.K * a.N / 2 < L && (a.K / a.group) * a.N * 2 + (int64_t)BN * 8 < L &&
           (int64_t)(a.N + BN) * 4 * 8 < L;
}

// ------------------------------------------------------------------ 256 x 128 kernel
// Large-m variant (k % 64 == 0; GPTQ4 / AWQ4 with groups that are a multiple
// of 32, or Q4_0). Workgroup tile 256 x 128 of Y, eight waves in 4 x 2, each
// 64 x 64 (2 x 2 MFMA tiles), one workgroup per compute unit. Each decoded
// weight tile then serves 256 rows of X instead of 128, which halves the
// decode work per MFMA.
//  - X k-tiles are copied from global memory straight into LDS by buffer
//    loads with an LDS destination (no registers, no LDS-write
//    instructions), three k-tiles in a ring. Rows past m lie beyond the
//    descriptor's range and land as zeros.
//  - The codes (and zero points) of k-tile kt + 2 are loaded into registers
//    while tile kt is multiplied; those of kt + 1, loaded a tile earlier,
//    are decoded to bf16 (q - z) and written to the other of two LDS weight
//    buffers. One barrier per k-tile.
//  - Each lane loads the scales of its two output columns itself; at the
//    end of a group (GPTQ4 / AWQ4 with groups that are a multiple of 64) or
//    of each 32-k half of a k-tile (Q4_0, and odd multiples of 32) the
//    partial sums are scaled and added to the totals as above.
// X and the decoded weights share one LDS layout: blocks of 8 rows, chunk c
// (k = 8c .. 8c + 7) of row r at (r / 8) * 1152 + c * 128 + (r % 8) * 16, so
// one 64-lane copy fills 8 rows x 128 bytes with lane i at 16 i, and the
// fragment reads of 32 consecutive rows are conflict-free.
// The range check of a buffer load covers the lane's offset but not the
// uniform one. The weight-side loads therefore carry every offset that
// depends on k or the group in the lane's offset, and lanes whose columns lie
// past n read the last valid column (their outputs are never stored). The X
// copies keep k in the uniform offset: a row past m is out of range by its
// lane offset alone, and valid rows stay inside X for every k-tile.
namespace big {

constexpr int BM = 256, BN = 128, BK = 64;
constexpr int WAVES = 8, THREADS = WAVES * kWave;
constexpr int BLK = 1152;
constexpr int A_STAGE = BM / 8 * BLK;
constexpr int B_STAGE = BN / 8 * BLK;
constexpr int XS = 3;
constexpr int B_OFF = XS * A_STAGE;
constexpr int D_STAGE = 4 * BN * 4;           // Q4_0: the d of the k-tile's two blocks per column, then unused slots
constexpr int B_BUF = B_STAGE + D_STAGE;      // one weight buffer (decoded codes, then Q4_0 d)
constexpr int SMEM = B_OFF + 2 * B_BUF;
constexpr int NX = BM / 8 / WAVES;  // X copies per wave per k-tile

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int frag(int r, int c) { return (r / 8) * BLK + c * 128 + (r % 8) * 16; }

// 16 bytes per lane from buffer offset voff + soff into LDS at base + 16 * lane.
__device__ __forceinline__ void copy16(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff, uint8_t *base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)base, 16, voff, soff, 0, 0);
}

__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ u32x4 bf16x8_of(const float (&v)[8]) {
    return u32x4{bf16_pair(v[0], v[1]), bf16_pair(v[2], v[3]), bf16_pair(v[4], v[5]), bf16_pair(v[6], v[7])};
}

// Decode roles: where a thread's codes come from and where their (q - z)
// values go in the LDS weight buffer.
template <int FMT>
struct Role;

// GPTQ4: column nl = t % 128 of the tile, word rows r0 = t / 128 and r0 + 4
// (k = 8 r .. 8 r + 7 of the k-tile); one 16-byte chunk per word.
template <>
struct Role<QBN_GPTQ4> {
    struct Regs {
        uint32_t w[2];
        uint32_t z[2];  // zero-point bytes of the two words' groups
    };
    int nl, r0;
    uint32_t wo, zo, w4, step, nz;
    __device__ __forceinline__ Role(const Args &p, int64_t n0, int t) {
        nl = t % BN;
        r0 = t / BN;
        const int64_t nw = min(n0 + nl, p.N - 1);
        wo = (uint32_t)((r0 * p.N + nw) * 4);
        w4 = (uint32_t)(16 * p.N);
        step = (uint32_t)(32 * p.N);  // 8 word rows per k-tile
        zo = (uint32_t)nw;
        nz = (uint32_t)p.N;
    }
    // g0, g1: groups of the k-tile's two 32-k halves (equal unless HALF);
    // word row r0 lies in the first half, r0 + 4 in the second
    template <bool HALF>
    __device__ __forceinline__ void load(Regs &R, __amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t rz, int kt,
                                         int g0, int g1) const {
        const uint32_t o = wo + (uint32_t)kt * step;
        R.w[0] = __builtin_amdgcn_raw_buffer_load_b32(rw, o, 0, 0);
        R.w[1] = __builtin_amdgcn_raw_buffer_load_b32(rw, o + w4, 0, 0);
        R.z[0] = __builtin_amdgcn_raw_buffer_load_b8(rz, (uint32_t)g0 * nz + zo, 0, 0);
        R.z[1] = HALF ? __builtin_amdgcn_raw_buffer_load_b8(rz, (uint32_t)g1 * nz + zo, 0, 0) : R.z[0];
    }
    __device__ __forceinline__ void store(const Regs &R, uint8_t *wst) const {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float z = (float)(R.z[h] & 0xFFu);
            const float zz[8] = {z, z, z, z, z, z, z, z};
            float v[8];
            nibbles_minus(R.w[h], zz, v);
            *reinterpret_cast<u32x4 *>(wst + frag(nl, r0 + 4 * h)) = bf16x8_of(v);
        }
    }
};

// AWQ4: word column c = (t / 4) % 16 (columns 8c .. 8c + 7; slot s of a
// word holds column 0,2,4,6,1,3,5,7 [s]), word rows 8r .. 8r + 7 of the
// k-tile with r = t / 64; lane q = t % 4 takes slots q and q + 4, i.e.
// columns 8c + 2q and 8c + 2q + 1, and writes one 16-byte chunk for each.
// (The four lanes of a word column read the same words; the 64 lanes of a
// wave then write 16-byte chunks of eight different rows of each 8-row
// block.)
template <>
struct Role<QBN_AWQ4> {
    struct Regs {
        uint32_t w[8];
        uint32_t z;  // zero points of columns 8c + 2q and 8c + 2q + 1 (low two bytes)
    };
    int c, q, r;
    uint32_t wo, row, step, zo, nz;
    __device__ __forceinline__ Role(const Args &p, int64_t n0, int t) {
        q = t % 4;
        c = (t / 4) % 16;
        r = t / 64;
        const int64_t wc = min(n0 / 8 + c, p.N / 8 - 1);
        row = (uint32_t)((p.N / 8) * 4);
        wo = (uint32_t)((8 * r) * row + wc * 4);
        step = (uint32_t)BK * row;
        zo = (uint32_t)(wc * 8 + 2 * q);
        nz = (uint32_t)p.N;
    }
    // word rows 8r .. 8r + 7 lie in 32-k half r / 4 of the k-tile
    template <bool HALF>
    __device__ __forceinline__ void load(Regs &R, __amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t rz, int kt,
                                         int g0, int g1) const {
        const uint32_t o = wo + (uint32_t)kt * step;
#pragma unroll
        for (int i = 0; i < 8; ++i) R.w[i] = __builtin_amdgcn_raw_buffer_load_b32(rw, o + (uint32_t)i * row, 0, 0);
        const int g = (HALF && r >= 4) ? g1 : g0;
        R.z = __builtin_amdgcn_raw_buffer_load_b16(rz, (uint32_t)g * nz + zo, 0, 0);
    }
    __device__ __forceinline__ void store(const Regs &R, uint8_t *wst) const {
        const float z0 = (float)(R.z & 0xFFu), z1 = (float)((R.z >> 8) & 0xFFu);
        // word i: nibble q (column 2q) and nibble q + 4 (column 2q + 1) read
        // as the two halves of a binary16 pair of subnormals: q * 2^-24
        float v0[8], v1[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const f16x2 h = __builtin_bit_cast(f16x2, (R.w[i] >> (4 * q)) & 0x000F000Fu);
            v0[i] = __builtin_fmaf((float)h.x, 0x1p24f, -z0);
            v1[i] = __builtin_fmaf((float)h.y, 0x1p24f, -z1);
        }
        *reinterpret_cast<u32x4 *>(wst + frag(8 * c + 2 * q, r)) = bf16x8_of(v0);
        *reinterpret_cast<u32x4 *>(wst + frag(8 * c + 2 * q + 1, r)) = bf16x8_of(v1);
    }
};

// Q4_0: column nl = t / 4, quarter q = t % 4 of its two blocks in the k-tile:
// block b = q / 2 (k = 32 b .. 32 b + 31), half hh = q % 2 of its 16 code
// bytes. Byte j holds element j (low nibble) and element 16 + j (high
// nibble), so bytes 8 hh .. 8 hh + 7 give chunks 4 b + hh and 4 b + 2 + hh.
// With k % 64 == 0 a block starts on a dword boundary (b = 0) or 2 bytes
// past one (b = 1), so the eight code bytes start 2 bytes past a dword
// boundary (b = 0) or on one (b = 1); the lane reads the 12 dword-aligned
// bytes that end at most 2 bytes past them (b = 0: into the k-tile's second
// block), so the four lanes of a column cover its 36 bytes. The lanes with
// hh = 0 hold their block's d (its first two bytes) and put it in LDS for
// the scaling.
template <>
struct Role<QBN_Q4_0> {
    struct Regs {
        uint32_t w[3];
    };
    int nl, b, hh;
    uint32_t wo, step;
    __device__ __forceinline__ Role(const Args &p, int64_t n0, int t) {
        nl = t / 4;
        b = (t % 4) / 2;
        hh = t % 2;
        const int64_t n = min(n0 + nl, p.N - 1);
        // codes of block b of k-tile 0 start at (n K/32 + b) 18 + 2 + 8 hh
        wo = (uint32_t)((n * (p.K / 32) + b) * 18 + 2 + 8 * hh - (b ? 4 : 2));
        step = 2 * 18;
    }
    template <bool HALF>
    __device__ __forceinline__ void load(Regs &R, __amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t, int kt, int,
                                         int) const {
        const uint32_t o = wo + (uint32_t)kt * step;
        R.w[0] = __builtin_amdgcn_raw_buffer_load_b32(rw, o, 0, 0);
        R.w[1] = __builtin_amdgcn_raw_buffer_load_b32(rw, o + 4, 0, 0);
        R.w[2] = __builtin_amdgcn_raw_buffer_load_b32(rw, o + 8, 0, 0);
    }
    __device__ __forceinline__ void store(const Regs &R, uint8_t *wst) const {
        const uint32_t c0 = b ? R.w[1] : __builtin_amdgcn_alignbyte(R.w[1], R.w[0], 2);
        const uint32_t c1 = b ? R.w[2] : __builtin_amdgcn_alignbyte(R.w[2], R.w[1], 2);
        const float z8[8] = {8.0f, 8.0f, 8.0f, 8.0f, 8.0f, 8.0f, 8.0f, 8.0f};
        // nibbles_minus of dword d: v[2j] = element 8 hh + 4d + j, v[2j + 1] = 16 + the same
        float v0[8], v1[8];
        nibbles_minus(c0, z8, v0);
        nibbles_minus(c1, z8, v1);
        *reinterpret_cast<u32x4 *>(wst + frag(nl, 4 * b + hh)) =
            u32x4{bf16_pair(v0[0], v0[2]), bf16_pair(v0[4], v0[6]), bf16_pair(v1[0], v1[2]), bf16_pair(v1[4], v1[6])};
        *reinterpret_cast<u32x4 *>(wst + frag(nl, 4 * b + 2 + hh)) =
            u32x4{bf16_pair(v0[1], v0[3]), bf16_pair(v0[5], v0[7]), bf16_pair(v1[1], v1[3]), bf16_pair(v1[5], v1[7])};
        // d: bytes 0-1 of the window when b = 0, bytes 2-3 when b = 1 (for
        // hh = 1 these bytes are codes, stored in a slot nobody reads)
        *reinterpret_cast<uint32_t *>(wst + B_STAGE + 4 * (BN * (2 * hh + b) + nl)) = b ? R.w[0] >> 16 : R.w[0] & 0xFFFFu;
    }
};

struct Frag {
    bf16x8 a[2], b[2];
};

__device__ __forceinline__ void read_frag(Frag &f, const uint8_t *xs, const uint8_t *ws, int ks) {
    f.a[0] = *reinterpret_cast<const bf16x8 *>(xs + 256 * ks);
    f.a[1] = *reinterpret_cast<const bf16x8 *>(xs + 4 * BLK + 256 * ks);
    f.b[0] = *reinterpret_cast<const bf16x8 *>(ws + 256 * ks);
    f.b[1] = *reinterpret_cast<const bf16x8 *>(ws + 4 * BLK + 256 * ks);
}

template <bool FRESH>
__device__ __forceinline__ void mma(const Frag &f, f32x16 (&part)[2][2]) {
    const f32x16 zero = {};
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            part[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], FRESH ? zero : part[i][j], 0, 0, 0);
}

__device__ __forceinline__ void scale_add(uint32_t s16, const f32x16 &part, f32x16 &tot) {
    const float s = f16_to_f32(s16);
#pragma unroll
    for (int v = 0; v < 16; ++v) tot[v] = __builtin_fmaf(s, part[v], tot[v]);
}

// The last MFMA step of a group: each 32 x 32 tile's partial sums are scaled
// into its totals right after the next tile's MFMA is issued, so that the
// scaling overlaps the matrix core's work instead of waiting for all four.
__device__ __forceinline__ void mma_last(const Frag &f, uint32_t s0, uint32_t s1, f32x16 (&part)[2][2],
                                         f32x16 (&tot)[2][2]) {
    part[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[0], f.b[0], part[0][0], 0, 0, 0);
    part[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[0], f.b[1], part[0][1], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    scale_add(s0, part[0][0], tot[0][0]);
    part[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[1], f.b[0], part[1][0], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    scale_add(s1, part[0][1], tot[0][1]);
    part[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[1], f.b[1], part[1][1], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    scale_add(s0, part[1][0], tot[1][0]);
    scale_add(s1, part[1][1], tot[1][1]);
}

// Pipeline of one k-tile kt (every wave issues the same loads in every
// k-tile, tiles past the end clamped to the last one, so that the
// compiler's wait counts for the register loads are static):
//   issue: scales of k-tile kt + 1, codes and zero points of kt + 2 (into the
//          register set kt % 2), then X of kt + 2 (into ring slot
//          (kt + 2) % 3) as the tile's last memory issues;
//   MFMA steps 0..2 of kt, each step's fragments read one step ahead;
//   decode the codes of kt + 1 into LDS buffer (kt + 1) % 2;
//   wait for X of kt + 1, barrier; read step 0 of kt + 1; MFMA step 3 of kt;
//   at the end of a group, scale the partial sums into the totals.
// The buffers written in k-tile kt were last read before the barrier of
// k-tile kt - 1.
// TPG: k-tiles per group when it is 1 or 2 (group 64 or 128; the group
// boundaries then fall on fixed k-tile parities of the two-tile unrolled
// loop), 0 for any other multiple of 64, -1 for odd multiples of 32 (32, 96,
// ...). Q4_0 (32-k blocks) and TPG = -1 rescale after steps 1 and 3 of every
// k-tile, each 32-k half with its own scale.
template <int FMT, bool YF32, int TPG>
__global__ __launch_bounds__(THREADS) void k_gemm_int4_big(Args p, int tiles_m, int tiles_n) {
    constexpr bool Q40 = FMT == QBN_Q4_0;
    constexpr bool HALF = Q40 || TPG < 0;
    __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
    // tile order as in k_gemm_int4, with groups of GM row tiles
    constexpr int GM = 4;
    const int nblk = gridDim.x, q8 = nblk / 8, r8 = nblk % 8, xcd = blockIdx.x % 8;
    const int lt = xcd * q8 + min(xcd, r8) + blockIdx.x / 8;
    const int per_group = GM * tiles_n;
    const int first_m = (lt / per_group) * GM;
    const int gm = min(tiles_m - first_m, GM);
    const int64_t m0 = (int64_t)(first_m + (lt % per_group) % gm) * BM;
    const int64_t n0 = (int64_t)((lt % per_group) / gm) * BN;

    const int t = threadIdx.x;
    const int lane = t % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
    const int wm = wave / 2, wn = wave % 2;
    const int lr = lane % 32, lh = lane / 32;
    const int nk = (int)(p.K / BK);
    const int tpg = HALF ? 1 : TPG ? TPG : (int)(p.group / BK);
    const int group = (int)p.group;
    // (HALF) group of 32-k half h of k-tile kt
    auto grp = [&](int kt, int h) { return (BK * kt + 32 * h) / group; };
    const int64_t N = p.N;

    const __amdgpu_buffer_rsrc_t rx = rsrc(p.X, (uint32_t)(((p.M - 1) * p.ldx + p.K) * 2));
    __amdgpu_buffer_rsrc_t rw, rz, rs;
    if (Q40) {
        rw = rsrc(p.data, (uint32_t)(N * (p.K / 32) * 18));
        rz = rw;
        rs = rw;
    } else {
        rw = rsrc(p.data, (uint32_t)(p.K * N / 2));
        rz = rsrc(p.zeros, (uint32_t)((p.K / p.group) * N));
        rs = rsrc(p.scales, (uint32_t)((p.K / p.group) * N * 2));
    }

    // X copy i of this wave: rows 8 q .. 8 q + 7 of the tile, q = wave + 8 i;
    // lane: row 8 q + lane % 8, chunk lane / 8. The k-tile goes in the
    // uniform offset; a row past m is past the descriptor's range.
    uint32_t xo[NX];
#pragma unroll
    for (int i = 0; i < NX; ++i)
        xo[i] = (uint32_t)(((m0 + 8 * (wave + WAVES * i) + lane % 8) * p.ldx + 8 * (lane / 8)) * 2);
    auto copy_x = [&](int slot, int kt) {
#pragma unroll
        for (int i = 0; i < NX; ++i)
            copy16(rx, xo[i], kt * BK * 2, smem + slot * A_STAGE + (wave + WAVES * i) * BLK);
    };

    const Role<FMT> role(p, n0, t);
    using Regs = typename Role<FMT>::Regs;

    // The scales of this lane's output columns (MFMA column lr of tiles j =
    // 0, 1), s[j]: GPTQ4 / AWQ4 the two fp16 scales of a group, loaded a
    // k-tile ahead. HALF, s[2 h + j] for the k-tile's 32-k half h: Q4_0 the d
    // of its two blocks, read from the LDS weight buffer; GPTQ4 / AWQ4 the
    // scales of the halves' groups, loaded a k-tile ahead.
    const int64_t c0 = min(n0 + wn * 64 + lr, N - 1), c1 = min(n0 + wn * 64 + 32 + lr, N - 1);
    const uint32_t so0 = (uint32_t)(c0 * 2), so1 = (uint32_t)(c1 * 2);
    struct SRegs {
        uint32_t s[HALF ? 4 : 2];
    };
    // u: the group (GPTQ4 / AWQ4) or, with HALF, the k-tile
    auto load_s = [&](SRegs &S, int u) {
        if constexpr (Q40) return;
        if constexpr (HALF) {
            const uint32_t g0 = (uint32_t)(grp(u, 0) * N * 2), g1 = (uint32_t)(grp(u, 1) * N * 2);
            S.s[0] = __builtin_amdgcn_raw_buffer_load_b16(rs, so0 + g0, 0, 0);
            S.s[1] = __builtin_amdgcn_raw_buffer_load_b16(rs, so1 + g0, 0, 0);
            S.s[2] = __builtin_amdgcn_raw_buffer_load_b16(rs, so0 + g1, 0, 0);
            S.s[3] = __builtin_amdgcn_raw_buffer_load_b16(rs, so1 + g1, 0, 0);
        } else {
            const uint32_t go = (uint32_t)(u * N * 2);
            S.s[0] = __builtin_amdgcn_raw_buffer_load_b16(rs, so0 + go, 0, 0);
            S.s[1] = __builtin_amdgcn_raw_buffer_load_b16(rs, so1 + go, 0, 0);
        }
    };
    // codes and zero points of k-tile kt (g: its group, without HALF)
    auto load_w = [&](Regs &R, int kt, int g) {
        if constexpr (HALF)
            role.template load<true>(R, rw, rz, kt, grp(kt, 0), grp(kt, 1));
        else
            role.template load<false>(R, rw, rz, kt, g, g);
    };
    const int d_lane = B_STAGE + 4 * (wn * 64 + lr);
    auto read_d = [&](SRegs &S, const uint8_t *wbuf) {
        if constexpr (Q40) {
            S.s[0] = *reinterpret_cast<const uint32_t *>(wbuf + d_lane);
            S.s[1] = *reinterpret_cast<const uint32_t *>(wbuf + d_lane + 128);
            S.s[2] = *reinterpret_cast<const uint32_t *>(wbuf + d_lane + 4 * BN);
            S.s[3] = *reinterpret_cast<const uint32_t *>(wbuf + d_lane + 4 * BN + 128);
        }
    };

    const int a_lane = frag(wm * 64 + lr, lh);
    const int b_lane = B_OFF + frag(wn * 64 + lr, lh);
    f32x16 part[2][2], tot[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            part[i][j] = f32x16{};
            tot[i][j] = f32x16{};
        }

    Regs R[2];
    SRegs S[2];
    const int last = nk - 1;
    // group cursors (GPTQ4 / AWQ4): k-tile kt + 1 (scales) and kt + 2 (codes),
    // clamped to the last k-tile like the loads themselves
    int gs = 0, ts = 0, gw = 0, tw = 0;
    auto advance = [&](int &g, int &tl, int kt_next) {
        if (kt_next > last) return;
        if (++tl == tpg) {
            tl = 0;
            ++g;
        }
    };
    load_w(R[0], 0, 0);
    copy_x(0, 0);
    load_s(S[0], 0);
    advance(gw, tw, 1);
    load_w(R[1], min(1, last), gw);
    __builtin_amdgcn_sched_barrier(0);
    copy_x(1, min(1, last));
    role.store(R[0], smem + B_OFF);
    // X of k-tile 0 has landed once at most k-tile 1's copies remain. (A
    // count that also allowed the register loads issued after it would
    // break wherever the compiler drops a load whose value is unused.)
    __builtin_amdgcn_s_waitcnt(0xF70 | NX);
    lds_barrier();
    Frag f[2];
    read_frag(f[0], smem + a_lane, smem + b_lane, 0);

    int tig = 0;
    int slot = 0;  // ring slot of k-tile kt
    auto tile = [&](int kt, auto par) {
        constexpr int P = decltype(par)::value;  // kt % 2
        advance(gs, ts, kt + 1);
        advance(gw, tw, kt + 2);
        load_s(S[P ^ 1], HALF ? min(kt + 1, last) : gs);
        load_w(R[P], min(kt + 2, last), gw);
        // the X copies are this tile's last memory issues (see the wait below)
        __builtin_amdgcn_sched_barrier(0);
        copy_x(slot == 0 ? 2 : slot - 1, min(kt + 2, last));
        const uint8_t *xs = smem + slot * A_STAGE + a_lane;
        const uint8_t *ws = smem + P * B_BUF + b_lane;
        read_frag(f[1], xs, ws, 1);
        if constexpr (HALF) {
            if constexpr (Q40) read_d(S[P], smem + B_OFF + P * B_BUF);
            mma<true>(f[0], part);
            read_frag(f[0], xs, ws, 2);
            mma_last(f[1], S[P].s[0], S[P].s[1], part, tot);
            __builtin_amdgcn_sched_barrier(0);
            read_frag(f[1], xs, ws, 3);
            mma<true>(f[0], part);
        } else {
            const bool first = TPG == 1 ? true : TPG == 2 ? P == 0 : tig == 0;
            if (first)
                mma<true>(f[0], part);
            else
                mma<false>(f[0], part);
            read_frag(f[0], xs, ws, 2);
            mma<false>(f[1], part);
            read_frag(f[1], xs, ws, 3);
            mma<false>(f[0], part);
        }
        role.store(R[P ^ 1], smem + B_OFF + (P ^ 1) * B_BUF);
        __builtin_amdgcn_s_waitcnt(0xF70 | NX);  // X of k-tile kt + 1: issued before this tile's copies
        lds_barrier();
        slot = slot == 2 ? 0 : slot + 1;
        read_frag(f[0], smem + slot * A_STAGE + a_lane, smem + (P ^ 1) * B_BUF + b_lane, 0);
        bool end = true;
        if (!HALF && TPG == 0) {
            end = ++tig == tpg;
            if (end) tig = 0;
        } else if (!HALF && TPG == 2) {
            end = P == 1;
        }
        if constexpr (HALF) {
            mma_last(f[1], S[P].s[2], S[P].s[3], part, tot);
        } else if (TPG != 0 && end) {
            mma_last(f[1], S[P].s[0], S[P].s[1], part, tot);
        } else {
            // (other group sizes: the interleaved form costs a spill there)
            mma<false>(f[1], part);
            if (end) {
                scale_add(S[P].s[0], part[0][0], tot[0][0]);
                scale_add(S[P].s[1], part[0][1], tot[0][1]);
                scale_add(S[P].s[0], part[1][0], tot[1][0]);
                scale_add(S[P].s[1], part[1][1], tot[1][1]);
            }
        }
    };
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
        tile(kt, std::integral_constant<int, 0>{});
        tile(kt + 1, std::integral_constant<int, 1>{});
    }
    if (kt < nk) tile(kt, std::integral_constant<int, 0>{});
    // no copy into LDS may still be in flight when the workgroup ends
    __builtin_amdgcn_s_waitcnt(0xF70);

    // lane holds C[i][j] with j = lane % 32, i = 8(v/4) + 4(lane/32) + v%4
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t n = n0 + wn * 64 + 32 * j + lr;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t m = m0 + wm * 64 + 32 * i + 8 * (v / 4) + 4 * lh + (v % 4);
                if (m < p.M && n < N) {
                    if (YF32)
                        ((float *)p.Y)[m * p.ldy + n] = tot[i][j][v];
                    else
                        ((uint16_t *)p.Y)[m * p.ldy + n] = bf16_bits_rne(tot[i][j][v]);
                }
            }
        }
}

// Shapes the 256 x 128 kernel takes: m >= 256, n >= 128, k % 64 == 0, every
// byte offset (X rows of the last tile included) within 31 bits; GPTQ4 /
// AWQ4 with groups that are a multiple of 32 (GPTQ4: n even, 4-byte aligned
// codes; AWQ4: 4-byte aligned codes, 2-byte aligned zero points); Q4_0 with
// dword-aligned blocks.
bool fits(int fmt, const Args &a) {
    constexpr int64_t L = (int64_t)1 << 31;
    if (!(a.M >= BM && a.N >= BN && a.K % BK == 0 && ((a.M + BM) * a.ldx + a.K) * 2 < L)) return false;
    if (fmt == QBN_Q4_0) return (uintptr_t)a.data % 4 == 0 && a.N * (a.K / 32) * 18 < L;
    if (a.group % 32 != 0 || a.K * a.N / 2 >= L || (a.K / a.group) * a.N * 2 >= L) return false;
    if (fmt == QBN_GPTQ4) return a.N % 2 == 0 && (uintptr_t)a.data % 4 == 0;
    return (uintptr_t)a.data % 4 == 0 && (uintptr_t)a.zeros % 2 == 0;
}

template <int FMT, bool YF32>
void launch(const Args &a, int tm, int tn, hipStream_t s) {
    const dim3 grid((unsigned)(tm * tn)), block(THREADS);
    if constexpr (FMT == QBN_Q4_0) {
        hipLaunchKernelGGL((k_gemm_int4_big<FMT, YF32, 1>), grid, block, 0, s, a, tm, tn);
    } else {
        if (a.group == 64)
            hipLaunchKernelGGL((k_gemm_int4_big<FMT, YF32, 1>), grid, block, 0, s, a, tm, tn);
        else if (a.group == 128)
            hipLaunchKernelGGL((k_gemm_int4_big<FMT, YF32, 2>), grid, block, 0, s, a, tm, tn);
        else if (a.group % BK == 0)
            hipLaunchKernelGGL((k_gemm_int4_big<FMT, YF32, 0>), grid, block, 0, s, a, tm, tn);
        else
            hipLaunchKernelGGL((k_gemm_int4_big<FMT, YF32, -1>), grid, block, 0, s, a, tm, tn);
    }
}

template <int FMT>
hipError_t run(const Args &a, bool yf32, hipStream_t s) {
    const int tm = (int)((a.M + BM - 1) / BM), tn = (int)((a.N + BN - 1) / BN);
    if (yf32)
        launch<FMT, true>(a, tm, tn, s);
    else
        launch<FMT, false>(a, tm, tn, s);
    return hipGetLastError();
}

}  // namespace big

template <int FMT>
hipError_t run(const Args &a, bool yf32, hipStream_t s) {
    if (big::fits(FMT, a)) return big::run<FMT>(a, yf32, s);
    // X through its descriptor when k % 64 == 0: measured 4-6% faster for
    // Q4_0 and GPTQ; AWQ's general path spills more with it and is slower.
    const bool xb = FMT != QBN_AWQ4 && a.K % BK == 0 && x_buf_fits(a);
    if constexpr (FMT == QBN_Q4_0) {
        // buffer path: k % 64 == 0, dword-aligned blocks, offsets in 31 bits
        const bool qb = xb && (uintptr_t)a.data % 4 == 0 && (a.N + BN) * (a.K / 32) * 18 + 64 < ((int64_t)1 << 31);
        if (qb) return run3<FMT, false, false, true, true>(a, yf32, s);
        return xb ? run3<FMT, false, false, false, true>(a, yf32, s) : run3<FMT, false, false>(a, yf32, s);
    } else {
        const bool vec = a.N % 8 == 0 && (uintptr_t)a.data % 16 == 0 && (uintptr_t)a.zeros % 8 == 0;
        if (a.group % BK == 0) {
            if (vec && buf_fits(a)) return run3<FMT, true, true, true>(a, yf32, s);
            if (xb) return vec ? run3<FMT, true, true, false, true>(a, yf32, s) : run3<FMT, true, false, false, true>(a, yf32, s);
            return vec ? run3<FMT, true, true>(a, yf32, s) : run3<FMT, true, false>(a, yf32, s);
        }
        // per-32-k path: the buffer loads pay off for GPTQ4 only (AWQ4 measured
        // slower with them than with the general loader)
        if (FMT == QBN_GPTQ4 && vec && a.K % BK == 0 && buf_fits(a)) return run3<FMT, false, true, true>(a, yf32, s);
        if (xb) return vec ? run3<FMT, false, true, false, true>(a, yf32, s) : run3<FMT, false, false, false, true>(a, yf32, s);
        return vec ? run3<FMT, false, true>(a, yf32, s) : run3<FMT, false, false>(a, yf32, s);
    }
}

}  // namespace

bool gemm_int4_grid_fits(int64_t m, int64_t n) {
    const int64_t tiles = ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
    return tiles < ((int64_t)1 << 31);
}

hipError_t launch_gemm_int4(const qbn_tensor &w, int64_t m, const void *x, int64_t ldx, void *y, int y_dtype,
                            int64_t ldy, hipStream_t s) {
    Args a;
    a.X = (const uint16_t *)x;
    a.ldx = ldx;
    a.data = (const uint8_t *)w.data;
    a.scales = (const uint16_t *)w.scales;
    a.zeros = (const uint8_t *)w.zeros;
    a.group = w.format == QBN_Q4_0 ? 32 : w.group;
    a.Y = y;
    a.ldy = ldy;
    a.M = m;
    a.N = w.n;
    a.K = w.k;
    const bool yf32 = y_dtype == QBN_F32;
    switch (w.format) {
    case QBN_GPTQ4: return run<QBN_GPTQ4>(a, yf32, s);
    case QBN_AWQ4: return run<QBN_AWQ4>(a, yf32, s);
    case QBN_Q4_0: return run<QBN_Q4_0>(a, yf32, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qbn
