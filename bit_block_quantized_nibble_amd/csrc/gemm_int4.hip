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
// group (every sub-block for Q4_0) the partial is multiplied by its column's
// scale and added to the running total, so every product is exact and each
// output sees k/16 MFMA steps plus k/group scaled additions in binary32.
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

struct Smem {
    uint16_t a[2][BM * LDK];  // X tile, [m][k]
    uint16_t b[2][BN * LDK];  // decoded codes (q - z) as bf16, [n][k]
    float s[2][2][BN];        // scale of each column for the tile's two 32-k sub-blocks
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
//   GPTQ4: word row r = t/32 (k = 8r .. 8r+7 of the tile), 4 columns 4(t%32) .. +3;
//   AWQ4:  k rows 4(t/16) .. +3, word column t % 16 (columns 8(t%16) .. +7);
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

template <int FMT>
__device__ __forceinline__ void stage_load(Stage<FMT> &st, const Args &p, int64_t m0, int64_t n0, int64_t k0) {
    const int t = threadIdx.x;
    {
        const int c16 = t % 8;
        const int64_t k = k0 + 8 * c16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t m = m0 + t / 8 + 32 * i;
            st.a[i] = (m < p.M && k < p.K) ? ld16(p.X + m * p.ldx + k) : u32x4{0u, 0u, 0u, 0u};
        }
    }
    if (FMT == QBN_GPTQ4) {
        const int r = t / 32;
        const int64_t kk = k0 + 8 * r;
        const int64_t n = n0 + 4 * (t % 32);
        const bool kok = kk < p.K;
        const int64_t g = (kok ? kk : 0) / p.group;
        const uint32_t *src = reinterpret_cast<const uint32_t *>(p.data) + (kk / 8) * p.N + n;
        uint32_t zz = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = kok && (n + i < p.N);
            st.w[i] = ok ? src[i] : 0u;
            zz |= (ok ? (uint32_t)p.zeros[g * p.N + n + i] : 0u) << (8 * i);
        }
        st.zb[0] = zz;
    } else if (FMT == QBN_AWQ4) {
        const int h = t / 16, c = t % 16;
        const int64_t n = n0 + 8 * c;
        const int64_t kk = k0 + 4 * h;
        const bool nok = n < p.N;
        const int64_t g = (kk < p.K ? kk : 0) / p.group;
        const uint32_t *src = reinterpret_cast<const uint32_t *>(p.data) + kk * (p.N / 8) + n / 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) st.w[i] = (nok && kk + i < p.K) ? src[i * (p.N / 8)] : 0u;
        uint32_t z0 = 0, z1 = 0;
        if (nok) {
            const uint8_t *zp = p.zeros + g * p.N + n;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                z0 |= (uint32_t)zp[j] << (8 * j);
                z1 |= (uint32_t)zp[4 + j] << (8 * j);
            }
        }
        st.zb[0] = z0;
        st.zb[1] = z1;
    } else {  // Q4_0
        const int64_t n = n0 + t / 2;
        const int64_t b = k0 / 32 + (t % 2);
        const bool ok = n < p.N && 32 * b < p.K;
        Q40B blk = {0, {0u, 0u, 0u, 0u}};
        if (ok) blk = *reinterpret_cast<const Q40B *>(p.data + (n * (p.K / 32) + b) * 18);
#pragma unroll
        for (int i = 0; i < 4; ++i) st.w[i] = blk.c[i];
        st.s = f16_to_f32(blk.d);
    }
    if (FMT != QBN_Q4_0) {
        const int sb = t / 128;
        const int64_t n = n0 + t % 128;
        const int64_t kk = k0 + 32 * sb;
        st.s = (n < p.N && kk < p.K) ? f16_to_f32(p.scales[(kk / p.group) * p.N + n]) : 0.0f;
    }
}

template <int FMT>
__device__ __forceinline__ void stage_store(const Stage<FMT> &st, Smem &sm, int buf) {
    const int t = threadIdx.x;
    {
        const int c16 = t % 8;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<u32x4 *>(&sm.a[buf][(t / 8 + 32 * i) * LDK + 8 * c16]) = st.a[i];
    }
    if (FMT == QBN_GPTQ4) {
        const int r = t / 32;
        const int c = 4 * (t % 32);
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
        const int h = t / 16, c = t % 16;
        // slot tt of a word holds column 0,2,4,6,1,3,5,7 [tt] of its eight
        float zs[8];
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
            constexpr int col[8] = {0, 2, 4, 6, 1, 3, 5, 7};
            zs[tt] = (float)((st.zb[col[tt] / 4] >> (8 * (col[tt] % 4))) & 0xFFu);
        }
        float v[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i) nibbles_minus(st.w[i], zs, v[i]);  // v[i][slot]: k = 4h + i
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
            constexpr int col[8] = {0, 2, 4, 6, 1, 3, 5, 7};
            *reinterpret_cast<u32x2 *>(&sm.b[buf][(8 * c + col[tt]) * LDK + 4 * h]) =
                u32x2{bf16_pair(v[0][tt], v[1][tt]), bf16_pair(v[2][tt], v[3][tt])};
        }
        sm.s[buf][t / 128][t % 128] = st.s;
    } else {
        // code dword d holds bytes 4d .. 4d+3: nibble 2j of it is element 4d + j,
        // nibble 2j + 1 element 16 + 4d + j
        const float z8[8] = {8.0f, 8.0f, 8.0f, 8.0f, 8.0f, 8.0f, 8.0f, 8.0f};
        uint32_t lo[8], hi[8];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            float v[8];
            nibbles_minus(st.w[d], z8, v);
            lo[2 * d] = bf16_pair(v[0], v[2]);
            lo[2 * d + 1] = bf16_pair(v[4], v[6]);
            hi[2 * d] = bf16_pair(v[1], v[3]);
            hi[2 * d + 1] = bf16_pair(v[5], v[7]);
        }
        uint16_t *dst = &sm.b[buf][(t / 2) * LDK + 32 * (t % 2)];
        *reinterpret_cast<u32x4 *>(dst) = u32x4{lo[0], lo[1], lo[2], lo[3]};
        *reinterpret_cast<u32x4 *>(dst + 8) = u32x4{lo[4], lo[5], lo[6], lo[7]};
        *reinterpret_cast<u32x4 *>(dst + 16) = u32x4{hi[0], hi[1], hi[2], hi[3]};
        *reinterpret_cast<u32x4 *>(dst + 24) = u32x4{hi[4], hi[5], hi[6], hi[7]};
        sm.s[buf][t % 2][t / 2] = st.s;
    }
}

template <int FMT, bool YF32>
__global__ __launch_bounds__(kThreads) void k_gemm_int4(Args p) {
    __shared__ Smem sm;
    const int64_t tiles_n = (p.N + BN - 1) / BN;
    const int64_t m0 = (int64_t)(blockIdx.x / tiles_n) * BM;
    const int64_t n0 = (int64_t)(blockIdx.x % tiles_n) * BN;
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int wm = wave / 2, wn = wave % 2;
    const int nk = (int)((p.K + BK - 1) / BK);
    const int nsub = (int)(p.K / 32);                       // 32-k sub-blocks of k (k % 32 == 0)
    const int spg = FMT == QBN_Q4_0 ? 1 : (int)(p.group / 32);  // sub-blocks per group

    f32x16 part[2][2], tot[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            part[i][j] = f32x16{};
            tot[i][j] = f32x16{};
        }

    Stage<FMT> st;
    stage_load<FMT>(st, p, m0, n0, 0);
    stage_store<FMT>(st, sm, 0);
    __syncthreads();

    const int arow = wm * 64 + (lane % 32);
    const int brow = wn * 64 + (lane % 32);
    const int kofs = 8 * (lane / 32);
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) stage_load<FMT>(st, p, m0, n0, (int64_t)(kt + 1) * BK);
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
            for (int ks = 2 * sb; ks < 2 * sb + 2; ++ks) {
                const bf16x8 a0 = lds_frag(&sm.a[buf][(arow)*LDK + 16 * ks + kofs]);
                const bf16x8 a1 = lds_frag(&sm.a[buf][(arow + 32) * LDK + 16 * ks + kofs]);
                const bf16x8 b0 = lds_frag(&sm.b[buf][(brow)*LDK + 16 * ks + kofs]);
                const bf16x8 b1 = lds_frag(&sm.b[buf][(brow + 32) * LDK + 16 * ks + kofs]);
                part[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, part[0][0], 0, 0, 0);
                part[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, part[0][1], 0, 0, 0);
                part[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, part[1][0], 0, 0, 0);
                part[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, part[1][1], 0, 0, 0);
            }
            const int gsb = 2 * kt + sb;  // global sub-block index (uniform)
            if ((gsb + 1) % spg == 0 || gsb + 1 >= nsub) {
                // lane holds column n = lane % 32 of each MFMA tile
                const float s0 = sm.s[buf][sb][wn * 64 + (lane % 32)];
                const float s1 = sm.s[buf][sb][wn * 64 + 32 + (lane % 32)];
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        tot[i][0][v] = __builtin_fmaf(s0, part[i][0][v], tot[i][0][v]);
                        tot[i][1][v] = __builtin_fmaf(s1, part[i][1][v], tot[i][1][v]);
                    }
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) part[i][j] = f32x16{};
            }
        }
        if (kt + 1 < nk) stage_store<FMT>(st, sm, buf ^ 1);
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

template <int FMT>
hipError_t run(const Args &a, bool yf32, hipStream_t s) {
    const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    if (yf32)
        hipLaunchKernelGGL((k_gemm_int4<FMT, true>), dim3((unsigned)tiles), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((k_gemm_int4<FMT, false>), dim3((unsigned)tiles), dim3(kThreads), 0, s, a);
    return hipGetLastError();
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
