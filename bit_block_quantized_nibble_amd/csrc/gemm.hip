// Prefill GEMM with packed MXFP4 weights: Y[m][n] = sum_k X[m][k] * W_hat[n][k],
// X bf16 [M][ldx], W MXFP4 (n x k codes + E8M0 scale per 32 along k),
// Y bf16 [M][ldy], binary32 accumulation on the bf16 matrix cores.
//
// "Why 4-Bit Quantization Is King", sections 7 and 7d: a weight-only W4
// kernel keeps B packed, loads a tile of A and the packed tile of B with its
// scales, decodes, multiplies and accumulates in a wider type; with a large
// prefill batch every decoded weight is reused across many rows, so the
// contraction, not the weight stream, is the cost.
//
// MXFP4 maps exactly onto bf16: an E2M1 value times 2^e has at most two
// significant bits and bf16 shares binary32's exponent range, so the gfx950
// FP4 -> bf16 conversion with the E8M0 scale folded in as 2^e is exact (every
// code and scale byte is checked against the CPU reference). Each weight
// tile is expanded once per workgroup into LDS, next to the X tile, and both
// feed v_mfma_f32_32x32x16_bf16.
//
// Tiling: workgroup 128 x 128 of Y, four waves in a 2 x 2 grid, each wave
// 64 x 64 (2 x 2 MFMA tiles of 32 x 32); k advances 64 at a time, with the
// next k-tile loaded into registers while the current one is multiplied
// from LDS (two LDS buffers, one barrier per k-tile). Accumulation is
// blocked: each 512-long slice of k is summed in its own accumulator and
// then added to the running total, so no binary32 chain exceeds ~64 terms.
#include "qbn_device.h"
#include "qbn_launch.h"

namespace qbn {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kThreads = 256;
constexpr int LDK = BK + 8;     // LDS row pitch in bf16 (16 bytes of padding against bank conflicts)
constexpr int SLICE = 8;        // k-tiles per accumulation slice (8 * 64 = 512)

struct Smem {
    uint16_t a[2][BM * LDK];  // X tile, [m][k]
    uint16_t b[2][BN * LDK];  // expanded W tile, [n][k]
};

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t *p) { return *reinterpret_cast<const bf16x8 *>(p); }

struct Stage {
    u32x4 a[4];   // 4 x 16 bytes of X
    u32x4 w;      // 16 code bytes = 32 MXFP4 elements (one scale group)
    uint32_t sb;  // its E8M0 byte
};

__device__ __forceinline__ void stage_load(Stage &st, const uint16_t *__restrict__ X, int64_t ldx,
                                           const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
                                           int64_t M, int64_t N, int64_t K, int64_t m0, int64_t n0, int64_t k0) {
    const int t = threadIdx.x;
    const int c16 = t % 8;  // 16-byte chunk within a 64-element row
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + t / 8 + 32 * i;
        const int64_t k = k0 + 8 * c16;
        st.a[i] = (m < M && k < K) ? ld16(X + m * ldx + k) : u32x4{0u, 0u, 0u, 0u};
    }
    const int64_t n = n0 + t / 2;
    const int64_t kk = k0 + 32 * (t % 2);
    const bool ok = (n < N) && (kk < K);
    st.w = ok ? ld16(codes + n * (K / 2) + kk / 2) : u32x4{0u, 0u, 0u, 0u};
    st.sb = ok ? (uint32_t)scales[n * (K / 32) + kk / 32] : 127u;
}

__device__ __forceinline__ void stage_store(const Stage &st, Smem &sm, int buf) {
    const int t = threadIdx.x;
    const int c16 = t % 8;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x4 *>(&sm.a[buf][(t / 8 + 32 * i) * LDK + 8 * c16]) = st.a[i];
    // 32 codes -> 32 bf16 with the E8M0 scale folded in (exact)
    const float scale = __builtin_amdgcn_ldexpf(1.0f, e8m0_exponent(st.sb));
    uint32_t o[16];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t w = st.w[d];
        o[4 * d + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
        o[4 * d + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
        o[4 * d + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
        o[4 * d + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
    }
    uint16_t *dst = &sm.b[buf][(t / 2) * LDK + 32 * (t % 2)];
#pragma unroll
    for (int q = 0; q < 4; ++q)
        *reinterpret_cast<u32x4 *>(dst + 8 * q) = u32x4{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
}

__global__ __launch_bounds__(kThreads) void k_gemm_mxfp4_bf16(const uint16_t *__restrict__ X, int64_t ldx,
                                                               const uint8_t *__restrict__ codes,
                                                               const uint8_t *__restrict__ scales,
                                                               uint16_t *__restrict__ Y, int64_t ldy, int64_t M,
                                                               int64_t N, int64_t K) {
    __shared__ Smem sm;
    const int64_t tiles_n = (N + BN - 1) / BN;
    const int64_t m0 = (int64_t)(blockIdx.x / tiles_n) * BM;
    const int64_t n0 = (int64_t)(blockIdx.x % tiles_n) * BN;
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int wm = wave / 2, wn = wave % 2;
    const int nk = (int)((K + BK - 1) / BK);

    f32x16 acc[2][2], tot[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            acc[i][j] = f32x16{};
            tot[i][j] = f32x16{};
        }

    Stage st;
    stage_load(st, X, ldx, codes, scales, M, N, K, m0, n0, 0);
    stage_store(st, sm, 0);
    __syncthreads();

    const int arow = wm * 64 + (lane % 32);
    const int brow = wn * 64 + (lane % 32);
    const int kofs = 8 * (lane / 32);
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) stage_load(st, X, ldx, codes, scales, M, N, K, m0, n0, (int64_t)(kt + 1) * BK);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const bf16x8 a0 = lds_frag(&sm.a[buf][(arow) * LDK + 16 * ks + kofs]);
            const bf16x8 a1 = lds_frag(&sm.a[buf][(arow + 32) * LDK + 16 * ks + kofs]);
            const bf16x8 b0 = lds_frag(&sm.b[buf][(brow) * LDK + 16 * ks + kofs]);
            const bf16x8 b1 = lds_frag(&sm.b[buf][(brow + 32) * LDK + 16 * ks + kofs]);
            acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc[1][1], 0, 0, 0);
        }
        if ((kt + 1) % SLICE == 0 || kt + 1 == nk) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    tot[i][j] += acc[i][j];
                    acc[i][j] = f32x16{};
                }
        }
        if (kt + 1 < nk) stage_store(st, sm, buf ^ 1);
        __syncthreads();
    }

    // epilogue: lane holds C[i][j] with j = lane % 32, i = 8(v/4) + 4(lane/32) + v%4
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t n = n0 + wn * 64 + 32 * j + (lane % 32);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t m = m0 + wm * 64 + 32 * i + 8 * (v / 4) + 4 * (lane / 32) + (v % 4);
                if (m < M && n < N) Y[m * ldy + n] = bf16_bits_rne(tot[i][j][v]);
            }
        }
}

}  // namespace

hipError_t launch_gemm(const qbn_tensor &w, int64_t m, const void *x, int64_t ldx, void *y, int64_t ldy,
                       hipStream_t s) {
    const int64_t tiles = ((m + BM - 1) / BM) * ((w.n + BN - 1) / BN);
    hipLaunchKernelGGL(k_gemm_mxfp4_bf16, dim3((unsigned)tiles), dim3(kThreads), 0, s, (const uint16_t *)x, ldx,
                       (const uint8_t *)w.data, (const uint8_t *)w.scales, (uint16_t *)y, ldy, m, w.n, w.k);
    return hipGetLastError();
}

}  // namespace qbn
