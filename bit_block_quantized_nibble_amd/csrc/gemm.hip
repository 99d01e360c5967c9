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

// ------------------------------------------------------------------ 256 x 256 kernel
// Large-problem variant: workgroup tile 256 x 256, four waves in 2 x 2, each
// owning a 128 x 128 block of Y (4 x 4 MFMA tiles, 256 accumulator
// registers). X is staged in LDS as bf16 with an XOR swizzle of its
// 16-byte chunks (chunk c of row r at position c ^ (r & 7)), so the 32 rows a
// fragment read touches hit distinct LDS banks. W is staged as packed FP4
// codes plus E8M0 bytes (a quarter of the bf16 bytes) and each wave expands
// its B fragments to bf16 right after reading them, with the scale folded
// into the conversion. The accumulation runs the full k in the MFMA
// accumulators: at most k/16 binary32 roundings per output (512 at
// k = 8192), each at most half an ulp of a partial sum.
namespace big {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int STAGES = 3;

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

// Asynchronous 16-byte global -> LDS copy: lane i of the wave writes its 16
// bytes at lds_base + 16 * i (lds_base must be the same for the whole wave).
// It counts in vmcnt like any vector load.
__device__ __forceinline__ void dma16(const void *g, void *lds_base) {
    __builtin_amdgcn_global_load_lds((glb_void *)g, (lds_void *)lds_base, 16, 0, 0);
}

// The same for 2 bytes (2-byte aligned source): lane i's value lands
// zero-extended in the dword at lds_base + 4 * i.
__device__ __forceinline__ void dma2(const void *g, void *lds_base) {
    __builtin_amdgcn_global_load_lds((glb_void *)g, (lds_void *)lds_base, 2, 0, 0);
}

// Wait until at most n of this wave's vector-memory loads are outstanding
// (n is wave-uniform). Loads complete in issue order.
__device__ __forceinline__ void wait_vm(int n) {
    switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0xF70 | 0); break;
    case 1: __builtin_amdgcn_s_waitcnt(0xF70 | 1); break;
    case 2: __builtin_amdgcn_s_waitcnt(0xF70 | 2); break;
    case 3: __builtin_amdgcn_s_waitcnt(0xF70 | 3); break;
    case 4: __builtin_amdgcn_s_waitcnt(0xF70 | 4); break;
    case 5: __builtin_amdgcn_s_waitcnt(0xF70 | 5); break;
    case 6: __builtin_amdgcn_s_waitcnt(0xF70 | 6); break;
    default: __builtin_amdgcn_s_waitcnt(0xF70 | 7); break;
    }
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS
// operations, not for its outstanding global loads (which __syncthreads'
// fence would also drain). The memory clobber keeps the compiler from moving
// LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// LDS layout of one k-tile (X: 256 rows x 128 bytes; W codes: 256 rows x 32
// bytes; E8M0: one dword per row whose low 16 bits hold the row's two scale
// bytes, first block in the low byte). X and W swizzle 16-byte chunks by row
// so that the 32 rows a fragment read touches spread over the LDS banks:
//   X chunk c of row r  -> row r, slot c ^ (r & 7)
//   W half  h of row n  -> row n, slot h ^ ((n >> 3) & 1)
struct Smem {
    uint8_t a[STAGES][BM * 128];
    uint8_t b[STAGES][BN * 32];
    uint8_t s[STAGES][BN * 4];
};

__device__ __forceinline__ int a_off(int r, int c) { return r * 128 + ((c ^ (r & 7)) * 16); }
__device__ __forceinline__ int b_off(int n, int h) { return n * 32 + ((h ^ ((n >> 3) & 1)) * 16); }

template <int THREADS>
struct Loader {
    static constexpr int WAVES = THREADS / 64;
    static constexpr int NA = BM * 8 / THREADS;  // X chunks per thread (register path)
    static constexpr int NXW = BM / 8 / WAVES;   // X wave-copies per wave (direct path)
    static_assert(BM * 8 % THREADS == 0 && NA >= 1 && (BM / 8) % WAVES == 0, "X tile split");

    // Direct copies this wave issues per k-tile: X, then W codes (copies
    // q < BN/32 go to wave q % WAVES), then scale pairs (copies q < BN/64 go
    // to wave (BN/32 + q) % WAVES).
    __device__ __forceinline__ static int direct_count(int wave) {
        int c = NXW;
        for (int q = 0; q < BN / 32; ++q) c += (q % WAVES == wave);
        for (int q = 0; q < BN / 64; ++q) c += ((BN / 32 + q) % WAVES == wave);
        return c;
    }

    // Interior tiles (every row, column and k of the tile exists, scales
    // 2-byte aligned): X, W codes and scale pairs go straight from global
    // memory into LDS, no registers involved.
    __device__ __forceinline__ static void direct(Smem &sm, int buf, const uint16_t *__restrict__ X, int64_t ldx,
                                                  const uint8_t *__restrict__ codes,
                                                  const uint8_t *__restrict__ scales, int64_t K, int64_t m0,
                                                  int64_t n0, int64_t k0, int lane, int wave) {
        // X: 32 KB = BM/8 wave-copies of 1 KB (8 rows of 128 bytes each)
#pragma unroll
        for (int q = 0; q < NXW; ++q) {
            const int blk = wave * NXW + q;
            const int r = blk * 8 + lane / 8;
            const int c = (lane % 8) ^ (r & 7);
            dma16(X + (m0 + r) * ldx + k0 + 8 * c, &sm.a[buf][blk * 1024]);
        }
        // W codes: 8 KB = BN/32 wave-copies of 1 KB (32 rows of 32 bytes each)
#pragma unroll
        for (int q = 0; q < BN / 32; ++q) {
            if (q % WAVES != wave) continue;
            const int n = q * 32 + lane / 2;
            const int h = (lane % 2) ^ ((n >> 3) & 1);
            dma16(codes + (n0 + n) * (K / 2) + k0 / 2 + 16 * h, &sm.b[buf][q * 1024]);
        }
        // scale pairs: BN/64 wave-copies of 64 rows; lane l's 2 bytes land
        // zero-extended in dword l
#pragma unroll
        for (int q = 0; q < BN / 64; ++q) {
            if ((BN / 32 + q) % WAVES != wave) continue;
            const int n = q * 64 + lane;
            dma2(scales + (n0 + n) * (K / 32) + k0 / 32, &sm.s[buf][q * 256]);
        }
    }

    // Edge tiles: through registers, zero-filling what lies outside.
    __device__ __forceinline__ static void staged(Smem &sm, int buf, const uint16_t *__restrict__ X, int64_t ldx,
                                                  const uint8_t *__restrict__ codes, int64_t M, int64_t N,
                                                  int64_t K, int64_t m0, int64_t n0, int64_t k0) {
        const int t = threadIdx.x;
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int r = t / 8 + (THREADS / 8) * i;
            const int c = t % 8;
            const int64_t m = m0 + r, k = k0 + 8 * c;
            const u32x4 v = (m < M && k < K) ? ld16(X + m * ldx + k) : u32x4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4 *>(&sm.a[buf][a_off(r, c)]) = v;
        }
        for (int i = t; i < BN * 2; i += THREADS) {
            const int n = i / 2, h = i % 2;
            const int64_t nn = n0 + n, k = k0 + 32 * h;
            const u32x4 v = (nn < N && k < K) ? ld16(codes + nn * (K / 2) + k / 2) : u32x4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4 *>(&sm.b[buf][b_off(n, h)]) = v;
        }
    }

    // Edge tiles: the two E8M0 bytes of row t (t < BN) of the k-tile at k0;
    // missing rows or blocks read as 127 (scale 1, multiplying zero codes).
    __device__ __forceinline__ static void scales_edge(Smem &sm, int buf, const uint8_t *__restrict__ scales,
                                                       int64_t N, int64_t K, int64_t n0, int64_t k0) {
        const int t = threadIdx.x;
        if (t >= BN) return;
        uint32_t b0 = 127u, b1 = 127u;
        if (n0 + t < N) {
            const uint8_t *sp = scales + (n0 + t) * (K / 32) + k0 / 32;
            if (k0 < K) b0 = sp[0];
            if (k0 + 32 < K) b1 = sp[1];
        }
        *reinterpret_cast<uint32_t *>(&sm.s[buf][4 * t]) = b0 | (b1 << 8);
    }
};

// One k-tile of MFMA work for a wave owning TM x TN tiles of 32 x 32.
template <int TM, int TN>
__device__ __forceinline__ void mma_ktile(const Smem &sm, int buf, int wm, int wn, int lr, int lh,
                                          f32x16 (&acc)[TM][TN]) {
    // this k-tile's scales of the lane's TN B rows, as 2^e
    float sc[TN][2];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int n = wn * (32 * TN) + 32 * j + lr;
        const uint32_t b2 = *reinterpret_cast<const uint32_t *>(&sm.s[buf][4 * n]);
        sc[j][0] = __builtin_amdgcn_ldexpf(1.0f, e8m0_exponent(b2 & 0xFFu));
        sc[j][1] = __builtin_amdgcn_ldexpf(1.0f, e8m0_exponent((b2 >> 8) & 0xFFu));
    }
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
        bf16x8 af[TM], bfr[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int r = wm * (32 * TM) + 32 * i + lr;
            af[i] = *reinterpret_cast<const bf16x8 *>(&sm.a[buf][a_off(r, 2 * ks + lh)]);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = wn * (32 * TN) + 32 * j + lr;
            // dword (2ks + lh) of row n: half ks / 2, dword (2ks + lh) % 4 within it
            const uint32_t w =
                *reinterpret_cast<const uint32_t *>(&sm.b[buf][b_off(n, ks / 2) + 4 * ((2 * ks + lh) % 4)]);
            const float scale = sc[j][ks / 2];
            const uint32_t p0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
            const uint32_t p1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
            const uint32_t p2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
            const uint32_t p3 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
            bfr[j] = __builtin_bit_cast(bf16x8, u32x4{p0, p1, p2, p3});
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
}

// Workgroup tile 256 x 256 of Y; WGM x WGN waves, each owning a
// (256/WGM) x (256/WGN) block = TM x TN MFMA tiles of 32 x 32. K is walked
// in tiles of 64 through a ring of three LDS buffers: tile kt + 2 is being
// copied in while tile kt is multiplied.
template <int WGM, int WGN>
__global__ __launch_bounds__(WGM * WGN * 64) void k_gemm(const uint16_t *__restrict__ X, int64_t ldx,
                                                          const uint8_t *__restrict__ codes,
                                                          const uint8_t *__restrict__ scales,
                                                          uint16_t *__restrict__ Y, int64_t ldy, int64_t M,
                                                          int64_t N, int64_t K, int tiles_m, int tiles_n) {
    constexpr int THREADS = WGM * WGN * 64;
    constexpr int TM = BM / WGM / 32, TN = BN / WGN / 32;
    using L = Loader<THREADS>;
    __shared__ Smem sm;
    // XCD-aware order: consecutive workgroups go to different XCDs (round
    // robin), so give the workgroups of one XCD the same row panel of X.
    const int nwg = tiles_m * tiles_n;
    const int bid = blockIdx.x;
    int tm, tn;
    {
        const int xcd = bid % 8, local = bid / 8;
        const int per_xcd = (nwg + 7) / 8;
        const int lin = xcd * per_xcd + local;  // position in an m-major order
        if ((nwg % 8) == 0 && lin < nwg) {
            tm = lin / tiles_n;
            tn = lin % tiles_n;
        } else {
            tm = bid / tiles_n;
            tn = bid % tiles_n;
        }
    }
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const bool interior =
        (m0 + BM <= M) && (n0 + BN <= N) && (K % BK == 0) && ((reinterpret_cast<uintptr_t>(scales) & 1) == 0);
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wm = wave / WGN, wn = wave % WGN;
    const int lr = lane % 32, lh = lane / 32;
    const int nk = (int)((K + BK - 1) / BK);

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

    if (interior) {
        // At the top of iteration kt only this wave's newest copies (those
        // of tile kt + 1) may still be in flight.
        const int ndirect = L::direct_count(wave);
        L::direct(sm, 0, X, ldx, codes, scales, K, m0, n0, 0, lane, wave);
        if (nk > 1) L::direct(sm, 1, X, ldx, codes, scales, K, m0, n0, BK, lane, wave);
        for (int kt = 0; kt < nk; ++kt) {
            wait_vm(kt + 1 < nk ? ndirect : 0);
            lds_barrier();
            if (kt + 2 < nk)
                L::direct(sm, (kt + 2) % STAGES, X, ldx, codes, scales, K, m0, n0, (int64_t)(kt + 2) * BK, lane, wave);
            mma_ktile<TM, TN>(sm, kt % STAGES, wm, wn, lr, lh, acc);
        }
    } else {
        L::staged(sm, 0, X, ldx, codes, M, N, K, m0, n0, 0);
        L::scales_edge(sm, 0, scales, N, K, n0, 0);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int buf = kt % STAGES;
            mma_ktile<TM, TN>(sm, buf, wm, wn, lr, lh, acc);
            if (kt + 1 < nk) {
                const int64_t k1 = (int64_t)(kt + 1) * BK;
                L::staged(sm, (kt + 1) % STAGES, X, ldx, codes, M, N, K, m0, n0, k1);
                L::scales_edge(sm, (kt + 1) % STAGES, scales, N, K, n0, k1);
            }
            __syncthreads();
        }
    }

#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t n = n0 + wn * (32 * TN) + 32 * j + lr;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t m = m0 + wm * (32 * TM) + 32 * i + 8 * (v / 4) + 4 * lh + (v % 4);
                if (m < M && n < N) Y[m * ldy + n] = bf16_bits_rne(acc[i][j][v]);
            }
        }
}

template <int WGM, int WGN>
hipError_t run(const qbn_tensor &w, int64_t m, const void *x, int64_t ldx, void *y, int64_t ldy, hipStream_t s) {
    const int64_t tm = (m + BM - 1) / BM, tn = (w.n + BN - 1) / BN;
    hipLaunchKernelGGL((k_gemm<WGM, WGN>), dim3((unsigned)(tm * tn)), dim3(WGM * WGN * 64), 0, s,
                       (const uint16_t *)x, ldx, (const uint8_t *)w.data, (const uint8_t *)w.scales, (uint16_t *)y,
                       ldy, m, w.n, w.k, (int)tm, (int)tn);
    return hipGetLastError();
}

}  // namespace big

}  // namespace

hipError_t launch_gemm(const qbn_tensor &w, int64_t m, const void *x, int64_t ldx, void *y, int64_t ldy,
                       hipStream_t s) {
    if (m >= big::BM && w.n >= big::BN) return big::run<4, 4>(w, m, x, ldx, y, ldy, s);
    const int64_t tiles = ((m + BM - 1) / BM) * ((w.n + BN - 1) / BN);
    hipLaunchKernelGGL(k_gemm_mxfp4_bf16, dim3((unsigned)tiles), dim3(kThreads), 0, s, (const uint16_t *)x, ldx,
                       (const uint8_t *)w.data, (const uint8_t *)w.scales, (uint16_t *)y, ldy, m, w.n, w.k);
    return hipGetLastError();
}

}  // namespace qbn
