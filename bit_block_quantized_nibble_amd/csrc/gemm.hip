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
// Large-problem variant: workgroup tile 256 x 256, eight waves in 4 x 2, each
// owning a 64 x 128 block of Y (2 x 4 MFMA tiles, 128 accumulator
// registers). X is staged in LDS as bf16 in blocks of 8 rows (layout below),
// so the 32 rows a fragment read touches hit distinct LDS banks. W is staged
// as packed FP4 codes plus E8M0 bytes (a quarter of the bf16 bytes) and each
// wave expands its B fragments to bf16 right after reading them, with the
// scale folded into the conversion. The accumulation runs the full k in the
// MFMA accumulators: at most k/16 binary32 roundings per output (512 at
// k = 8192), each at most half an ulp of a partial sum.
namespace big {

constexpr int BM = 256, BN = 256, BK = 64;

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

// Asynchronous 16-byte global -> LDS copy: lane i of the wave writes its 16
// bytes at lds_base + 16 * i (lds_base is the same for the whole wave). It
// counts in vmcnt like any vector load.
__device__ __forceinline__ void dma16(const void *g, void *lds_base) {
    __builtin_amdgcn_global_load_lds((glb_void *)g, (lds_void *)lds_base, 16, 0, 0);
}

// The same for 2 bytes (2-byte aligned source): lane i's value lands
// zero-extended in the dword at lds_base + 4 * i.
__device__ __forceinline__ void dma2(const void *g, void *lds_base) {
    __builtin_amdgcn_global_load_lds((glb_void *)g, (lds_void *)lds_base, 2, 0, 0);
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS
// operations, not for its outstanding global loads (which __syncthreads'
// fence would also drain). The memory clobber keeps the compiler from moving
// LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---------------------------------------------------------------------------
// LDS layouts.
//
// X stage (256 rows x 64 bf16 of one k-tile): blocks of 8 rows; inside a
// block the 16-byte chunk c (k = 8c .. 8c + 7) of row r sits at c * 128 +
// (r % 8) * 16, and blocks are 1152 bytes apart (128 bytes of padding). A
// fragment read (32 consecutive rows, one chunk) is contiguous within each
// group of 8 lanes, and consecutive groups land 128 bytes apart modulo 256:
// no bank conflicts for 8- or 16-lane groups.
//
// Per-tile W / scale stages (the general interior path and edge tiles):
//   W codes, 256 rows x 32 bytes: half h of row n at
//     (n / 32) * 1024 + h * 512 + (n % 32) * 16;
//   scales: one dword per row, low 16 bits = the row's two bytes.
// Chunked W / scale stages (interior tiles when k is a multiple of 512):
//   W codes of 4 k-tiles, 256 rows x 128 bytes: the 16-byte piece p of row n
//     (tile p / 2, half p % 2) at n * 128 + (p ^ g(n)) * 16, with
//     g(n) = (n % 8) ^ ((n / 8) & 1) so that any 8 or 16 consecutive rows
//     read at one p hit distinct banks;
//   scales of 8 k-tiles: the 16 bytes of row n at n * 16.
// Every X fragment address is affine in the MFMA indices, so the X reads use
// one base register and immediate offsets.
constexpr int A_BLK = 1152;
constexpr int A_STAGE = BM / 8 * A_BLK;

struct LayoutTile {  // 3-stage ring of whole k-tiles
    static constexpr int XS = 3;
    static constexpr int W_OFF = XS * A_STAGE, W_STAGE = BN * 32;
    static constexpr int S_OFF = W_OFF + XS * W_STAGE, S_STAGE = BN * 4;
    static constexpr int BYTES = S_OFF + XS * S_STAGE;
};
struct LayoutChunk {  // 2-stage X ring, 2-chunk W and scale rings
    static constexpr int XS = 2;
    static constexpr int WT = 4, ST = 8;  // k-tiles per W / scale chunk
    static constexpr int W_OFF = XS * A_STAGE, W_STAGE = BN * 32 * WT;
    static constexpr int S_OFF = W_OFF + 2 * W_STAGE, S_STAGE = BN * 2 * ST;
    static constexpr int BYTES = S_OFF + 2 * S_STAGE;
};

__device__ __forceinline__ int a_off(int r, int c) { return (r / 8) * A_BLK + c * 128 + (r % 8) * 16; }
__device__ __forceinline__ int b_off(int n, int h) { return (n / 32) * 1024 + h * 512 + (n % 32) * 16; }
__device__ __forceinline__ int w_slot(int n) { return (n % 8) ^ ((n / 8) & 1); }

// ---------------------------------------------------------------------------
// Direct copies of interior tiles. Copy q of a kind goes to wave q % WAVES,
// so each wave's copies differ by uniform offsets from one per-lane pointer.
//   X: 32 copies of 8 rows x 128 bytes (one k-tile);
//   per-tile W: 8 copies of 32 rows x 32 bytes; per-tile scales: 8 half-wave
//     copies of 32 rows x 2 bytes (with 16 waves: waves 0-7 W, 8-15 scales);
//   W chunk: 32 copies of 8 rows x 128 bytes (4 k-tiles);
//   scale chunk: 4 copies of 64 rows x 16 bytes (8 k-tiles), waves 0-3.
template <int WAVES>
struct Copier {
    static_assert(WAVES == 8 || WAVES == 16, "8 or 16 waves");
    static constexpr int NX = (BM / 8) / WAVES;          // X copies per wave
    static constexpr int NWC = (BN / 8) / WAVES;         // W-chunk copies per wave
    static constexpr int TILE_COPIES = NX + (WAVES == 16 ? 1 : 2);

    const uint16_t *xg;  // X element of this lane's first copy at k = 0
    int64_t xstep;       // elements between this wave's X copies
    int xo;              // LDS offset of this wave's first X copy
    const uint8_t *wg;   // per-tile W: code byte at k = 0; chunked: piece of the first copy at k = 0
    const uint8_t *sg;   // scale byte of this lane's row at k = 0
    int64_t wstep;       // chunked: bytes between this wave's W copies
    bool has_w, has_s;   // per-tile mode: this wave copies W / scales
    int wo, so;          // per-tile mode LDS offsets
    int lane;

    __device__ __forceinline__ Copier(const uint16_t *X, int64_t ldx, const uint8_t *codes, const uint8_t *scales,
                                      int64_t K, int64_t m0, int64_t n0, int lane_, int wave, bool chunked)
        : lane(lane_) {
        {
            const int r = wave * 8 + lane % 8, c = lane / 8;
            xg = X + (m0 + r) * ldx + 8 * c;
            xstep = (int64_t)WAVES * 8 * ldx;
            xo = wave * A_BLK;
        }
        if (chunked) {
            const int row = wave * 8 + lane / 8;
            wg = codes + (n0 + row) * (K / 2) + ((lane % 8) ^ w_slot(row)) * 16;
            wstep = (int64_t)WAVES * 8 * (K / 2);
            sg = scales + (n0 + 64 * wave + lane) * (K / 32);
            has_w = false;
            has_s = wave < BN / 64;
            wo = so = 0;
        } else {
            const int qw = wave, qs = (WAVES == 16) ? wave - 8 : wave;
            has_w = (WAVES == 16) ? (wave < 8) : true;
            has_s = (WAVES == 16) ? (wave >= 8) : true;
            const int nw = 32 * (has_w ? qw : 0) + lane % 32, hw = lane / 32;
            wg = codes + (n0 + nw) * (K / 2) + 16 * hw;
            wo = (has_w ? qw : 0) * 1024;
            const int ns = 32 * (has_s ? qs : 0) + lane % 32;
            sg = scales + (n0 + ns) * (K / 32);
            so = (has_s ? qs : 0) * 128;
            wstep = 0;
        }
    }

    __device__ __forceinline__ void x_tile(uint8_t *xstage, int64_t k0) const {
#pragma unroll
        for (int q = 0; q < NX; ++q) dma16(xg + q * xstep + k0, xstage + xo + q * WAVES * A_BLK);
    }
    // per-tile mode: W codes and scale pairs of the k-tile at k0
    __device__ __forceinline__ void ws_tile(uint8_t *wstage, uint8_t *sstage, int64_t k0) const {
        if (has_w) dma16(wg + k0 / 2, wstage + wo);
        if (has_s && lane < 32) dma2(sg + k0 / 32, sstage + so);
    }
    // chunked mode: W codes of k-tiles 4c .. 4c + 3
    __device__ __forceinline__ void w_chunk(uint8_t *wstage, int64_t c, int wave) const {
#pragma unroll
        for (int q = 0; q < NWC; ++q) dma16(wg + q * wstep + c * 128, wstage + (wave + q * WAVES) * 1024);
    }
    // chunked mode: scale bytes of k-tiles 8c .. 8c + 7
    __device__ __forceinline__ void s_chunk(uint8_t *sstage, int64_t c, int wave) const {
        if (has_s) dma16(sg + c * 16, sstage + wave * 1024);
    }
};

// Edge tiles: through registers into the per-tile layout, zero-filling what
// lies outside; scale bytes of missing rows or blocks read as 127 (scale 1,
// zero codes).
template <int THREADS>
__device__ __forceinline__ void stage_edge(uint8_t *xs, uint8_t *ws, uint8_t *ss, const uint16_t *__restrict__ X,
                                           int64_t ldx, const uint8_t *__restrict__ codes,
                                           const uint8_t *__restrict__ scales, int64_t M, int64_t N, int64_t K,
                                           int64_t m0, int64_t n0, int64_t k0) {
    const int t = threadIdx.x;
    for (int i = t; i < BM * 8; i += THREADS) {
        const int r = i / 8, c = i % 8;
        const int64_t m = m0 + r, k = k0 + 8 * c;
        const u32x4 v = (m < M && k < K) ? ld16(X + m * ldx + k) : u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4 *>(xs + a_off(r, c)) = v;
    }
    for (int i = t; i < BN * 2; i += THREADS) {
        const int n = i / 2, h = i % 2;
        const int64_t nn = n0 + n, k = k0 + 32 * h;
        const u32x4 v = (nn < N && k < K) ? ld16(codes + nn * (K / 2) + k / 2) : u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4 *>(ws + b_off(n, h)) = v;
    }
    for (int n = t; n < BN; n += THREADS) {
        uint32_t b0 = 127u, b1 = 127u;
        if (n0 + n < N) {
            const uint8_t *sp = scales + (n0 + n) * (K / 32) + k0 / 32;
            if (k0 < K) b0 = sp[0];
            if (k0 + 32 < K) b1 = sp[1];
        }
        *reinterpret_cast<uint32_t *>(ss + 4 * n) = b0 | (b1 << 8);
    }
}

// ---------------------------------------------------------------------------
// MFMA work of one wave owning TM x TN tiles of 32 x 32.
// The 64 k of a tile are dealt to the MFMA steps in a permuted order that
// both operands share (the sum over k does not depend on it): at step ks the
// lanes of half lh (k slots 8 lh .. 8 lh + 7 of the instruction) take k
// = 8 (4 lh + ks) .. + 7. A lane's codes for the whole tile are then one
// 16-byte piece (half lh of its W row) under one scale (block lh).
template <int TM, int TN>
struct Frags {
    bf16x8 a[TM];     // X fragments of the next step
    u32x4 bw[TN];     // the tile's codes
    uint32_t sb[TN];  // the dword holding the tile's scale byte (converted at first use)
};

template <int TM>
__device__ __forceinline__ void read_a(const uint8_t *a_lane, int ks, bf16x8 (&a)[TM]) {
#pragma unroll
    for (int i = 0; i < TM; ++i) a[i] = *reinterpret_cast<const bf16x8 *>(a_lane + 4 * A_BLK * i + 128 * ks);
}

// Codes, scales and step-0 X fragments of a tile; W and scale addresses of
// MFMA column tile j are BJ and SJ bytes apart.
template <int TM, int TN, int BJ, int SJ>
__device__ __forceinline__ void read_head(const uint8_t *a_lane, const uint8_t *b_lane, const uint8_t *s_lane,
                                          Frags<TM, TN> &f) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        f.sb[j] = *reinterpret_cast<const uint32_t *>(s_lane + SJ * j);
        f.bw[j] = *reinterpret_cast<const u32x4 *>(b_lane + BJ * j);
    }
    read_a<TM>(a_lane, 0, f.a);
}

template <int TN>
__device__ __forceinline__ void scales_of(const uint32_t (&sb)[TN], int shift, float (&sc)[TN]) {
#pragma unroll
    for (int j = 0; j < TN; ++j) sc[j] = __builtin_amdgcn_ldexpf(1.0f, e8m0_exponent((sb[j] >> shift) & 0xFFu));
}

template <int TM, int TN>
__device__ __forceinline__ void mma_step(const bf16x8 (&a)[TM], const u32x4 (&bw)[TN], const float (&sc)[TN], int ks,
                                         f32x16 (&acc)[TM][TN]) {
    bf16x8 bfr[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const uint32_t w = bw[j][ks];
        const float scale = sc[j];
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
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bfr[j], acc[i][j], 0, 0, 0);
}

// Steps 0 .. 2 of a tile whose head is in f; leaves step 3's X fragments in f.a.
template <int TM, int TN>
__device__ __forceinline__ void mma_first_steps(const uint8_t *a_lane, Frags<TM, TN> &f, const float (&sc)[TN],
                                                f32x16 (&acc)[TM][TN]) {
#pragma unroll
    for (int ks = 0; ks < BK / 16 - 1; ++ks) {
        bf16x8 a[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) a[i] = f.a[i];
        read_a<TM>(a_lane, ks + 1, f.a);
        __builtin_amdgcn_sched_barrier(0);
        mma_step<TM, TN>(a, f.bw, sc, ks, acc);
    }
}

// ---------------------------------------------------------------------------
// Workgroup tile 256 x 256 of Y; WGM x WGN waves, each owning a
// (256/WGM) x (256/WGN) block = TM x TN MFMA tiles of 32 x 32.
//
// Interior tiles: the barrier of tile kt sits before its last MFMA step. By
// then every wave has read all of tile kt, so its buffers can be refilled,
// and the head of tile kt + 1 is read while the last step's MFMAs run.
//  - CHUNKED (k % 512 == 0, scales 16-byte aligned): X in a 2-stage ring
//    (tile kt + 2 is copied during tile kt + 1's wait window), W codes in
//    chunks of 4 k-tiles and scales in chunks of 8, each in a ring of two,
//    so every global row segment fetched is a whole 128-byte line (W) or
//    16 bytes (scales) instead of 32 and 2 bytes per k-tile.
//  - otherwise: X, W codes and scale pairs per k-tile in a 3-stage ring.
// Edge tiles go through registers one k-tile at a time.
template <int WGM, int WGN, bool CHUNKED>
__global__ __launch_bounds__(WGM * WGN * 64) void k_gemm(const uint16_t *__restrict__ X, int64_t ldx,
                                                          const uint8_t *__restrict__ codes,
                                                          const uint8_t *__restrict__ scales,
                                                          uint16_t *__restrict__ Y, int64_t ldy, int64_t M,
                                                          int64_t N, int64_t K, int tiles_m, int tiles_n) {
    constexpr int THREADS = WGM * WGN * 64;
    constexpr int WAVES = WGM * WGN;
    constexpr int TM = BM / WGM / 32, TN = BN / WGN / 32;
    constexpr int SMEM = CHUNKED ? LayoutChunk::BYTES : LayoutTile::BYTES;
    static_assert(LayoutTile::BYTES <= SMEM, "edge tiles use the per-tile layout");
    __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
    using LT = LayoutTile;
    using LC = LayoutChunk;
    // XCD-aware order: consecutive workgroups go to different XCDs (round
    // robin), so workgroup bid is given position lin = xcd * per_xcd + local
    // of a banded order: bands of GM tile rows, column-major inside a band.
    // The workgroups of one XCD then cover a GM x (per_xcd / GM) block of
    // tiles (4 x 8 for 2048 x 8192), sharing GM row panels of X and
    // per_xcd / GM column panels of W in that XCD's L2.
    const int nwg = tiles_m * tiles_n;
    const int bid = blockIdx.x;
    int lin = bid;
    if ((nwg % 8) == 0) lin = (bid % 8) * (nwg / 8) + bid / 8;
    constexpr int GM = 4;
    const int band = lin / (GM * tiles_n);
    const int rows = (tiles_m - band * GM) < GM ? (tiles_m - band * GM) : GM;
    const int rb = lin - band * (GM * tiles_n);
    const int tm = band * GM + rb % rows, tn = rb / rows;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const bool inside = (m0 + BM <= M) && (n0 + BN <= N);
    const bool interior =
        inside && (CHUNKED || ((K % BK == 0) && ((reinterpret_cast<uintptr_t>(scales) & 1) == 0)));
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wm = wave / WGN, wn = wave % WGN;
    const int lr = lane % 32, lh = lane / 32;
    const int nk = (int)((K + BK - 1) / BK);

    // per-lane fragment bases
    const int r0 = wm * (32 * TM) + lr;
    const int a_lane = a_off(r0, 4 * lh);
    const int n0w = wn * (32 * TN) + lr;

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

    using C = Copier<WAVES>;
    Frags<TM, TN> f;
    if (CHUNKED && interior) {
        const C cp(X, ldx, codes, scales, K, m0, n0, lane, wave, true);
        uint8_t *const xs = smem, *const wsb = smem + LC::W_OFF, *const ssb = smem + LC::S_OFF;
        const int w_row = n0w * 128, w_sl = w_slot(n0w), s_row = n0w * 16;
        // Prologue: scale chunks 0 and 1, W chunks 0 and 1, X tiles 0 and 1.
        cp.s_chunk(ssb, 0, wave);
        if (nk > LC::ST) cp.s_chunk(ssb + LC::S_STAGE, 1, wave);
        cp.w_chunk(wsb, 0, wave);
        if (nk > LC::WT) cp.w_chunk(wsb + LC::W_STAGE, 1, wave);
        cp.x_tile(xs, 0);
        if (nk > 1) {
            cp.x_tile(xs + A_STAGE, BK);
            __builtin_amdgcn_s_waitcnt(0xF70 | C::NX);
        } else {
            __builtin_amdgcn_s_waitcnt(0xF70);
        }
        lds_barrier();
        read_head<TM, TN, 32 * 128, 32 * 16>(xs + a_lane, wsb + w_row + ((lh ^ w_sl) * 16), ssb + s_row, f);
        for (int kt = 0; kt < nk; ++kt) {
            const int xb = kt & 1;
            float sc[TN];
            scales_of<TN>(f.sb, 8 * (((kt & 7) & 1) * 2 + lh), sc);
            mma_first_steps<TM, TN>(xs + xb * A_STAGE + a_lane, f, sc, acc);
            bf16x8 a[TM];
            u32x4 bw[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) a[i] = f.a[i];
#pragma unroll
            for (int j = 0; j < TN; ++j) bw[j] = f.bw[j];
            if (kt + 1 < nk) {
                // everything issued before this point has landed, in
                // particular tile kt + 1 (issued one tile ago)
                __builtin_amdgcn_s_waitcnt(0xF70);
                lds_barrier();
                if (kt + 2 < nk) cp.x_tile(xs + xb * A_STAGE, (int64_t)(kt + 2) * BK);
                if ((kt & 3) == 3 && (kt + 5) < nk)
                    cp.w_chunk(wsb + (((kt + 5) / 4) & 1) * LC::W_STAGE, (kt + 5) / 4, wave);
                if ((kt & 7) == 7 && (kt + 9) < nk)
                    cp.s_chunk(ssb + (((kt + 9) / 8) & 1) * LC::S_STAGE, (kt + 9) / 8, wave);
                const int t1 = kt + 1;
                const int piece = 2 * (t1 & 3) + lh;
                read_head<TM, TN, 32 * 128, 32 * 16>(
                    xs + (xb ^ 1) * A_STAGE + a_lane,
                    wsb + ((t1 / 4) & 1) * LC::W_STAGE + w_row + ((piece ^ w_sl) * 16),
                    ssb + ((t1 / 8) & 1) * LC::S_STAGE + s_row + 4 * ((t1 & 7) / 2), f);
                __builtin_amdgcn_sched_barrier(0);
            }
            mma_step<TM, TN>(a, bw, sc, BK / 16 - 1, acc);
        }
    } else if (!CHUNKED && interior) {
        // Ring of three buffers; tile t lives in buffer t % 3.
        const C cp(X, ldx, codes, scales, K, m0, n0, lane, wave, false);
        const int b_lane = b_off(n0w, lh), s_lane = 4 * n0w;
        auto xst = [&](int buf) { return smem + buf * A_STAGE; };
        auto wst = [&](int buf) { return smem + LT::W_OFF + buf * LT::W_STAGE; };
        auto sst = [&](int buf) { return smem + LT::S_OFF + buf * LT::S_STAGE; };
        for (int t = 0; t < 3 && t < nk; ++t) {
            cp.x_tile(xst(t), (int64_t)t * BK);
            cp.ws_tile(wst(t), sst(t), (int64_t)t * BK);
        }
        if (nk > 2) __builtin_amdgcn_s_waitcnt(0xF70 | (2 * C::TILE_COPIES));
        else if (nk > 1) __builtin_amdgcn_s_waitcnt(0xF70 | C::TILE_COPIES);
        else __builtin_amdgcn_s_waitcnt(0xF70);
        lds_barrier();
        read_head<TM, TN, 1024, 128>(xst(0) + a_lane, wst(0) + b_lane, sst(0) + s_lane, f);
        int rd = 0;
        for (int kt = 0; kt < nk; ++kt) {
            const int nx = (rd == 2) ? 0 : rd + 1;
            float sc[TN];
            scales_of<TN>(f.sb, 8 * lh, sc);
            mma_first_steps<TM, TN>(xst(rd) + a_lane, f, sc, acc);
            bf16x8 a[TM];
            u32x4 bw[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) a[i] = f.a[i];
#pragma unroll
            for (int j = 0; j < TN; ++j) bw[j] = f.bw[j];
            if (kt + 1 < nk) {
                // tile kt + 1 has landed once only tile kt + 2's copies remain
                if (kt + 2 < nk) __builtin_amdgcn_s_waitcnt(0xF70 | C::TILE_COPIES);
                else __builtin_amdgcn_s_waitcnt(0xF70);
                lds_barrier();
                if (kt + 3 < nk) {
                    cp.x_tile(xst(rd), (int64_t)(kt + 3) * BK);
                    cp.ws_tile(wst(rd), sst(rd), (int64_t)(kt + 3) * BK);
                }
                read_head<TM, TN, 1024, 128>(xst(nx) + a_lane, wst(nx) + b_lane, sst(nx) + s_lane, f);
                __builtin_amdgcn_sched_barrier(0);
            }
            mma_step<TM, TN>(a, bw, sc, BK / 16 - 1, acc);
            rd = nx;
        }
    } else {
        const int b_lane = b_off(n0w, lh), s_lane = 4 * n0w;
        stage_edge<THREADS>(smem, smem + LT::W_OFF, smem + LT::S_OFF, X, ldx, codes, scales, M, N, K, m0, n0, 0);
        __syncthreads();
        int buf = 0;
        for (int kt = 0; kt < nk; ++kt) {
            uint8_t *xs = smem + buf * A_STAGE, *ws = smem + LT::W_OFF + buf * LT::W_STAGE,
                    *ss = smem + LT::S_OFF + buf * LT::S_STAGE;
            read_head<TM, TN, 1024, 128>(xs + a_lane, ws + b_lane, ss + s_lane, f);
            float sc[TN];
            scales_of<TN>(f.sb, 8 * lh, sc);
            mma_first_steps<TM, TN>(xs + a_lane, f, sc, acc);
            mma_step<TM, TN>(f.a, f.bw, sc, BK / 16 - 1, acc);
            const int nxt = buf ^ 1;
            if (kt + 1 < nk)
                stage_edge<THREADS>(smem + nxt * A_STAGE, smem + LT::W_OFF + nxt * LT::W_STAGE,
                                    smem + LT::S_OFF + nxt * LT::S_STAGE, X, ldx, codes, scales, M, N, K, m0, n0,
                                    (int64_t)(kt + 1) * BK);
            __syncthreads();
            buf = nxt;
        }
    }

    // Y is written once and read by no later step of this kernel: non-temporal
    // stores (all 256 workgroups write their tiles at about the same time)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t n = n0 + wn * (32 * TN) + 32 * j + lr;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t m = m0 + wm * (32 * TM) + 32 * i + 8 * (v / 4) + 4 * lh + (v % 4);
                if (m < M && n < N) __builtin_nontemporal_store(bf16_bits_rne(acc[i][j][v]), Y + m * ldy + n);
            }
        }
}

// The chunked interior path needs whole 8-tile scale chunks (k % 512 == 0)
// and 16-byte aligned scale rows.
inline bool chunkable(const qbn_tensor &w) {
    return (w.k % 512) == 0 && (reinterpret_cast<uintptr_t>(w.scales) % 16) == 0;
}

template <int WGM, int WGN>
hipError_t run(const qbn_tensor &w, int64_t m, const void *x, int64_t ldx, void *y, int64_t ldy, hipStream_t s) {
    const int64_t tm = (m + BM - 1) / BM, tn = (w.n + BN - 1) / BN;
    if (chunkable(w))
        hipLaunchKernelGGL((k_gemm<WGM, WGN, true>), dim3((unsigned)(tm * tn)), dim3(WGM * WGN * 64), 0, s,
                           (const uint16_t *)x, ldx, (const uint8_t *)w.data, (const uint8_t *)w.scales,
                           (uint16_t *)y, ldy, m, w.n, w.k, (int)tm, (int)tn);
    else
        hipLaunchKernelGGL((k_gemm<WGM, WGN, false>), dim3((unsigned)(tm * tn)), dim3(WGM * WGN * 64), 0, s,
                           (const uint16_t *)x, ldx, (const uint8_t *)w.data, (const uint8_t *)w.scales,
                           (uint16_t *)y, ldy, m, w.n, w.k, (int)tm, (int)tn);
    return hipGetLastError();
}

}  // namespace big

}  // namespace

hipError_t launch_gemm(const qbn_tensor &w, int64_t m, const void *x, int64_t ldx, void *y, int64_t ldy,
                       hipStream_t s) {
    if (m >= big::BM && w.n >= big::BN) return big::run<4, 2>(w, m, x, ldx, y, ldy, s);
    const int64_t tiles = ((m + BM - 1) / BM) * ((w.n + BN - 1) / BN);
    hipLaunchKernelGGL(k_gemm_mxfp4_bf16, dim3((unsigned)tiles), dim3(kThreads), 0, s, (const uint16_t *)x, ldx,
                       (const uint8_t *)w.data, (const uint8_t *)w.scales, (uint16_t *)y, ldy, m, w.n, w.k);
    return hipGetLastError();
}

}  // namespace qbn
