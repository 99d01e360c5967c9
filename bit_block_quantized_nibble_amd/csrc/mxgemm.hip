// MX activations and the MX-native block-scaled GEMM on gfx950 ("Why 4-Bit
// Quantization Is King", sections 5 and 7 (the FP4 matrix-instruction
// path; the OCP MX contract), "Four Bits, Three Contracts", section 3 (MXFP4:
// E2M1 codes, one E8M0 scale per 32)).
//
// Activation quantization follows the OCP MX rule: per 32 consecutive
// elements of a row, shared exponent e = floor(log2 max|x|) - emax (emax 2
// for E2M1, 8 for E4M3), clamped to [-127, 127]; each element is x * 2^-e
// (exact) rounded to the element grid with ties to even and saturated. The
// hardware FP4 conversion saturates by itself; the FP8 conversion does not
// (it overflows to NaN), so values are clamped to +-448 first.
//
// The GEMM multiplies MXFP4 (or MXFP8) activations by MXFP4 weights with
// v_mfma_scale_f32_32x32x64_f8f6f4: both E8M0 scales are applied by the
// matrix core, so no element is ever converted; products are exact and the
// accumulation is binary32.
#include "qbn_device.h"
#include "qbn_launch.h"

namespace qbn {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------------ activation quantization

template <typename XT>
struct XLoad4;
template <>
struct XLoad4<float> {
    __device__ __forceinline__ static f32x4 at(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
};
template <>
struct XLoad4<__bf16> {
    __device__ __forceinline__ static f32x4 at(const __bf16 *p) {
        const u32x2 w = ld8(p);
        return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u), __uint_as_float(w.y << 16),
                     __uint_as_float(w.y & 0xFFFF0000u)};
    }
};

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Eight lanes per 32-element block, four consecutive elements per lane.
// E8 = true: E4M3FN elements (codes [m][k]); false: E2M1 (codes [m][k/2]).
template <typename XT, bool E8>
__global__ __launch_bounds__(256) void k_quantize_mx(const XT *__restrict__ x, int64_t ldx, uint8_t *__restrict__ codes,
                                                     uint8_t *__restrict__ scales, int64_t m, int64_t k) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t quads = k / 4;
    const int64_t row = t / quads;
    if (row >= m) return;  // whole 8-lane groups leave together (k / 4 is a multiple of 8)
    const int64_t c4 = 4 * (t % quads);
    const f32x4 v = XLoad4<XT>::at(x + row * ldx + c4);
    // block maximum over the 8 lanes (bit patterns of magnitudes order like the values)
    uint32_t a = max(max(__float_as_uint(v.x) & 0x7FFFFFFFu, __float_as_uint(v.y) & 0x7FFFFFFFu),
                     max(__float_as_uint(v.z) & 0x7FFFFFFFu, __float_as_uint(v.w) & 0x7FFFFFFFu));
    a = max(a, dpp_u32<0xB1>(a));   // quad_perm [1,0,3,2]
    a = max(a, dpp_u32<0x4E>(a));   // quad_perm [2,3,0,1]
    a = max(a, dpp_u32<0x141>(a));  // row_half_mirror: all 8 lanes of the block
    // floor(log2 amax) is the exponent field - 127 for normal amax; zero or
    // subnormal amax gives <= -127 - emax, which clamps to -127 anyway
    constexpr int EMAX = E8 ? 8 : 2;
    int e = (int)(a >> 23) - 127 - EMAX;
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
    const float s0 = __builtin_amdgcn_ldexpf(v.x, -e), s1 = __builtin_amdgcn_ldexpf(v.y, -e);
    const float s2 = __builtin_amdgcn_ldexpf(v.z, -e), s3 = __builtin_amdgcn_ldexpf(v.w, -e);
    if (E8) {
        typedef short v2s __attribute__((ext_vector_type(2)));
        const float lim = 448.0f;
        v2s lo = {0, 0}, hi = {0, 0};
        lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, __builtin_fminf(__builtin_fmaxf(s0, -lim), lim),
                                                      __builtin_fminf(__builtin_fmaxf(s1, -lim), lim), 1.0f, false);
        hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, __builtin_fminf(__builtin_fmaxf(s2, -lim), lim),
                                                      __builtin_fminf(__builtin_fmaxf(s3, -lim), lim), 1.0f, false);
        const uint32_t w = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)hi[0] << 16);
        *reinterpret_cast<uint32_t *>(codes + row * k + c4) = w;
    } else {
        uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, s0, s1, 1.0f, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, s2, s3, 1.0f, 1);
        *reinterpret_cast<uint16_t *>(codes + row * (k / 2) + c4 / 2) = (uint16_t)w;
    }
    if ((threadIdx.x & 7) == 0) scales[row * (k / 32) + c4 / 32] = (uint8_t)(e + 127);
}

// ------------------------------------------------------------------ GEMM, 256 x 256 tiles

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

__device__ __forceinline__ void dma16(const void *g, void *lds_base) {
    __builtin_amdgcn_global_load_lds((glb_void *)g, (lds_void *)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void *g, void *lds_base) {
    __builtin_amdgcn_global_load_lds((glb_void *)g, (lds_void *)lds_base, 4, 0, 0);
}
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

constexpr int BM = 256, BN = 256, BKS = 256;  // tile rows, tile columns, k per LDS stage
constexpr int WAVES = 8;                      // 4 x 2 waves, each 64 x 128 = 2 x 4 MFMA tiles
constexpr int WGM = 4, WGN = 2, TM = 2, TN = 4;

// LDS stage (k = 256): A (activation codes) and B (weight codes), 256 rows of
// (256 / 2 / ELEM) bytes, then the 8 scale bytes of each row of A and of B.
// Code piece p (16 bytes = 32 E2M1 values) of row n sits at
//   n * ROW + ((p ^ g(n)) * 16),  g(n) = (n % 8) ^ ((n / 8) & 1)
// so that 8 or 16 consecutive rows read at one p hit distinct banks.
template <bool A8>
struct Lay {
    static constexpr int AROW = A8 ? 256 : 128;  // bytes of A codes per row per stage
    static constexpr int BROW = 128;
    static constexpr int A_OFF = 0, B_OFF = BM * AROW;
    static constexpr int SA_OFF = B_OFF + BN * BROW, SB_OFF = SA_OFF + BM * 8;
    static constexpr int STAGE = SB_OFF + BN * 8;
    static constexpr int NST = A8 ? 1 : 2;  // stages in the ring (LDS holds 160 KB)
    static constexpr int BYTES = NST * STAGE;
};

__device__ __forceinline__ int gsw(int n) { return (n % 8) ^ ((n / 8) & 1); }

// Copies of one stage: 32 row groups of 8 rows per operand (16-byte pieces,
// swizzled on the global side so the LDS image is the layout above) and 8
// groups of 32 rows per scale array (4 bytes per lane).
// Rows past M (N) re-read row M-1 (N-1); their results are not stored.
// Offsets are 32-bit from the (uniform) tensor bases: the launcher sends
// tensors of 2 GB or more to the small kernel.
template <bool A8>
struct StageCopy {
    static constexpr int AP = Lay<A8>::AROW / 16;         // 16-byte pieces per A row
    static constexpr int RPC = 64 / AP;                   // A rows per copy
    static constexpr int NA = BM / RPC / WAVES;           // A copies per wave
    static constexpr int NB = BN / 8 / WAVES;             // B copies per wave
    static constexpr int COPIES = NA + NB + 2;
    const uint8_t *xc, *xs, *wc, *ws;                     // tensor bases
    uint32_t ag[NA], bg[NB], sag, sbg;                    // per-lane byte offsets at k = 0
    int ao, bo, sao, sbo;                                 // LDS offsets of this wave's first copies

    __device__ __forceinline__ StageCopy(const uint8_t *xc_, const uint8_t *xs_, const uint8_t *wc_,
                                         const uint8_t *ws_, int64_t M, int64_t N, int64_t K, int64_t m0, int64_t n0,
                                         int lane, int wave)
        : xc(xc_), xs(xs_), wc(wc_), ws(ws_) {
        using L = Lay<A8>;
        const int64_t arow = A8 ? K : K / 2;
#pragma unroll
        for (int q = 0; q < NA; ++q) {
            // copy c = wave + WAVES q holds rows RPC c .. RPC c + RPC - 1
            const int r = (wave + WAVES * q) * RPC + lane / AP, sl = lane % AP;
            const int p = sl ^ (gsw(r) & (AP - 1));
            ag[q] = (uint32_t)(min(m0 + r, M - 1) * arow + 16 * p);
        }
#pragma unroll
        for (int q = 0; q < NB; ++q) {
            const int r = (wave + WAVES * q) * 8 + lane / 8, sl = lane % 8;
            bg[q] = (uint32_t)(min(n0 + r, N - 1) * (K / 2) + 16 * (sl ^ gsw(r)));
        }
        ao = L::A_OFF + wave * 1024;
        bo = L::B_OFF + wave * 1024;
        const int r = wave * 32 + lane / 2, h = lane % 2;  // one 4-byte copy per wave covers 32 rows
        sag = (uint32_t)(min(m0 + r, M - 1) * (K / 32) + 4 * h);
        sbg = (uint32_t)(min(n0 + r, N - 1) * (K / 32) + 4 * h);
        sao = L::SA_OFF + wave * 256;
        sbo = L::SB_OFF + wave * 256;
    }

    __device__ __forceinline__ void copy(uint8_t *stage, int64_t k0) const {
        const uint32_t ak = (uint32_t)(A8 ? k0 : k0 / 2), bk = (uint32_t)(k0 / 2), sk = (uint32_t)(k0 / 32);
#pragma unroll
        for (int q = 0; q < NA; ++q) dma16(xc + (ag[q] + ak), stage + ao + q * WAVES * 1024);
#pragma unroll
        for (int q = 0; q < NB; ++q) dma16(wc + (bg[q] + bk), stage + bo + q * WAVES * 1024);
        dma4(xs + (sag + sk), stage + sao);
        dma4(ws + (sbg + sk), stage + sbo);
    }
};

// A 4-byte-element operand (E2M1) uses the low half of the register block;
// the upper half is left undefined so that no registers are spent on it.
__device__ __forceinline__ v8i widen(u32x4 v) {
    const v8i w = __builtin_bit_cast(v8i, __builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1));
    return w;
}

template <bool A8>
__device__ __forceinline__ void read_frags(const uint8_t *sm, int aoff, int boff, v8i (&a)[TM], v8i (&b)[TN]) {
    using L = Lay<A8>;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        if (A8) {
            const u32x4 lo = *reinterpret_cast<const u32x4 *>(sm + aoff + i * 32 * L::AROW);
            const u32x4 hi = *reinterpret_cast<const u32x4 *>(sm + (aoff ^ 16) + i * 32 * L::AROW);
            a[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        } else {
            a[i] = widen(*reinterpret_cast<const u32x4 *>(sm + aoff + i * 32 * L::AROW));
        }
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) b[j] = widen(*reinterpret_cast<const u32x4 *>(sm + boff + j * 32 * L::BROW));
}

template <typename YT>
__device__ __forceinline__ void put_out(YT *y, int64_t idx, float v);
template <>
__device__ __forceinline__ void put_out<uint16_t>(uint16_t *y, int64_t idx, float v) {
    y[idx] = bf16_bits_rne(v);
}
template <>
__device__ __forceinline__ void put_out<float>(float *y, int64_t idx, float v) {
    y[idx] = v;
}

// Y tile 256 x 256: wave (wm, wn) owns rows wm*64 .. +63 and columns
// wn*128 .. +127 as 2 x 4 MFMA tiles of 32 x 32. A k-step of 64 is one MFMA
// per tile: lane half lh holds k 32 lh .. 32 lh + 31 of the step (piece 2 s + lh
// of a stage) for its row (A) or column (B), under one E8M0 byte each.
template <bool A8, typename YT>
__global__ __launch_bounds__(WAVES * 64) void k_mxgemm(const uint8_t *__restrict__ xc,
                                                       const uint8_t *__restrict__ xs,
                                                       const uint8_t *__restrict__ wc,
                                                       const uint8_t *__restrict__ ws, YT *__restrict__ Y,
                                                       int64_t ldy, int64_t M, int64_t N, int64_t K, int tiles_m,
                                                       int tiles_n) {
    using L = Lay<A8>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[L::BYTES];
    // XCD-aware banded order (as in the bf16 GEMM): the workgroups of one XCD
    // cover a block of GM tile rows x (per-XCD count / GM) tile columns
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

    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wm = wave / WGN, wn = wave % WGN;
    const int lr = lane % 32, lh = lane / 32;
    const int nst = (int)(K / BKS);

    // per-lane LDS offsets (row bases; the piece slot is added per step)
    const int ra = wm * 64 + lr, rbn = wn * 128 + lr;
    const int gl = gsw(lr);  // g(n) of every row this lane reads: n = 16 * (...) + lr
    int a_off[4], b_off[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int p = 2 * s + lh;
        a_off[s] = A8 ? (L::A_OFF + ra * L::AROW + (((2 * p) ^ gl) * 16))  // fp8: 32 bytes = pieces 2p, 2p+1
                      : (L::A_OFF + ra * L::AROW + ((p ^ gl) * 16));
        b_off[s] = L::B_OFF + rbn * L::BROW + ((p ^ gl) * 16);
    }
    const int sa_off = L::SA_OFF + ra * 8, sb_off = L::SB_OFF + rbn * 8;

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

    const StageCopy<A8> cp(xc, xs, wc, ws, M, N, K, m0, n0, lane, wave);
    cp.copy(smem, 0);
    if (L::NST > 1 && nst > 1) cp.copy(smem + L::STAGE, BKS);

    for (int st = 0; st < nst; ++st) {
        uint8_t *const sm = smem + (L::NST > 1 ? (st & 1) * L::STAGE : 0);
        // this stage's copies have landed once at most the next stage's remain
        if (L::NST > 1 && st + 1 < nst) __builtin_amdgcn_s_waitcnt(0xF70 | StageCopy<A8>::COPIES);
        else __builtin_amdgcn_s_waitcnt(0xF70);
        lds_barrier();
        uint32_t sa[TM][2], sb[TN][2];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const u32x2 v = *reinterpret_cast<const u32x2 *>(sm + sa_off + i * 32 * 8);
            sa[i][0] = v.x >> (8 * lh);
            sa[i][1] = v.y >> (8 * lh);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const u32x2 v = *reinterpret_cast<const u32x2 *>(sm + sb_off + j * 32 * 8);
            sb[j][0] = v.x >> (8 * lh);
            sb[j][1] = v.y >> (8 * lh);
        }
        // two fragment sets: step s + 1 is read while step s's MFMAs run
        v8i a[2][TM], b[2][TN];
        read_frags<A8>(sm, a_off[0], b_off[0], a[0], b[0]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s < 3) read_frags<A8>(sm, a_off[s + 1], b_off[s + 1], a[(s + 1) & 1], b[(s + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int sai = (int)(sa[i][s / 2] >> (16 * (s % 2)));
                    const int sbj = (int)(sb[j][s / 2] >> (16 * (s % 2)));
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[s & 1][i], b[s & 1][j], acc[i][j],
                                                                               A8 ? 0 : 4, 4, 0, sai, 0, sbj);
                }
            __builtin_amdgcn_sched_barrier(0);
        }
        // every wave is done with this buffer before it is refilled
        if (st + L::NST < nst) {
            lds_barrier();
            cp.copy(sm, (int64_t)(st + L::NST) * BKS);
        }
    }

#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t n = n0 + wn * 128 + 32 * j + lr;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t m = m0 + wm * 64 + 32 * i + 8 * (v / 4) + 4 * lh + (v % 4);
                if (m < M && n < N) put_out<YT>(Y, m * ldy + n, acc[i][j][v]);
            }
        }
}

// Any shape with k % 32 == 0: one wave per 32 x 32 tile of Y, fragments read
// straight from global memory, the k-step past the end padded with zero
// codes under scale byte 127.
template <bool A8, typename YT>
__global__ __launch_bounds__(256) void k_mxgemm_small(const uint8_t *__restrict__ xc, const uint8_t *__restrict__ xs,
                                                      const uint8_t *__restrict__ wc, const uint8_t *__restrict__ ws,
                                                      YT *__restrict__ Y, int64_t ldy, int64_t M, int64_t N,
                                                      int64_t K, int64_t tiles_n) {
    const int64_t tile = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
    const int64_t tm = tile / tiles_n, tn = tile % tiles_n;
    const int64_t m0 = tm * 32, n0 = tn * 32;
    if (m0 >= M) return;  // whole waves only; no barrier follows
    const int lane = threadIdx.x % kWave;
    const int lr = lane % 32, lh = lane / 32;
    const int64_t ma = min(m0 + lr, M - 1), nb = min(n0 + lr, N - 1);
    const int64_t xrow = A8 ? K : K / 2;
    f32x16 acc = f32x16{};
    for (int64_t k0 = 0; k0 < K; k0 += 64) {
        const int64_t kk = k0 + 32 * lh;
        const bool in = kk < K;
        v8i a, b;
        if (A8) {
            const u32x4 lo = in ? ld16(xc + ma * xrow + kk) : u32x4{0u, 0u, 0u, 0u};
            const u32x4 hi = in ? ld16(xc + ma * xrow + kk + 16) : u32x4{0u, 0u, 0u, 0u};
            a = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        } else {
            const u32x4 v = in ? ld16(xc + ma * xrow + kk / 2) : u32x4{0u, 0u, 0u, 0u};
            a = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        }
        const u32x4 w = in ? ld16(wc + nb * (K / 2) + kk / 2) : u32x4{0u, 0u, 0u, 0u};
        b = v8i{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
        const int sa = in ? xs[ma * (K / 32) + kk / 32] : 127;
        const int sb = in ? ws[nb * (K / 32) + kk / 32] : 127;
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, A8 ? 0 : 4, 4, 0, sa, 0, sb);
    }
    const int64_t n = n0 + lr;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int64_t m = m0 + 8 * (v / 4) + 4 * lh + (v % 4);
        if (m < M && n < N) put_out<YT>(Y, m * ldy + n, acc[v]);
    }
}

template <bool A8, typename YT>
hipError_t run_mxgemm(const qbn_tensor &w, int64_t m, const void *xc, const void *xs, void *y, int64_t ldy,
                      hipStream_t s) {
    const int64_t xbytes = m * (A8 ? w.k : w.k / 2), wbytes = w.n * (w.k / 2);
    const bool big = m >= BM && w.n >= BN && (w.k % BKS) == 0 && xbytes < ((int64_t)1 << 31) &&
                     wbytes < ((int64_t)1 << 31) && ((uintptr_t)xs % 4) == 0 && ((uintptr_t)w.scales % 4) == 0;
    if (big) {
        const int64_t tm = (m + BM - 1) / BM, tn = (w.n + BN - 1) / BN;
        hipLaunchKernelGGL((k_mxgemm<A8, YT>), dim3((unsigned)(tm * tn)), dim3(WAVES * 64), 0, s,
                           (const uint8_t *)xc, (const uint8_t *)xs, (const uint8_t *)w.data,
                           (const uint8_t *)w.scales, (YT *)y, ldy, m, w.n, w.k, (int)tm, (int)tn);
    } else {
        const int64_t tm = (m + 31) / 32, tn = (w.n + 31) / 32;
        hipLaunchKernelGGL((k_mxgemm_small<A8, YT>), dim3((unsigned)((tm * tn + 3) / 4)), dim3(256), 0, s,
                           (const uint8_t *)xc, (const uint8_t *)xs, (const uint8_t *)w.data,
                           (const uint8_t *)w.scales, (YT *)y, ldy, m, w.n, w.k, tn);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_mx(const void *x, int x_dtype, int64_t m, int64_t k, int64_t ldx, int x_format,
                              void *codes, void *scales, hipStream_t s) {
    const int64_t threads = m * (k / 4);
    const unsigned grid = (unsigned)((threads + 255) / 256);
    const bool e8 = x_format == QBN_MXFP8;
    if (x_dtype == QBN_BF16) {
        if (e8)
            hipLaunchKernelGGL((k_quantize_mx<__bf16, true>), dim3(grid), dim3(256), 0, s, (const __bf16 *)x, ldx,
                               (uint8_t *)codes, (uint8_t *)scales, m, k);
        else
            hipLaunchKernelGGL((k_quantize_mx<__bf16, false>), dim3(grid), dim3(256), 0, s, (const __bf16 *)x, ldx,
                               (uint8_t *)codes, (uint8_t *)scales, m, k);
    } else {
        if (e8)
            hipLaunchKernelGGL((k_quantize_mx<float, true>), dim3(grid), dim3(256), 0, s, (const float *)x, ldx,
                               (uint8_t *)codes, (uint8_t *)scales, m, k);
        else
            hipLaunchKernelGGL((k_quantize_mx<float, false>), dim3(grid), dim3(256), 0, s, (const float *)x, ldx,
                               (uint8_t *)codes, (uint8_t *)scales, m, k);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_mx(const qbn_tensor &w, int64_t m, int x_format, const void *xcodes, const void *xscales,
                          void *y, int y_dtype, int64_t ldy, hipStream_t s) {
    const bool e8 = x_format == QBN_MXFP8;
    if (y_dtype == QBN_F32)
        return e8 ? run_mxgemm<true, float>(w, m, xcodes, xscales, y, ldy, s)
                  : run_mxgemm<false, float>(w, m, xcodes, xscales, y, ldy, s);
    return e8 ? run_mxgemm<true, uint16_t>(w, m, xcodes, xscales, y, ldy, s)
              : run_mxgemm<false, uint16_t>(w, m, xcodes, xscales, y, ldy, s);
}

}  // namespace qbn
