// Decode GEMV straight from the integer int4 layouts ("Bit Packing
// Architecture", "Real layouts compared"; the GPTQ / AWQ / Q4_0 rows of the
// adjacent-formats list):
//   GPTQ4 / AWQ4: y[c] = sum_k s[k/g][c] * (q[k][c] - z[k/g][c]) * x[k], the
//     weight stored input-major (K x N logical matrix; GPTQ packs 8 k per
//     int32 word of one column, AWQ 8 columns per word of one k, in the slot
//     order 0,2,4,6,1,3,5,7);
//   Q4_0: y[r] = sum_b d_b * sum_j (q_j - 8) * x[32 b + j], rows of 18-byte
//     blocks (fp16 d, byte j = element j low | element j + 16 high).
// The integer difference q - z (or q - 8) is exact in binary32; the group
// scale multiplies each group's partial sum once. Reductions run in a fixed
// order (DPP / shuffles / LDS), so results are deterministic.
#include "qbn_device.h"
#include "qbn_launch.h"

namespace qbn {
namespace {

template <typename XT>
struct X8;  // eight consecutive activations: raw load, then binary32
template <>
struct X8<float> {
    struct Raw {
        f32x4 a, b;
    };
    __device__ __forceinline__ static Raw raw(const float *x, int64_t k) {
        return Raw{*reinterpret_cast<const f32x4 *>(x + k), *reinterpret_cast<const f32x4 *>(x + k + 4)};
    }
    __device__ __forceinline__ static void unpack(const Raw &r, float (&v)[8]) {
        v[0] = r.a.x, v[1] = r.a.y, v[2] = r.a.z, v[3] = r.a.w, v[4] = r.b.x, v[5] = r.b.y, v[6] = r.b.z,
        v[7] = r.b.w;
    }
};
template <>
struct X8<__bf16> {
    typedef u32x4 Raw;
    __device__ __forceinline__ static Raw raw(const __bf16 *x, int64_t k) { return ld16(x + k); }
    __device__ __forceinline__ static void unpack(const Raw &w, float (&v)[8]) {
        const uint32_t p[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __builtin_bit_cast(float, p[i] << 16);
            v[2 * i + 1] = __builtin_bit_cast(float, p[i] & 0xFFFF0000u);
        }
    }
};

// Byte B of a word as binary32 (one v_cvt_f32_ubyteB).
template <int B>
__device__ __forceinline__ float ubyte(uint32_t w) {
    return (float)((w >> (8 * B)) & 0xFFu);
}

// q_m - z[m] (exact) for the eight 4-bit codes q_m of a word (bits 4m..4m+3).
// Each nibble is read as a binary16 subnormal (q * 2^-24, or 16 q * 2^-24
// for the high nibble of a byte) straight from masked bits, and one mixed
// fma per code scales it back and subtracts the zero point.
__device__ __forceinline__ void nib_minus(uint32_t v, const float (&z)[8], float (&w)[8]) {
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

// ------------------------------------------------------------------ GPTQ / AWQ
// A workgroup covers CW lanes x 8 columns and all of K, split into SL =
// threads / CW slices; a lane takes rounds of SPL consecutive 8-row steps
// (SPL divides group / 8, so a round lies in one group), requests all of a
// round's codes, activations, scales and zero points before multiplying,
// and keeps 8 column sums. (Holding a second round in registers to overlap
// the next requests with the arithmetic measured no faster.) GPTQ: CW = 4 (a lane's 8 columns
// are 32 contiguous bytes, 4 lanes a 128-byte line per step). AWQ: CW = 8
// (one word of 8 columns per lane per row, 32 bytes per row across the 8
// lanes). Narrower column blocks (CW = 1 or 2, more workgroups for the 256
// CUs) lose the whole-line loads and measured 10-60% slower.
template <int FMT, int THREADS_ = (FMT == QBN_GPTQ4 ? 256 : 512), int CW_ = (FMT == QBN_GPTQ4 ? 4 : 8)>
struct AffShape {
    static constexpr int CW = CW_;
    static constexpr int THREADS = THREADS_;
    static constexpr int SL = THREADS / CW;
    static constexpr int WAVES = THREADS / 64;
};

// The raw bytes of one round: SPL steps of codes and activations, and the
// round's group scales and zero points (VEC: as vectors; else per column).
template <int SPL, typename XT>
struct AffRound {
    uint32_t w[SPL][8];
    typename X8<XT>::Raw x[SPL];
    u32x4 s4;
    u32x2 z2;
    uint16_t se[8];
    uint8_t ze[8];
};

template <int FMT, bool VEC, int SPL, typename XT>
__device__ __forceinline__ void aff_load(AffRound<SPL, XT> &rd, const uint32_t *__restrict__ qw,
                                         const uint16_t *__restrict__ sc, const uint8_t *__restrict__ zp,
                                         const XT *__restrict__ x, int64_t n, int64_t group, int64_t c0,
                                         const int64_t (&cc)[8], int64_t jb) {
#pragma unroll
    for (int st = 0; st < SPL; ++st) {
        const int64_t j = jb + st;
        if (FMT == QBN_GPTQ4) {
            // word i holds rows 8j .. 8j+7 of column c0 + i, row 8j + e at bits 4e
            if (VEC) {
                const u32x4 a = ld16(qw + j * n + c0), b = ld16(qw + j * n + c0 + 4);
                rd.w[st][0] = a.x, rd.w[st][1] = a.y, rd.w[st][2] = a.z, rd.w[st][3] = a.w;
                rd.w[st][4] = b.x, rd.w[st][5] = b.y, rd.w[st][6] = b.z, rd.w[st][7] = b.w;
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) rd.w[st][i] = qw[j * n + cc[i]];
            }
        } else {
            // word e holds columns c0 .. c0+7 of row 8j + e
#pragma unroll
            for (int e = 0; e < 8; ++e) rd.w[st][e] = qw[(8 * j + e) * (n / 8) + c0 / 8];
        }
        rd.x[st] = X8<XT>::raw(x, 8 * j);
    }
    const int64_t gi = (8 * jb) / group;
    if (VEC) {
        rd.s4 = ld16(sc + gi * n + c0);
        rd.z2 = ld8(zp + gi * n + c0);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            rd.se[i] = sc[gi * n + cc[i]];
            rd.ze[i] = zp[gi * n + cc[i]];
        }
    }
}

// Multiply one round into the 8 column sums: per step, q - z times x; the
// round's group scale multiplies its partial sums once.
template <int FMT, bool VEC, int SPL, typename XT>
__device__ __forceinline__ void aff_compute(const AffRound<SPL, XT> &cur, float (&tot)[8]) {
    float sf[8], zf[8];
    if (VEC) {
        const uint32_t sw[4] = {cur.s4.x, cur.s4.y, cur.s4.z, cur.s4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sf[2 * i] = f16_bits_f32(sw[i] & 0xFFFFu);
            sf[2 * i + 1] = f16_bits_f32(sw[i] >> 16);
        }
        zf[0] = ubyte<0>(cur.z2.x), zf[1] = ubyte<1>(cur.z2.x), zf[2] = ubyte<2>(cur.z2.x);
        zf[3] = ubyte<3>(cur.z2.x), zf[4] = ubyte<0>(cur.z2.y), zf[5] = ubyte<1>(cur.z2.y);
        zf[6] = ubyte<2>(cur.z2.y), zf[7] = ubyte<3>(cur.z2.y);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            sf[i] = f16_bits_f32(cur.se[i]);
            zf[i] = (float)cur.ze[i];
        }
    }
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int st = 0; st < SPL; ++st) {
        float xv[8];
        X8<XT>::unpack(cur.x[st], xv);
        if (FMT == QBN_GPTQ4) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float zi[8] = {zf[i], zf[i], zf[i], zf[i], zf[i], zf[i], zf[i], zf[i]};
                float d[8];
                nib_minus(cur.w[st][i], zi, d);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[i] = fmaf(d[e], xv[e], acc[i]);
            }
        } else {
            // slot tt of a word is column 0,2,4,6,1,3,5,7 [tt]
            constexpr int col[8] = {0, 2, 4, 6, 1, 3, 5, 7};
            const float zs[8] = {zf[0], zf[2], zf[4], zf[6], zf[1], zf[3], zf[5], zf[7]};  // by slot
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float d[8];
                nib_minus(cur.w[st][e], zs, d);
#pragma unroll
                for (int tt = 0; tt < 8; ++tt) acc[col[tt]] = fmaf(d[tt], xv[e], acc[col[tt]]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) tot[i] = fmaf(sf[i], acc[i], tot[i]);
}

// VEC: the 8 columns of a lane are loaded as 16-byte (codes, scales) and
// 8-byte (zeros) vectors; needs n % 8 == 0 and 16-byte aligned data and
// scales. Otherwise element loads with columns past n clamped (not stored).
template <int FMT, typename XT, bool VEC, int SPL, int THREADS = AffShape<FMT>::THREADS,
          int CWT = AffShape<FMT>::CW>
__global__ __launch_bounds__(THREADS) void k_gemv_affine(const uint32_t *__restrict__ qw, const uint16_t *__restrict__ sc,
                                                     const uint8_t *__restrict__ zp, const XT *__restrict__ x,
                                                     float *__restrict__ y, int64_t n, int64_t k, int64_t group) {
    using Sh = AffShape<FMT, THREADS, CWT>;
    constexpr int CW = Sh::CW, SL = Sh::SL, WAVES = Sh::WAVES;
    __shared__ float red[WAVES][CW][8];
    const int t = threadIdx.x;
    const int cw = t % CW, sl = t / CW;
    // Workgroups are dealt to the 8 XCDs in turn (block b to XCD b % 8). The
    // column blocks that share cache lines (AWQ: four blocks per 128-byte
    // line) are given to one XCD, so that its L2 serves the line once:
    // XCD x takes logical blocks x * q + min(x, r) onwards (q, r = grid / 8,
    // grid % 8), in dispatch order.
    const int64_t nblk = gridDim.x, q8 = nblk / 8, r8 = nblk % 8, xcd = blockIdx.x % 8;
    const int64_t blk = xcd * q8 + min(xcd, r8) + blockIdx.x / 8;
    const int64_t c0 = blk * (8 * CW) + 8 * cw;
    const int64_t nsteps = k / 8;  // a multiple of SPL
    int64_t cc[8];                 // clamped columns (element loads)
#pragma unroll
    for (int i = 0; i < 8; ++i) cc[i] = min(c0 + i, n - 1);
    const bool live = c0 < n;

    float tot[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) tot[i] = 0.0f;
    // rounds of this lane: jb = sl * SPL + r * SL * SPL
    for (int64_t jb = live ? (int64_t)sl * SPL : nsteps; jb < nsteps; jb += (int64_t)SL * SPL) {
        AffRound<SPL, XT> rd;
        aff_load<FMT, VEC>(rd, qw, sc, zp, x, n, group, c0, cc, jb);
        aff_compute<FMT, VEC>(rd, tot);
    }

    // slices: the wave's 64 / CW, then the waves in order
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float v = tot[i];
#pragma unroll
        for (int off = CW; off < 64; off *= 2) v += __shfl_xor(v, off, 64);
        tot[i] = v;
    }
    const int lane = t % 64, wave = t / 64;
    if (lane < CW) {
#pragma unroll
        for (int i = 0; i < 8; ++i) red[wave][lane][i] = tot[i];
    }
    __syncthreads();
    if (wave == 0 && lane < CW && live) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float v = red[0][lane][i];
#pragma unroll
            for (int wv = 1; wv < WAVES; ++wv) v += red[wv][lane][i];
            if (c0 + i < n) y[c0 + i] = v;
        }
    }
}

// Balanced form (GPTQ4, VEC layout): the n / 8 column groups of 8 are dealt out
// evenly, floor or ceil(groups / grid) consecutive groups per workgroup, with
// grid = 256 (one workgroup per compute unit; one per group when there are
// fewer) unless that would need more than 8 groups per workgroup. The
// 11008-column layer then runs 5 or 6 groups per compute unit instead of 1
// or 2 blocks of 4 (with one cached weight copy the blocks took as long as 2
// full rounds: 10.2 us against 6.6 us for 8192 columns). k is split
// into 128 slices of SPL-step rounds (an 8-row step each); lane t of a
// workgroup with CWB groups owns group t % CWB and slice t / CWB (whole
// lines: consecutive lanes read consecutive 32-byte column groups of one
// row). The slices' column sums go through LDS and are added in a fixed
// order: 16 threads per column each add 8 consecutive slices, then a
// butterfly over the 16.
constexpr int kBalSlices = 128;
constexpr int kBalMaxGroups = 8;
constexpr int kBalCUs = 256;

template <int FMT, typename XT, int SPL>
__global__ __launch_bounds__(kBalMaxGroups * kBalSlices) void k_gemv_affine_bal(
    const uint32_t *__restrict__ qw, const uint16_t *__restrict__ sc, const uint8_t *__restrict__ zp,
    const XT *__restrict__ x, float *__restrict__ y, int64_t n, int64_t k, int64_t group) {
    __shared__ float red[kBalSlices][kBalMaxGroups * 8];
    const int t = threadIdx.x;
    const int64_t groups = n / 8;
    // XCD-aware order, as in k_gemv_affine: neighbouring column ranges (which
    // share cache lines at their ends) go to one XCD
    const int64_t nblk = gridDim.x, q8 = nblk / 8, r8 = nblk % 8, xcd = blockIdx.x % 8;
    const int64_t blk = xcd * q8 + min(xcd, r8) + blockIdx.x / 8;
    const int64_t g0 = blk * groups / nblk, g1 = (blk + 1) * groups / nblk;
    const int cwb = (int)(g1 - g0);  // 1 .. kBalMaxGroups
    const bool live = t < cwb * kBalSlices;
    const int cw = live ? t % cwb : 0, sl = live ? t / cwb : 0;
    const int64_t c0 = (g0 + cw) * 8;
    const int64_t nsteps = k / 8;
    int64_t cc[8];  // (element loads only; the VEC path reads 8 columns as vectors)
#pragma unroll
    for (int i = 0; i < 8; ++i) cc[i] = c0 + i;

    float tot[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) tot[i] = 0.0f;
    for (int64_t jb = live ? (int64_t)sl * SPL : nsteps; jb < nsteps; jb += (int64_t)kBalSlices * SPL) {
        AffRound<SPL, XT> rd;
        aff_load<FMT, true, SPL>(rd, qw, sc, zp, x, n, group, c0, cc, jb);
        aff_compute<FMT, true, SPL>(rd, tot);
    }
    if (live) {
#pragma unroll
        for (int i = 0; i < 8; ++i) red[sl][8 * cw + i] = tot[i];
    }
    __syncthreads();
    // column j = t / 16 (of cwb * 8), part p = t % 16: slices 8p .. 8p + 7
    const int j = t / 16, pp = t % 16;
    float v = 0.0f;
    if (j < cwb * 8) {
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) v += red[8 * pp + s8][j];
    }
    v += __shfl_xor(v, 1, 16);
    v += __shfl_xor(v, 2, 16);
    v += __shfl_xor(v, 4, 16);
    v += __shfl_xor(v, 8, 16);
    if (j < cwb * 8 && pp == 0) y[g0 * 8 + j] = v;
}

template <int FMT, typename XT, int SPL>
hipError_t launch_affine_bal(const qbn_tensor &w, const XT *x, float *y, hipStream_t s) {
    const int64_t groups = w.n / 8;
    const int64_t grid = max(min((int64_t)kBalCUs, groups), (groups + kBalMaxGroups - 1) / kBalMaxGroups);
    hipLaunchKernelGGL((k_gemv_affine_bal<FMT, XT, SPL>), dim3((unsigned)grid), dim3(kBalMaxGroups * kBalSlices), 0, s,
                       (const uint32_t *)w.data, (const uint16_t *)w.scales, (const uint8_t *)w.zeros, x, y, w.n, w.k,
                       (int64_t)w.group);
    return hipGetLastError();
}

// ------------------------------------------------------------------ Q4_0
// One wave per R rows; lanes stride over the rows' blocks and load each
// block's activations once for all R rows.
struct __attribute__((packed, aligned(2))) Q40 {
    uint16_t d;
    uint32_t c[4];
};

template <typename XT>
struct X32;  // the 32 activations of a block as binary32
template <>
struct X32<float> {
    __device__ __forceinline__ static void at(const float *x, int64_t k, float (&v)[32]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const f32x4 a = *reinterpret_cast<const f32x4 *>(x + k + 4 * i);
            v[4 * i] = a.x, v[4 * i + 1] = a.y, v[4 * i + 2] = a.z, v[4 * i + 3] = a.w;
        }
    }
};
template <>
struct X32<__bf16> {
    __device__ __forceinline__ static void at(const __bf16 *x, int64_t k, float (&v)[32]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4 w = ld16(x + k + 8 * i);
            const uint32_t p[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                v[8 * i + 2 * h] = __builtin_bit_cast(float, p[h] << 16);
                v[8 * i + 2 * h + 1] = __builtin_bit_cast(float, p[h] & 0xFFFF0000u);
            }
        }
    }
};

// x is staged once per workgroup in LDS as binary32, 36 floats per block (32
// values and 4 of padding, so that 16 lanes reading their blocks' pieces at
// one index hit distinct banks). A lane's blocks (BPL of them, 64 apart) of
// all R rows are requested before any arithmetic. Rounds of 64 * BPL blocks.
// The first round's blocks are requested together with the workgroup's x
// pieces, before the staging barrier, which orders LDS only, so that the two
// memory latencies overlap instead of following one another.
constexpr int kQ40Pitch = 36;  // floats per staged block
constexpr int kQ40XP = 4;      // x pieces per thread issued ahead of the blocks (k <= 4096)

// Workgroup barrier ordering LDS only: unlike __syncthreads it does not wait
// for the blocks already requested.
__device__ __forceinline__ void q40_lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <typename XT>
struct XPiece;  // four x values (16-byte piece c of the staged row = x[4c .. 4c+3])
template <>
struct XPiece<float> {
    f32x4 v;
    __device__ __forceinline__ void load(const float *x, int64_t c) { v = *reinterpret_cast<const f32x4 *>(x + 4 * c); }
    __device__ __forceinline__ f32x4 f32() const { return v; }
};
template <>
struct XPiece<__bf16> {
    u32x2 v;
    __device__ __forceinline__ void load(const __bf16 *x, int64_t c) {
        v = ld8(reinterpret_cast<const uint16_t *>(x) + 4 * c);
    }
    __device__ __forceinline__ f32x4 f32() const {
        return f32x4{__builtin_bit_cast(float, v.x << 16), __builtin_bit_cast(float, v.x & 0xFFFF0000u),
                     __builtin_bit_cast(float, v.y << 16), __builtin_bit_cast(float, v.y & 0xFFFF0000u)};
    }
};

// LX = false (k too long for the staging buffer): x is read from global
// memory instead.
template <typename XT, int R, int BPL, bool LX>
__global__ __launch_bounds__(256) void k_gemv_q4_0(const uint8_t *__restrict__ blocks, const XT *__restrict__ x,
                                                   float *__restrict__ y, int64_t n, int64_t k) {
    extern __shared__ __attribute__((aligned(16))) float xs[];
    const int64_t nb = k / 32;
    const int lane = threadIdx.x % kWave;
    const int64_t r0 = ((int64_t)blockIdx.x * (256 / kWave) + threadIdx.x / kWave) * R;
    // blocks bb, bb + 64, ... of rows r0 .. r0 + R - 1 (indices clamped into
    // the matrix: waves past n and blocks past nb read valid bytes, unused)
    auto request = [&](Q40 (&blk)[BPL][R], int64_t bb) {
#pragma unroll
        for (int u = 0; u < BPL; ++u) {
            const int64_t b = min(bb + (int64_t)kWave * u, nb - 1);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int64_t row = min(r0 + r, n - 1);
                {
                    // blocks are read once: non-temporal loads, one per field
                    // (8.73 -> 8.45 us on 11008 x 4096)
                    const Q40 *q = reinterpret_cast<const Q40 *>(blocks + (row * nb + b) * 18);
                    blk[u][r].d = __builtin_nontemporal_load(&q->d);
#pragma unroll
                    for (int e = 0; e < 4; ++e) blk[u][r].c[e] = __builtin_nontemporal_load(&q->c[e]);
                }
            }
        }
    };
    // stage x: 16-byte pieces, piece p of block b at xs[36 b + 4 p]; the
    // first kQ40XP pieces of each thread are requested before the blocks
    const int64_t npc = LX ? 8 * nb : 0;
    XPiece<XT> xp[kQ40XP];
#pragma unroll
    for (int j = 0; j < kQ40XP; ++j) {
        const int64_t c = threadIdx.x + 256 * j;
        if (c < npc) xp[j].load(x, c);
    }
    Q40 blk[BPL][R];
    request(blk, lane);
#pragma unroll
    for (int j = 0; j < kQ40XP; ++j) {
        const int64_t c = threadIdx.x + 256 * j;
        if (c < npc) *reinterpret_cast<f32x4 *>(xs + kQ40Pitch * (c / 8) + 4 * (c % 8)) = xp[j].f32();
    }
    for (int64_t c = threadIdx.x + 256 * kQ40XP; c < npc; c += 256) {
        XPiece<XT> q;
        q.load(x, c);
        *reinterpret_cast<f32x4 *>(xs + kQ40Pitch * (c / 8) + 4 * (c % 8)) = q.f32();
    }
    q40_lds_barrier();
    if (r0 >= n) return;  // whole waves, after the only barrier
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0f;
    auto consume = [&](const Q40 (&blk)[BPL][R], int64_t bb) {
#pragma unroll
        for (int u = 0; u < BPL; ++u) {
            const int64_t b = bb + (int64_t)kWave * u;
            if (b >= nb) break;
            float xv[32];
            if (LX) {
#pragma unroll
                for (int p = 0; p < 8; ++p) {
                    const f32x4 a = *reinterpret_cast<const f32x4 *>(xs + kQ40Pitch * b + 4 * p);
                    xv[4 * p] = a.x, xv[4 * p + 1] = a.y, xv[4 * p + 2] = a.z, xv[4 * p + 3] = a.w;
                }
            } else {
                X32<XT>::at(x, 32 * b, xv);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float part = 0.0f;
                constexpr float z8[8] = {8.0f, 8.0f, 8.0f, 8.0f, 8.0f, 8.0f, 8.0f, 8.0f};
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    // byte 4w + i holds elements 4w + i (nibble 2i) and 16 + 4w + i (nibble 2i + 1)
                    float d[8];
                    nib_minus(blk[u][r].c[w], z8, d);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        part = fmaf(d[2 * i], xv[4 * w + i], part);
                        part = fmaf(d[2 * i + 1], xv[16 + 4 * w + i], part);
                    }
                }
                acc[r] = fmaf(f16_bits_f32(blk[u][r].d), part, acc[r]);
            }
        }
    };
    consume(blk, lane);
    for (int64_t bb = lane + (int64_t)kWave * BPL; bb < nb; bb += (int64_t)kWave * BPL) {
        Q40 nxt[BPL][R];
        request(nxt, bb);
        consume(nxt, bb);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = group_sum_last<64>(acc[r]);
    if (lane == kWave - 1) {
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (r0 + r < n) y[r0 + r] = acc[r];
    }
}

template <int FMT, typename XT, bool VEC, int TH, int SPL>
hipError_t launch_affine(const qbn_tensor &w, const XT *x, float *y, hipStream_t s) {
    constexpr int CW = AffShape<FMT>::CW;
    const unsigned grid = (unsigned)((w.n + 8 * CW - 1) / (8 * CW));
    hipLaunchKernelGGL((k_gemv_affine<FMT, XT, VEC, SPL, TH>), dim3(grid), dim3(TH), 0, s, (const uint32_t *)w.data,
                       (const uint16_t *)w.scales, (const uint8_t *)w.zeros, x, y, w.n, w.k, (int64_t)w.group);
    return hipGetLastError();
}

template <int FMT, typename XT, bool VEC>
hipError_t run_affine_spl(const qbn_tensor &w, const XT *x, float *y, hipStream_t s) {
    // Rounds of one step (any group size), measured on the 11008 x 4096 layer
    // against rounds of 2, 4 or 8: GPTQ with 512 threads 11.1 us (4-step
    // rounds 11.5, 1024 threads 11.3, 256 threads 12.6); AWQ with 1024 threads
    // 13.8 us (512 threads with 8-step rounds 14.6).
    if constexpr (FMT == QBN_GPTQ4) return launch_affine<FMT, XT, VEC, 512, 1>(w, x, y, s);
    else
        return launch_affine<FMT, XT, VEC, 1024, 1>(w, x, y, s);
}

template <int FMT, typename XT>
hipError_t run_affine(const qbn_tensor &w, const XT *x, float *y, hipStream_t s) {
    const bool vec = (w.n % 8) == 0 && ((uintptr_t)w.data % 16) == 0 && ((uintptr_t)w.scales % 16) == 0 &&
                     ((uintptr_t)w.zeros % 8) == 0;
    // GPTQ takes the balanced form, two 8-row steps per round when the group
    // allows (11008 x 4096: 8.8 us; one step 9.3, four 9.0; the blocked form
    // 10.2). AWQ measured slower in it (15.5-15.7 us against 11.4) and keeps
    // the blocked form.
    if (FMT == QBN_GPTQ4 && vec)
        return (w.group % 16 == 0) ? launch_affine_bal<FMT, XT, 2>(w, x, y, s) : launch_affine_bal<FMT, XT, 1>(w, x, y, s);
    return vec ? run_affine_spl<FMT, XT, true>(w, x, y, s) : run_affine_spl<FMT, XT, false>(w, x, y, s);
}

template <typename XT>
hipError_t run_q4_0(const qbn_tensor &w, const XT *x, float *y, hipStream_t s) {
    // two rows per wave: 11008 x 4096 in 8.7 us against 11.9 us with eight
    // (1376 waves then hold too few requests each to cover the latency, and
    // their arithmetic runs after the data arrives); four rows 8.9 us, one 9.0
    constexpr int R = 2, BPL = 2;
    const int64_t waves = (w.n + R - 1) / R;
    const size_t lds = (size_t)(w.k / 32) * kQ40Pitch * sizeof(float);
    if (lds <= 64 * 1024)
        hipLaunchKernelGGL((k_gemv_q4_0<XT, R, BPL, true>), dim3((unsigned)((waves + 3) / 4)), dim3(256), lds, s,
                           (const uint8_t *)w.data, x, y, w.n, w.k);
    else
        hipLaunchKernelGGL((k_gemv_q4_0<XT, R, BPL, false>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s,
                           (const uint8_t *)w.data, x, y, w.n, w.k);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_int4(const qbn_tensor &w, const void *x, int x_dtype, float *y, hipStream_t s) {
    const bool bf = (x_dtype == QBN_BF16);
    switch (w.format) {
    case QBN_GPTQ4:
        return bf ? run_affine<QBN_GPTQ4, __bf16>(w, (const __bf16 *)x, y, s)
                  : run_affine<QBN_GPTQ4, float>(w, (const float *)x, y, s);
    case QBN_AWQ4:
        return bf ? run_affine<QBN_AWQ4, __bf16>(w, (const __bf16 *)x, y, s)
                  : run_affine<QBN_AWQ4, float>(w, (const float *)x, y, s);
    case QBN_Q4_0:
        return bf ? run_q4_0<__bf16>(w, (const __bf16 *)x, y, s) : run_q4_0<float>(w, (const float *)x, y, s);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace qbn
