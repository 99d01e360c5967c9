// W4A8 decode on gfx950: int8 activation quantization and the Q4_K x int8
// GEMV ("Why 4-Bit Quantization Is King", section 7 and its W4A8 example,
// section 7b step 4, section 7c).
//
// Activations: the Q8_K grid of "Chapter 7 - NVFP4: the native lane",
// section 7.4.2: per 256 elements (a Q4_K super-block) the first element of
// largest magnitude mx, iscale = -127 / mx, codes RNE(x * iscale) clamped at
// 127, scale d = 1 / iscale (both divisions correctly rounded); blocks with
// |mx| < 2^-118 quantize to zero. The 32-element code sums of each block are
// written beside the codes, as the activation sums the integer route
// subtracts the minimum term with.
//
// GEMV: the integer route of section 7c. Weight nibbles stay small unsigned
// integers (0..15, so the signed 4 x int8 dot instruction takes them as
// they are), meet the activation codes in v_dot4_i32_i8, and each lane forms
// for its two sub-blocks j the exact integers
//     I1 = sum_j s_j * sum(q_w q_x),   I2 = sum_j m_j * sum(q_x)
// and then d * I1 - dmin * I2 in binary64: both products are exact there
// (11-bit fp16 significands times integers below 2^22), so this one
// rounding is the only one before the activation scale. That keeps the
// result within 2^-52 of each block's sum |w x_hat| even when the scale and
// minimum terms cancel, which binary32 (as the pages use) would not.
#include "qbn_device.h"
#include "qbn_launch.h"

namespace qbn {
namespace {

// ------------------------------------------------------------------ DPP helpers (integers)

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i32(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}

// Sum over aligned groups of 8 lanes; valid in every lane of the group.
__device__ __forceinline__ int group8_sum_i32(int v) {
    v += dpp_i32<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_i32<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_i32<0x141>(v);  // row_half_mirror
    return v;
}

// Maximum over the 64 lanes of non-negative binary32 values (as integers:
// their bit patterns order like the values), returned in every lane.
__device__ __forceinline__ float wave_max_nonneg(float a) {
    int v = __float_as_int(a);
    v = max(v, dpp_i32<0xB1>(v));
    v = max(v, dpp_i32<0x4E>(v));
    v = max(v, dpp_i32<0x141>(v));
    v = max(v, dpp_i32<0x140>(v));
    v = max(v, dpp_i32<0x142, 0xA>(v));  // row_bcast:15
    v = max(v, dpp_i32<0x143, 0xC>(v));  // row_bcast:31
    return __int_as_float(__builtin_amdgcn_readlane(v, 63));
}

// ------------------------------------------------------------------ activation quantization

template <typename XT>
struct X4;  // four consecutive activations as binary32
template <>
struct X4<float> {
    __device__ __forceinline__ static f32x4 load(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
};
template <>
struct X4<__bf16> {
    __device__ __forceinline__ static f32x4 load(const __bf16 *p) {
        const u32x2 w = ld8(p);
        return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u), __uint_as_float(w.y << 16),
                     __uint_as_float(w.y & 0xFFFF0000u)};
    }
};

// |v * iscale| <= 127 (1 + 2^-24)^2 for every element of the block, so the
// rounded code never falls below -127; only the upper clamp is needed.
__device__ __forceinline__ int q8_code(float v, float iscale) {
    const float t = __builtin_rintf(v * iscale);  // binary32 product, then nearest integer (ties to even)
    return (int)__builtin_fminf(t, 127.0f);
}

// One wave per 256-element block, lane l holding elements 4l .. 4l+3.
template <typename XT, int WPB>
__global__ __launch_bounds__(WPB * 64) void k_quantize_q8(const XT *__restrict__ x, int8_t *__restrict__ q,
                                                          float *__restrict__ d, int32_t *__restrict__ bsums,
                                                          int64_t nb) {
    const int64_t b = (int64_t)blockIdx.x * WPB + threadIdx.x / kWave;
    if (b >= nb) return;  // whole waves only; no barrier follows
    const int lane = threadIdx.x & (kWave - 1);
    const f32x4 v = X4<XT>::load(x + 256 * b + 4 * lane);
    const float a = __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(v.x), __builtin_fabsf(v.y)),
                                    __builtin_fmaxf(__builtin_fabsf(v.z), __builtin_fabsf(v.w)));
    const float amax = wave_max_nonneg(a);
    // the first element (lowest index) whose magnitude is amax: its lane is
    // the lowest lane holding one, and within the lane the lowest slot
    const float first = __builtin_fabsf(v.x) == amax ? v.x
                        : __builtin_fabsf(v.y) == amax ? v.y
                        : __builtin_fabsf(v.z) == amax ? v.z
                                                       : v.w;
    const uint64_t holders = __ballot(a == amax);
    const int src = holders ? __builtin_ctzll(holders) : 0;
    const float mx = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(first), src));
    uint32_t packed = 0;
    int part = 0;
    float scale = 0.0f;
    if (amax >= 0x1p-118f) {
        const float iscale = -127.0f / mx;
        scale = 1.0f / iscale;
        const int c0 = q8_code(v.x, iscale), c1 = q8_code(v.y, iscale), c2 = q8_code(v.z, iscale),
                  c3 = q8_code(v.w, iscale);
        packed = (uint32_t)(c0 & 0xFF) | ((uint32_t)(c1 & 0xFF) << 8) | ((uint32_t)(c2 & 0xFF) << 16) |
                 ((uint32_t)(c3 & 0xFF) << 24);
        part = c0 + c1 + c2 + c3;
    }
    reinterpret_cast<uint32_t *>(q + 256 * b)[lane] = packed;
    part = group8_sum_i32(part);
    if ((lane & 7) == 7) bsums[8 * b + (lane >> 3)] = part;
    if (lane == 0) d[b] = scale;
}

// ------------------------------------------------------------------ Q4_K x int8 GEMV

// Lane layout: 4 lanes per block, lane c (0..3) owning code bytes 32c .. 32c+31
// of the block (two 16-byte loads), i.e. all 32 weights of sub-blocks 2c (low
// nibbles) and 2c+1 (high nibbles), and the 64 activation codes
// 64c .. 64c+63 of the block. A wave holds SUB row groups of NBS = 16 / SUB
// block slots; slot s covers blocks s + NBS j, j < BPL, of each chunk of
// NBS * BPL blocks. The wave owns R consecutive row groups and requests all
// of their weights before its activations.

// Scales and minimums of the lane's sub-blocks 2c and 2c+1 from the 12 packed
// bytes B (h.y = B[0..3], h.z = B[4..7], h.w = B[8..11]), returned as the
// bytes [s_2c, s_2c+1, m_2c, m_2c+1]. Pairs j < 4 are the low six bits of
// B[j] (scale) and B[j+4] (minimum); pairs j >= 4 take the low / high nibble
// of B[j+4] and, as bits 4-5, the top two bits of B[j-4] / B[j]. With
// base = 2 (c & 1), both cases gather bytes base, base+1 of two words with
// one byte permute: U from (B[0..3], B[4..7]) and V from (B[8..11],
// B[8..11] >> 4).
struct PairSel {
    uint32_t sel;    // byte selector of the permutes
    uint32_t lmask;  // 0x3F3F3F3F (pairs 0..3) or 0x0F0F0F0F (pairs 4..7)
    uint32_t tmask;  // 0 or 0xC0C0C0C0
    bool hi;         // c >= 2
};

__device__ __forceinline__ PairSel pair_sel(int c) {
    PairSel p;
    const uint32_t base = 2u * (uint32_t)(c & 1);
    p.sel = base | ((base + 1u) << 8) | ((base + 4u) << 16) | ((base + 5u) << 24);
    p.hi = c >= 2;
    p.lmask = p.hi ? 0x0F0F0F0Fu : 0x3F3F3F3Fu;
    p.tmask = p.hi ? 0xC0C0C0C0u : 0u;
    return p;
}

__device__ __forceinline__ uint32_t scale_bytes(const u32x4 &h, const PairSel &p) {
    const uint32_t U = __builtin_amdgcn_perm(h.z, h.y, p.sel);
    const uint32_t V = __builtin_amdgcn_perm(h.w >> 4, h.w, p.sel);
    return ((p.hi ? V : U) & p.lmask) | ((U & p.tmask) >> 2);
}

struct XChunk {
    u32x4 lo[2], hi[2];  // activation codes 64c .. 64c+31 and 64c+32 .. 64c+63
    int32_t bs0, bs1;     // code sums of sub-blocks 2c and 2c+1
    double dx;            // activation scale of the block
};

// Integer sums of one lane for one block: D0 = sum over sub-block 2c of
// q_w q_x, D1 the same for 2c+1.
__device__ __forceinline__ void dot_chunk(const u32x4 &w0, const u32x4 &w1, const XChunk &xc, int &D0, int &D1) {
    const uint32_t m = 0x0F0F0F0Fu;
    int a = 0, b = 0;
    a = __builtin_amdgcn_sdot4((int)(w0.x & m), (int)xc.lo[0].x, a, false);
    b = __builtin_amdgcn_sdot4((int)((w0.x >> 4) & m), (int)xc.hi[0].x, b, false);
    a = __builtin_amdgcn_sdot4((int)(w0.y & m), (int)xc.lo[0].y, a, false);
    b = __builtin_amdgcn_sdot4((int)((w0.y >> 4) & m), (int)xc.hi[0].y, b, false);
    a = __builtin_amdgcn_sdot4((int)(w0.z & m), (int)xc.lo[0].z, a, false);
    b = __builtin_amdgcn_sdot4((int)((w0.z >> 4) & m), (int)xc.hi[0].z, b, false);
    a = __builtin_amdgcn_sdot4((int)(w0.w & m), (int)xc.lo[0].w, a, false);
    b = __builtin_amdgcn_sdot4((int)((w0.w >> 4) & m), (int)xc.hi[0].w, b, false);
    a = __builtin_amdgcn_sdot4((int)(w1.x & m), (int)xc.lo[1].x, a, false);
    b = __builtin_amdgcn_sdot4((int)((w1.x >> 4) & m), (int)xc.hi[1].x, b, false);
    a = __builtin_amdgcn_sdot4((int)(w1.y & m), (int)xc.lo[1].y, a, false);
    b = __builtin_amdgcn_sdot4((int)((w1.y >> 4) & m), (int)xc.hi[1].y, b, false);
    a = __builtin_amdgcn_sdot4((int)(w1.z & m), (int)xc.lo[1].z, a, false);
    b = __builtin_amdgcn_sdot4((int)((w1.z >> 4) & m), (int)xc.hi[1].z, b, false);
    a = __builtin_amdgcn_sdot4((int)(w1.w & m), (int)xc.lo[1].w, a, false);
    b = __builtin_amdgcn_sdot4((int)((w1.w >> 4) & m), (int)xc.hi[1].w, b, false);
    D0 = a;
    D1 = b;
}

// Contribution of one block to one lane's row sum: d_x * (d * I1 - dmin * I2).
__device__ __forceinline__ double block_term(const u32x4 &h, const u32x4 &w0, const u32x4 &w1, const XChunk &xc,
                                             const PairSel &ps) {
    int D0, D1;
    dot_chunk(w0, w1, xc, D0, D1);
    const uint32_t sm = scale_bytes(h, ps);
    // 24-bit multiplies suffice: scales < 64, |dot| < 2^16, |code sum| < 2^12
    const int I1 = __mul24((int)(sm & 0xFFu), D0) + __mul24((int)((sm >> 8) & 0xFFu), D1);
    const int I2 = __mul24((int)((sm >> 16) & 0xFFu), xc.bs0) + __mul24((int)(sm >> 24), xc.bs1);
    const double dd = (double)f16_bits_f32(h.x & 0xFFFFu);
    const double dm = (double)f16_bits_f32(h.x >> 16);
    const double t = __builtin_fma(-dm, (double)I2, dd * (double)I1);  // one rounding
    return t * xc.dx;
}

template <int SUB, int BPL, int R, int WPB>
__global__ __launch_bounds__(WPB * 64) void k_gemv_q4k_q8(const uint8_t *__restrict__ blocks,
                                                          const int8_t *__restrict__ q,
                                                          const float *__restrict__ dx,
                                                          const int32_t *__restrict__ bsums, float *__restrict__ y,
                                                          int64_t n, int64_t nb) {
    constexpr int NBS = 16 / SUB;     // block slots per row group
    constexpr int LPR = kWave / SUB;  // lanes per row group
    const int lane = threadIdx.x & (kWave - 1);
    const int c = lane & 3;
    const int slot = (lane >> 2) % NBS;
    const int g = (lane >> 2) / NBS;
    const int64_t wave = (int64_t)blockIdx.x * WPB + threadIdx.x / kWave;
    const int64_t row0 = wave * (R * SUB) + g;
    const int64_t row_bytes = 144 * nb;
    const PairSel ps = pair_sel(c);

    double acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0;

    // Rows past n and blocks past nb load a valid neighbour (row n-1, block
    // nb-1) instead of branching; their results are dropped below.
    for (int64_t b0 = 0; b0 < nb; b0 += NBS * BPL) {
        u32x4 h[R][BPL], w0[R][BPL], w1[R][BPL];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t row = min(row0 + (int64_t)r * SUB, n - 1);
#pragma unroll
            for (int j = 0; j < BPL; ++j) {
                const int64_t b = min(b0 + slot + NBS * j, nb - 1);
                const uint8_t *blk = blocks + row * row_bytes + 144 * b;
                w0[r][j] = ld16(blk + 16 + 32 * c);
                w1[r][j] = ld16(blk + 32 + 32 * c);
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t row = min(row0 + (int64_t)r * SUB, n - 1);
#pragma unroll
            for (int j = 0; j < BPL; ++j) {
                const int64_t b = min(b0 + slot + NBS * j, nb - 1);
                h[r][j] = ld16(blocks + row * row_bytes + 144 * b);
            }
        }
        XChunk xc[BPL];
#pragma unroll
        for (int j = 0; j < BPL; ++j) {
            const int64_t b = min(b0 + slot + NBS * j, nb - 1);
            const int8_t *xp = q + 256 * b + 64 * c;
            xc[j].lo[0] = ld16(xp);
            xc[j].lo[1] = ld16(xp + 16);
            xc[j].hi[0] = ld16(xp + 32);
            xc[j].hi[1] = ld16(xp + 48);
            const u32x2 s2 = ld8(bsums + 8 * b + 2 * c);
            xc[j].bs0 = (int32_t)s2.x;
            xc[j].bs1 = (int32_t)s2.y;
            xc[j].dx = (double)dx[b];
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int j = 0; j < BPL; ++j) {
                const double t = block_term(h[r][j], w0[r][j], w1[r][j], xc[j], ps);
                acc[r] += (b0 + slot + NBS * j < nb) ? t : 0.0;
            }
    }

#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float v = group_sum_last<LPR>((float)acc[r]);
        const int64_t row = row0 + (int64_t)r * SUB;
        if ((lane % LPR) == LPR - 1 && row < n) y[row] = v;
    }
}

// Row-loop form for rows of at most NBS * BPL blocks. The lane's activation
// codes, code sums and scales are loaded once. Wave w then owns the
// contiguous run of passes [w*q + min(w, r), ...) of length q or q + 1
// (passes = q * waves + r), walked with two register sets: the weights of
// pass i+1 are requested before pass i is computed. Every request inside the
// loop is unconditional (the one past the run re-reads its last pass), so
// each wait leaves exactly the newer requests in flight.
template <int BPL>
struct QFrag {
    u32x4 h[BPL], w0[BPL], w1[BPL];
};

// row < 2^32 (n * k < 2^40 with k >= 256) and row_bytes <= 144 * 64, so the
// row offset is one 32 x 32 -> 64-bit multiply.
template <int SUB, int BPL>
__device__ __forceinline__ void q8_load(QFrag<BPL> &f, const uint8_t *__restrict__ blocks, uint32_t row,
                                        uint32_t row_bytes, int slot, int c, int64_t nb) {
    constexpr int NBS = 16 / SUB;
    const uint8_t *base = blocks + (uint64_t)row * row_bytes;
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
        const uint8_t *blk = base + 144 * min((int64_t)(slot + NBS * j), nb - 1);
        f.w0[j] = ld16(blk + 16 + 32 * c);
        f.w1[j] = ld16(blk + 32 + 32 * c);
    }
#pragma unroll
    for (int j = 0; j < BPL; ++j) f.h[j] = ld16(base + 144 * min((int64_t)(slot + NBS * j), nb - 1));
}

template <int SUB, int BPL>
__device__ __forceinline__ float q8_pass(const QFrag<BPL> &f, const XChunk *xc, const bool *live, const PairSel &ps) {
    double acc = 0.0;
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
        const double t = block_term(f.h[j], f.w0[j], f.w1[j], xc[j], ps);
        acc += live[j] ? t : 0.0;
    }
    return group_sum_last<kWave / SUB>((float)acc);
}

// Park the row-group sums of pass i (valid in the last lane of each group) in
// lanes i*SUB .. i*SUB+SUB-1.
template <int SUB, int BPL, int WPB>
__global__ __launch_bounds__(WPB * 64) void k_gemv_q4k_q8_loop(const uint8_t *__restrict__ blocks,
                                                               const int8_t *__restrict__ q,
                                                               const float *__restrict__ dx,
                                                               const int32_t *__restrict__ bsums,
                                                               float *__restrict__ y, int64_t n, int64_t nb,
                                                               int64_t per_q, int64_t per_r) {
    constexpr int NBS = 16 / SUB;
    constexpr int LPR = kWave / SUB;
    const int lane = threadIdx.x & (kWave - 1);
    const int c = lane & 3;
    const int slot = (lane >> 2) % NBS;
    const int g = (lane >> 2) / NBS;
    const uint32_t row_bytes = 144u * (uint32_t)nb;
    const uint32_t last = (uint32_t)(n - 1);
    const int64_t w = (int64_t)blockIdx.x * WPB + threadIdx.x / kWave;
    const int64_t start = w * per_q + min(w, per_r);
    const int m = (int)(per_q + (w < per_r ? 1 : 0));
    const PairSel ps = pair_sel(c);
    auto row_of = [&](int i) -> uint32_t { return min((uint32_t)(start + i) * SUB + g, last); };

    QFrag<BPL> f0, f1;
    q8_load<SUB, BPL>(f0, blocks, row_of(0), row_bytes, slot, c, nb);
    XChunk xc[BPL];
    bool live[BPL];
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
        live[j] = slot + NBS * j < nb;
        const int64_t b = min((int64_t)(slot + NBS * j), nb - 1);
        const int8_t *xp = q + 256 * b + 64 * c;
        xc[j].lo[0] = ld16(xp);
        xc[j].lo[1] = ld16(xp + 16);
        xc[j].hi[0] = ld16(xp + 32);
        xc[j].hi[1] = ld16(xp + 48);
        const u32x2 s2 = ld8(bsums + 8 * b + 2 * c);
        xc[j].bs0 = (int32_t)s2.x;
        xc[j].bs1 = (int32_t)s2.y;
        xc[j].dx = (double)dx[b];
    }
    const bool writer = (lane % LPR) == LPR - 1;
    int i = 0;
    for (; i + 1 < m; i += 2) {
        q8_load<SUB, BPL>(f1, blocks, row_of(i + 1), row_bytes, slot, c, nb);
        __builtin_amdgcn_sched_barrier(0);
        float v = q8_pass<SUB, BPL>(f0, xc, live, ps);
        uint32_t row = (uint32_t)(start + i) * SUB + g;
        if (writer && row < n) y[row] = v;
        q8_load<SUB, BPL>(f0, blocks, row_of(min(i + 2, m - 1)), row_bytes, slot, c, nb);
        __builtin_amdgcn_sched_barrier(0);
        v = q8_pass<SUB, BPL>(f1, xc, live, ps);
        row += SUB;
        if (writer && row < n) y[row] = v;
    }
    if (i < m) {
        const float v = q8_pass<SUB, BPL>(f0, xc, live, ps);
        const uint32_t row = (uint32_t)(start + i) * SUB + g;
        if (writer && row < n) y[row] = v;
    }
}

constexpr int kQWaves = 4;

template <int SUB, int BPL, int R, int WPB>
hipError_t run_gemv_q8(const qbn_tensor &w, const int8_t *q, const float *d, const int32_t *bs, float *y,
                       hipStream_t s) {
    const int64_t nb = w.k / 256;
    const int64_t waves = (w.n + R * SUB - 1) / (R * SUB);
    const int64_t grid = (waves + WPB - 1) / WPB;
    hipLaunchKernelGGL((k_gemv_q4k_q8<SUB, BPL, R, WPB>), dim3((unsigned)grid), dim3(WPB * kWave), 0, s,
                       (const uint8_t *)w.data, q, d, bs, y, w.n, nb);
    return hipGetLastError();
}

// Grid of the row-loop kernel: at most PER_CU workgroups per compute unit,
// fewer when there are not enough passes.
template <int SUB, int BPL, int WPB, int PER_CU>
hipError_t run_gemv_q8_loop(const qbn_tensor &w, const int8_t *q, const float *d, const int32_t *bs, float *y,
                            hipStream_t s) {
    const int64_t nb = w.k / 256;
    const int64_t passes = (w.n + SUB - 1) / SUB;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    const int64_t want = (passes + WPB - 1) / WPB;
    const int64_t grid = want < (int64_t)cus * PER_CU ? want : (int64_t)cus * PER_CU;
    const int64_t waves = grid * WPB;  // waves past the last pass get an empty run
    hipLaunchKernelGGL((k_gemv_q4k_q8_loop<SUB, BPL, WPB>), dim3((unsigned)grid), dim3(WPB * kWave), 0, s,
                       (const uint8_t *)w.data, q, d, bs, y, w.n, nb, passes / waves, passes % waves);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_q8(const void *x, int x_dtype, int64_t k, int8_t *q, float *d, int32_t *bsums,
                              hipStream_t s) {
    const int64_t nb = k / 256;
    const int64_t grid = (nb + kQWaves - 1) / kQWaves;
    if (x_dtype == QBN_BF16)
        hipLaunchKernelGGL((k_quantize_q8<__bf16, kQWaves>), dim3((unsigned)grid), dim3(kQWaves * kWave), 0, s,
                           (const __bf16 *)x, q, d, bsums, nb);
    else
        hipLaunchKernelGGL((k_quantize_q8<float, kQWaves>), dim3((unsigned)grid), dim3(kQWaves * kWave), 0, s,
                           (const float *)x, q, d, bsums, nb);
    return hipGetLastError();
}

hipError_t launch_gemv_q8(const qbn_tensor &w, const int8_t *q, const float *d, const int32_t *bsums, float *y,
                          hipStream_t s) {
    const int64_t nb = w.k / 256;
    if (w.n >= ((int64_t)1 << 31)) return run_gemv_q8<1, 4, 1, 4>(w, q, d, bsums, y, s);  // 32-bit row math below
    if (nb == 1) return run_gemv_q8_loop<16, 1, 4, 3>(w, q, d, bsums, y, s);
    if (nb == 2) return run_gemv_q8_loop<8, 1, 4, 3>(w, q, d, bsums, y, s);
    if (nb <= 4) return run_gemv_q8_loop<4, 1, 4, 3>(w, q, d, bsums, y, s);
    if (nb <= 8) return run_gemv_q8_loop<2, 1, 4, 3>(w, q, d, bsums, y, s);
    if (nb <= 16) return run_gemv_q8_loop<1, 1, 4, 3>(w, q, d, bsums, y, s);
    if (nb <= 32) return run_gemv_q8_loop<1, 2, 4, 3>(w, q, d, bsums, y, s);
    if (nb <= 48) return run_gemv_q8_loop<1, 3, 4, 2>(w, q, d, bsums, y, s);
    if (nb <= 64) return run_gemv_q8_loop<1, 4, 4, 2>(w, q, d, bsums, y, s);
    return run_gemv_q8<1, 4, 1, 4>(w, q, d, bsums, y, s);  // one-shot, chunks of 64 blocks
}

}  // namespace qbn
