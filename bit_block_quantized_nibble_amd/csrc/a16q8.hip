// Integer-exact NVFP4 decode against Q8_K activations on gfx950
// ("Chapter 7 - NVFP4: the native lane", section 7.4.2).
//
// Per 256-element block the contraction is exact: each 16-element group's
// sum of e2m1 * q runs on bf16 dot instructions with binary32 accumulation,
// where every product (a 4-bit E2M1 value times an integer of at most 7
// bits) and every partial sum (a multiple of 1/2 below 2^14) is exactly
// representable, so the group sum is exact whatever the order; times the
// E4M3FN scale (exact in binary32: at most 15 + 4 significant bits); the 16
// group products of a block are added in binary64, where all of them are
// multiples of 2^-10 below 2^27, so the block total T = Q1*Q8*Q9 total *
// 2^-10 is exact and independent of the order and of the lane split.
// Only the page's epilogue rounds, in its order:
//   c = RN32(T)   (= fma(float(integer total), 2^-10, 0): scaling by 2^-10 is exact)
//   c = fma(c, d_b, 0);  c = fma(c, scale2, 0);  acc = acc + c  (blocks ascending)
// and the output is acc rounded to binary16.
#include "qbn_device.h"
#include "qbn_launch.h"

namespace qbn {
namespace {

// 64 activation codes of the lane as 32 bf16 pairs (element 2i low). An int8
// code is exact in bf16: its binary32 value has at most 7 significant bits.
struct QPairs {
    uint32_t p[32];
    float d;  // block scale 1 / iscale
};

__device__ __forceinline__ uint32_t bf16_pair_of_codes(int a, int b) {
    return (__float_as_uint((float)a) >> 16) | (__float_as_uint((float)b) & 0xFFFF0000u);
}

__device__ __forceinline__ void load_qpairs(QPairs &x, const int8_t *__restrict__ q, const float *__restrict__ d,
                                            int64_t b, int c) {
    const int8_t *p = q + 256 * b + 64 * c;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const u32x4 v = ld16(p + 16 * t);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int32_t s = (int32_t)w[i];
            x.p[8 * t + 2 * i] = bf16_pair_of_codes((s << 24) >> 24, (s << 16) >> 24);
            x.p[8 * t + 2 * i + 1] = bf16_pair_of_codes((s << 8) >> 24, s >> 24);
        }
    }
    x.d = d[b];
}

// The lane's share of one block: code bytes 32c .. 32c+31 of the block (64
// elements, groups 4c .. 4c+3) and those groups' four scale bytes.
struct AFrag {
    u32x4 w0, w1;
    uint32_t sc;
};

__device__ __forceinline__ void load_afrag(AFrag &f, const uint8_t *__restrict__ codes,
                                           const uint8_t *__restrict__ scales, uint32_t row, int64_t k, int64_t b,
                                           int c) {
    const uint8_t *cp = codes + (uint64_t)row * (uint64_t)(k / 2) + 128 * b + 32 * c;
    // the codes are read once: non-temporal (kernel 4.28 -> 4.09 us on 4096 x 4096)
    f.w0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(cp));
    f.w1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(cp + 16));
    // the four scale bytes too (kernel 4.09 -> 3.98 us; an unaligned address
    // is a legal load here)
    f.sc = __builtin_nontemporal_load(
        reinterpret_cast<const uint32_t *>(scales + (uint64_t)row * (uint64_t)(k / 16) + 16 * b + 4 * c));
}

// Exact sum over 16 elements (two code words) of e2m1 * q.
__device__ __forceinline__ float group_dot(uint32_t wa, uint32_t wb, const uint32_t *xp) {
    float g = 0.0f;
    g = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<0>(wa), as_bf16x2(xp[0]), g, false);
    g = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<1>(wa), as_bf16x2(xp[1]), g, false);
    g = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<2>(wa), as_bf16x2(xp[2]), g, false);
    g = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<3>(wa), as_bf16x2(xp[3]), g, false);
    g = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<0>(wb), as_bf16x2(xp[4]), g, false);
    g = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<1>(wb), as_bf16x2(xp[5]), g, false);
    g = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<2>(wb), as_bf16x2(xp[6]), g, false);
    g = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<3>(wb), as_bf16x2(xp[7]), g, false);
    return g;
}

// The lane's exact part of the block total, sum over its 4 groups of
// group dot * E4M3FN scale (binary64, exact).
__device__ __forceinline__ double lane_total(const AFrag &f, const QPairs &x) {
    const float p0 = group_dot(f.w0.x, f.w0.y, x.p + 0) * e4m3fn_f32_valid(f.sc & 0xFFu);
    const float p1 = group_dot(f.w0.z, f.w0.w, x.p + 8) * e4m3fn_f32_valid((f.sc >> 8) & 0xFFu);
    const float p2 = group_dot(f.w1.x, f.w1.y, x.p + 16) * e4m3fn_f32_valid((f.sc >> 16) & 0xFFu);
    const float p3 = group_dot(f.w1.z, f.w1.w, x.p + 24) * e4m3fn_f32_valid(f.sc >> 24);
    return ((double)p0 + (double)p1) + ((double)p2 + (double)p3);
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Block contribution after the pinned epilogue, in every lane of the block's
// quad: the quad sum of the exact lane totals, then RN32, * d, * scale2.
__device__ __forceinline__ float block_contribution(double t, float d, float scale2) {
    t += dpp_f64<0xB1>(t);  // quad_perm [1,0,3,2]
    t += dpp_f64<0x4E>(t);  // quad_perm [2,3,0,1]
    float c = (float)t;
    c = __builtin_fmaf(c, d, 0.0f);
    return __builtin_fmaf(c, scale2, 0.0f);
}

template <typename YT>
__device__ __forceinline__ void put_y(YT *y, uint32_t row, float acc);
template <>
__device__ __forceinline__ void put_y<float>(float *y, uint32_t row, float acc) {
    y[row] = (float)(_Float16)acc;
}
template <>
__device__ __forceinline__ void put_y<_Float16>(_Float16 *y, uint32_t row, float acc) {
    y[row] = (_Float16)acc;
}

// Rows of nb <= 16 * BPL blocks: lane (slot, c) holds blocks slot + 16 j of
// every row, j < BPL. Wave w owns a contiguous run of rows, walked with two
// register sets (the next row requested before the current one is
// computed; every request in the loop is unconditional). The ascending
// block sum of a row reads each block's contribution from lane 4 * slot.
template <int BPL>
struct ARow {
    AFrag f[BPL];
};

template <int BPL>
__device__ __forceinline__ void load_arow(ARow<BPL> &r, const uint8_t *__restrict__ codes,
                                          const uint8_t *__restrict__ scales, uint32_t row, int64_t k, int64_t nb,
                                          int slot, int c) {
#pragma unroll
    for (int j = 0; j < BPL; ++j) load_afrag(r.f[j], codes, scales, row, k, min((int64_t)(slot + 16 * j), nb - 1), c);
}

// FULL: nb == 16 * BPL, so every slot holds a real block.
template <int BPL, bool FULL = false>
__device__ __forceinline__ float row_sum(const ARow<BPL> &r, const QPairs *x, float scale2, int64_t nb) {
    float cb[BPL];
#pragma unroll
    for (int j = 0; j < BPL; ++j) cb[j] = block_contribution(lane_total(r.f[j], x[j]), x[j].d, scale2);
    // Blocks past nb add +0, which leaves acc unchanged (acc is never -0:
    // every contribution is an fma with a +0 addend).
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < BPL; ++j)
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cb[j]), 4 * s));
            acc = acc + ((FULL || 16 * j + s < nb) ? v : 0.0f);
        }
    return acc;
}

template <int BPL, int WPB, typename YT>
__global__ __launch_bounds__(WPB * 64) void k_gemv_nvfp4_a16q8(const uint8_t *__restrict__ codes,
                                                               const uint8_t *__restrict__ scales, float scale2,
                                                               const int8_t *__restrict__ q,
                                                               const float *__restrict__ d, YT *__restrict__ y,
                                                               int64_t n, int64_t k, int64_t per_q, int64_t per_r) {
    const int lane = threadIdx.x & (kWave - 1);
    const int c = lane & 3;
    const int slot = lane >> 2;
    const int64_t nb = k / 256;
    const int64_t w = (int64_t)blockIdx.x * WPB + threadIdx.x / kWave;
    const int64_t start = w * per_q + min(w, per_r);
    const int m = (int)(per_q + (w < per_r ? 1 : 0));
    const uint32_t last = (uint32_t)(n - 1);
    auto row_of = [&](int i) -> uint32_t { return min((uint32_t)(start + i), last); };

    ARow<BPL> r0, r1;
    load_arow<BPL>(r0, codes, scales, row_of(0), k, nb, slot, c);
    QPairs x[BPL];
#pragma unroll
    for (int j = 0; j < BPL; ++j) load_qpairs(x[j], q, d, min((int64_t)(slot + 16 * j), nb - 1), c);

    int i = 0;
    for (; i + 1 < m; i += 2) {
        load_arow<BPL>(r1, codes, scales, row_of(i + 1), k, nb, slot, c);
        __builtin_amdgcn_sched_barrier(0);
        float v = row_sum<BPL>(r0, x, scale2, nb);
        if (lane == 0) put_y<YT>(y, (uint32_t)(start + i), v);
        load_arow<BPL>(r0, codes, scales, row_of(min(i + 2, m - 1)), k, nb, slot, c);
        __builtin_amdgcn_sched_barrier(0);
        v = row_sum<BPL>(r1, x, scale2, nb);
        if (lane == 0) put_y<YT>(y, (uint32_t)(start + i + 1), v);
    }
    if (i < m) {
        const float v = row_sum<BPL>(r0, x, scale2, nb);
        if (lane == 0) put_y<YT>(y, (uint32_t)(start + i), v);
    }
}

// One-shot form for rows of at most 16 blocks: a wave owns R consecutive
// rows and requests all of their codes and scales before its activations
// (at these sizes this is as fast as the row loop, whose prefetch has few
// rows per wave to work with). Rows past n re-read row n-1 and are not
// stored.
template <int R, int WPB, bool FULL, typename YT>
__global__ __launch_bounds__(WPB * 64) void k_gemv_nvfp4_a16q8_rows(const uint8_t *__restrict__ codes,
                                                                    const uint8_t *__restrict__ scales, float scale2,
                                                                    const int8_t *__restrict__ q,
                                                                    const float *__restrict__ d, YT *__restrict__ y,
                                                                    int64_t n, int64_t k) {
    const int lane = threadIdx.x & (kWave - 1);
    const int c = lane & 3;
    const int slot = lane >> 2;
    const int64_t nb = k / 256;
    const int64_t row0 = ((int64_t)blockIdx.x * WPB + threadIdx.x / kWave) * R;
    if (row0 >= n) return;  // whole waves only; no barrier follows
    const int64_t b = min((int64_t)slot, nb - 1);
    ARow<1> rr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) load_arow<1>(rr[r], codes, scales, (uint32_t)min(row0 + r, n - 1), k, nb, slot, c);
    QPairs x[1];
    load_qpairs(x[0], q, d, b, c);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float v = row_sum<1, FULL>(rr[r], x, scale2, nb);
        if (lane == 0 && row0 + r < n) put_y<YT>(y, (uint32_t)(row0 + r), v);
    }
}

// Longer rows: one wave per row, chunks of 16 blocks in
// ascending order (lane (slot, c) holds block 16 * chunk + slot).
template <typename YT>
__global__ __launch_bounds__(256) void k_gemv_nvfp4_a16q8_long(const uint8_t *__restrict__ codes,
                                                               const uint8_t *__restrict__ scales, float scale2,
                                                               const int8_t *__restrict__ q,
                                                               const float *__restrict__ d, YT *__restrict__ y,
                                                               int64_t n, int64_t k) {
    const int lane = threadIdx.x & (kWave - 1);
    const int c = lane & 3;
    const int slot = lane >> 2;
    const int64_t nb = k / 256;
    const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
    if (row >= n) return;  // whole waves only; no barrier follows
    float acc = 0.0f;
    for (int64_t b0 = 0; b0 < nb; b0 += 16) {
        const int64_t b = min(b0 + slot, nb - 1);
        AFrag f;
        load_afrag(f, codes, scales, (uint32_t)row, k, b, c);
        QPairs x;
        load_qpairs(x, q, d, b, c);
        const float cb = block_contribution(lane_total(f, x), x.d, scale2);
        for (int s = 0; s < 16 && b0 + s < nb; ++s)
            acc = acc + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cb), 4 * s));
    }
    if (lane == 0) put_y<YT>(y, (uint32_t)row, acc);
}

template <int BPL, int WPB, int PER_CU, typename YT>
hipError_t run_a16q8(const qbn_tensor &w, const int8_t *q, const float *d, YT *y, hipStream_t s) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    const int64_t want = (w.n + WPB - 1) / WPB;
    const int64_t grid = want < (int64_t)cus * PER_CU ? want : (int64_t)cus * PER_CU;
    const int64_t waves = grid * WPB;
    hipLaunchKernelGGL((k_gemv_nvfp4_a16q8<BPL, WPB, YT>), dim3((unsigned)grid), dim3(WPB * kWave), 0, s,
                       (const uint8_t *)w.data, (const uint8_t *)w.scales, w.scale2, q, d, y, w.n, w.k,
                       w.n / waves, w.n % waves);
    return hipGetLastError();
}

template <int R, int WPB, bool FULL, typename YT>
hipError_t run_a16q8_rows(const qbn_tensor &w, const int8_t *q, const float *d, YT *y, hipStream_t s) {
    const int64_t waves = (w.n + R - 1) / R;
    hipLaunchKernelGGL((k_gemv_nvfp4_a16q8_rows<R, WPB, FULL, YT>), dim3((unsigned)((waves + WPB - 1) / WPB)),
                       dim3(WPB * kWave), 0, s, (const uint8_t *)w.data, (const uint8_t *)w.scales, w.scale2, q, d, y,
                       w.n, w.k);
    return hipGetLastError();
}

template <typename YT>
hipError_t launch_a16q8_typed(const qbn_tensor &w, const int8_t *q, const float *d, YT *y, hipStream_t s) {
    const int64_t nb = w.k / 256;
    if (w.n < ((int64_t)1 << 31)) {  // 32-bit row indices in the row-loop kernel
        if (nb == 16) return run_a16q8_rows<2, 8, true, YT>(w, q, d, y, s);
        if (nb < 16) return run_a16q8_rows<2, 8, false, YT>(w, q, d, y, s);
        if (nb <= 32) return run_a16q8<2, 4, 2, YT>(w, q, d, y, s);
    }
    const int64_t grid = (w.n + 3) / 4;
    hipLaunchKernelGGL((k_gemv_nvfp4_a16q8_long<YT>), dim3((unsigned)grid), dim3(256), 0, s, (const uint8_t *)w.data,
                       (const uint8_t *)w.scales, w.scale2, q, d, y, w.n, w.k);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_a16q8(const qbn_tensor &w, const int8_t *q, const float *d, void *y, int y_dtype,
                             hipStream_t s) {
    if (y_dtype == QBN_F16) return launch_a16q8_typed<_Float16>(w, q, d, (_Float16 *)y, s);
    return launch_a16q8_typed<float>(w, q, d, (float *)y, s);
}

}  // namespace qbn
