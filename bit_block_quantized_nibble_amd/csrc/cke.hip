// NVFP4 in CKE's split-half storage blocks ("Why 4-Bit Quantization Is
// King", section 5): 64 consecutive weights of a row in 36 bytes, the four
// E4M3FN subscales of its 16-weight subblocks first (byte j = subblock j),
// then eight code bytes per subblock; the low nibble of a subblock's byte i is
// weight i, the high nibble weight i + 8 (not the adjacent pairs of the plain
// NVFP4 layout). scale2 is a separate per-tensor operand and
// w = (e2m1 * e4m3) * scale2, as for NVFP4.
//
// A block is nine dwords: dword 0 holds the subscales, dwords 1 + 2j and
// 2 + 2j the code bytes 0-3 and 4-7 of subblock j. Byte i of a code dword
// converts (gfx950 FP4 -> bf16 / f32, exact) to the pair (w_i, w_{i+8}).
//
// Kernels: the decode GEMV, bulk dequantization, and the bit-exact repack to
// and from plain NVFP4 (codes u8 [n][k/2] with the even element in the low
// nibble, scales u8 [n][k/16]).
#include "qbn_device.h"
#include "qbn_launch.h"

namespace qbn {
namespace {

constexpr int kBlockBytes = 36;

struct Blk {
    uint32_t d[9];
};

__device__ __forceinline__ Blk load_blk(const uint8_t *p) {
    const uint32_t *q = reinterpret_cast<const uint32_t *>(p);
    Blk b;
#pragma unroll
    for (int i = 0; i < 9; ++i) b.d[i] = q[i];
    return b;
}

// 64 activations of one block, held in registers in the pair order the
// codes decode to: for bf16, dword 8j + i = (x[16j + i], x[16j + 8 + i]); for
// binary32, the 64 values in natural order.
template <typename XT>
struct XBlk;
template <>
struct XBlk<__bf16> {
    uint32_t p[32];
    __device__ __forceinline__ void load(const __bf16 *x, int64_t e0) {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(x + e0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32x4 a = src[2 * j], b = src[2 * j + 1];  // x[16j .. 16j+7], x[16j+8 .. 16j+15]
            const uint32_t lo[4] = {a.x, a.y, a.z, a.w};
            const uint32_t hi[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                // selector 0x05040100: low halves of (lo, hi); 0x07060302: high halves
                p[8 * j + 2 * q] = __builtin_amdgcn_perm(hi[q], lo[q], 0x05040100u);
                p[8 * j + 2 * q + 1] = __builtin_amdgcn_perm(hi[q], lo[q], 0x07060302u);
            }
        }
    }
    // sum over subblock j of w * x for the eight code bytes in c0 (bytes 0-3)
    // and c1 (bytes 4-7)
    __device__ __forceinline__ float dot(int j, uint32_t c0, uint32_t c1) const {
        float g = 0.0f;
        g = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<0>(c0), as_bf16x2(p[8 * j + 0]), g, false);
        g = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<1>(c0), as_bf16x2(p[8 * j + 1]), g, false);
        g = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<2>(c0), as_bf16x2(p[8 * j + 2]), g, false);
        g = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<3>(c0), as_bf16x2(p[8 * j + 3]), g, false);
        g = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<0>(c1), as_bf16x2(p[8 * j + 4]), g, false);
        g = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<1>(c1), as_bf16x2(p[8 * j + 5]), g, false);
        g = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<2>(c1), as_bf16x2(p[8 * j + 6]), g, false);
        g = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<3>(c1), as_bf16x2(p[8 * j + 7]), g, false);
        return g;
    }
};
template <>
struct XBlk<float> {
    f32x4 v[16];
    __device__ __forceinline__ void load(const float *x, int64_t e0) {
        const f32x4 *src = reinterpret_cast<const f32x4 *>(x + e0);
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = src[i];
    }
    __device__ __forceinline__ float xe(int e) const { return v[e / 4][e % 4]; }
    template <int SEL>
    __device__ __forceinline__ float pair(uint32_t c, int j, int i, float g) const {
        const f32x2 w = e2m1x2_f32<SEL>(c);
        g = __builtin_fmaf(w.x, xe(16 * j + i), g);
        return __builtin_fmaf(w.y, xe(16 * j + 8 + i), g);
    }
    __device__ __forceinline__ float dot(int j, uint32_t c0, uint32_t c1) const {
        float g = 0.0f;
        g = pair<0>(c0, j, 0, g);
        g = pair<1>(c0, j, 1, g);
        g = pair<2>(c0, j, 2, g);
        g = pair<3>(c0, j, 3, g);
        g = pair<0>(c1, j, 4, g);
        g = pair<1>(c1, j, 5, g);
        g = pair<2>(c1, j, 6, g);
        g = pair<3>(c1, j, 7, g);
        return g;
    }
};

// Block dot: each subblock sum times its subscale, accumulated in binary32
// (the scale factored out of the 16-element sums; scale2 applied once per row).
template <typename XT>
__device__ __forceinline__ float blk_dot(const Blk &b, const XBlk<XT> &xb, float acc) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
        acc = __builtin_fmaf(xb.dot(j, b.d[1 + 2 * j], b.d[2 + 2 * j]), e4m3fn_f32_valid((b.d[0] >> (8 * j)) & 0xFFu),
                             acc);
    return acc;
}

// ------------------------------------------------------------------ GEMV, multi-row
// LPR lanes per row (SUB = 64 / LPR rows side by side), lane li owns blocks
// li + LPR * j (j < BPL); a wave owns R row groups. All code blocks are
// requested first, then the activations (loaded and reordered once per lane,
// reused for every row), then the R dots.
template <typename XT, int LPR, int BPL, int R, int WPB>
__global__ __launch_bounds__(WPB * 64) void k_gemv_cke_rows(const uint8_t *__restrict__ data, float scale2,
                                                            const XT *__restrict__ x, float *__restrict__ y,
                                                            int64_t n, int64_t k) {
    constexpr int SUB = kWave / LPR;
    const int lane = threadIdx.x & (kWave - 1);
    const int sub = lane / LPR;
    const int li = lane % LPR;
    const int64_t wave = (int64_t)blockIdx.x * WPB + threadIdx.x / kWave;
    const int64_t row0 = wave * (R * SUB);
    if (row0 >= n) return;  // whole wave leaves together
    const int64_t row_bytes = (k / 64) * kBlockBytes;
    Blk b[R][BPL];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t row = row0 + r * SUB + sub;
        const int64_t rr = row < n ? row : row0;  // rows past n re-read row0 and are not stored
#pragma unroll
        for (int j = 0; j < BPL; ++j) b[r][j] = load_blk(data + rr * row_bytes + kBlockBytes * (li + (int64_t)LPR * j));
    }
    XBlk<XT> xb[BPL];
#pragma unroll
    for (int j = 0; j < BPL; ++j) xb[j].load(x, 64 * (li + (int64_t)LPR * j));
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < BPL; ++j) acc = blk_dot<XT>(b[r][j], xb[j], acc);
        acc = group_sum_last<LPR>(acc);
        const int64_t row = row0 + r * SUB + sub;
        if (li == LPR - 1 && row < n) y[row] = acc * scale2;
    }
}

// ------------------------------------------------------------------ GEMV, any k
// One wave per row; lanes stride over blocks, partial sums of up to 16
// blocks per lane added into the lane total (short binary32 chains).
template <typename XT>
__global__ __launch_bounds__(256) void k_gemv_cke_generic(const uint8_t *__restrict__ data, float scale2,
                                                          const XT *__restrict__ x, float *__restrict__ y, int64_t n,
                                                          int64_t k) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t row = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (row >= n) return;  // whole wave leaves together
    const int64_t nb = k / 64;
    const uint8_t *rp = data + row * nb * kBlockBytes;
    float acc = 0.0f;
    int64_t bi = lane;
    while (bi < nb) {
        float part = 0.0f;
        for (int t = 0; t < 16 && bi < nb; ++t, bi += kWave) {
            const Blk b = load_blk(rp + kBlockBytes * bi);
            XBlk<XT> xb;
            xb.load(x, 64 * bi);
            part = blk_dot<XT>(b, xb, part);
        }
        acc += part;
    }
    acc = group_sum_last<kWave>(acc);
    if (lane == kWave - 1) y[row] = acc * scale2;
}

template <typename XT, int LPR, int BPL, int R, int WPB>
hipError_t run_rows(const qbn_tensor &w, const XT *x, float *y, hipStream_t s) {
    constexpr int ROWS_PER_WAVE = R * (kWave / LPR);
    const int64_t waves = (w.n + ROWS_PER_WAVE - 1) / ROWS_PER_WAVE;
    const int64_t grid = (waves + WPB - 1) / WPB;
    hipLaunchKernelGGL((k_gemv_cke_rows<XT, LPR, BPL, R, WPB>), dim3((unsigned)grid), dim3(WPB * kWave), 0, s,
                       (const uint8_t *)w.data, w.scale2, x, y, w.n, w.k);
    return hipGetLastError();
}

template <typename XT>
hipError_t run_gemv(const qbn_tensor &w, const XT *x, float *y, hipStream_t s) {
    if (w.n < (int64_t)1 << 31) {
        switch (w.k / 64) {
        case 1: return run_rows<XT, 1, 1, 2, 4>(w, x, y, s);
        case 2: return run_rows<XT, 2, 1, 2, 4>(w, x, y, s);
        case 4: return run_rows<XT, 4, 1, 2, 4>(w, x, y, s);
        case 8: return run_rows<XT, 8, 1, 2, 4>(w, x, y, s);
        case 16: return run_rows<XT, 16, 1, 2, 4>(w, x, y, s);
        case 32: return run_rows<XT, 32, 1, 4, 4>(w, x, y, s);
        case 64: return run_rows<XT, 64, 1, 4, 4>(w, x, y, s);
        case 128: return run_rows<XT, 64, 2, 2, 4>(w, x, y, s);
        default: break;
        }
    }
    const int64_t grid = (w.n + 3) / 4;
    hipLaunchKernelGGL((k_gemv_cke_generic<XT>), dim3((unsigned)grid), dim3(256), 0, s, (const uint8_t *)w.data,
                       w.scale2, x, y, w.n, w.k);
    return hipGetLastError();
}

// ------------------------------------------------------------------ dequantize
// One thread per 16-weight subblock. LAYOUT 0 (out [n][k]): thread t is
// subblock t of the row-major order; LAYOUT 1 (out [k][n]): t -> (row t % n,
// subblock t / n), so consecutive lanes write consecutive rows.
template <bool BF16, int LAYOUT>
__global__ __launch_bounds__(256) void k_dequant_cke(const uint8_t *__restrict__ data, float scale2, int64_t n,
                                                     int64_t k, void *__restrict__ out) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t spr = k / 16;  // subblocks per row
    if (t >= n * spr) return;
    int64_t row, sb;
    if (LAYOUT == 0) {
        row = t / spr;
        sb = t - row * spr;
    } else {
        sb = t / n;
        row = t - sb * n;
    }
    const uint8_t *blk = data + (row * (k / 64) + sb / 4) * kBlockBytes;
    const int j = (int)(sb % 4);
    const float s = e4m3fn_f32(blk[j]);
    const uint32_t c[2] = {ld4(blk + 4 + 8 * j), ld4(blk + 8 + 8 * j)};
    float v[16];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const f32x2 p0 = e2m1x2_f32<0>(c[h]), p1 = e2m1x2_f32<1>(c[h]), p2 = e2m1x2_f32<2>(c[h]),
                    p3 = e2m1x2_f32<3>(c[h]);
        v[4 * h + 0] = p0.x; v[4 * h + 8] = p0.y;
        v[4 * h + 1] = p1.x; v[4 * h + 9] = p1.y;
        v[4 * h + 2] = p2.x; v[4 * h + 10] = p2.y;
        v[4 * h + 3] = p3.x; v[4 * h + 11] = p3.y;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float local = v[i] * s;  // exact: at most 6 significant bits
        v[i] = local * scale2;         // the single rounding
    }
    const int64_t col = 16 * sb;
    if (LAYOUT == 0) {
        const int64_t o = row * k + col;
        if (BF16) {
            uint16_t *p = (uint16_t *)out + o;
            *reinterpret_cast<u32x4 *>(p) = u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                  pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
            *reinterpret_cast<u32x4 *>(p + 8) = u32x4{pack_bf16x2(v[8], v[9]), pack_bf16x2(v[10], v[11]),
                                                      pack_bf16x2(v[12], v[13]), pack_bf16x2(v[14], v[15])};
        } else {
            f32x4 *p = reinterpret_cast<f32x4 *>((float *)out + o);
#pragma unroll
            for (int q = 0; q < 4; ++q) p[q] = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (BF16)
                ((uint16_t *)out)[(col + i) * n + row] = bf16_bits_rne(v[i]);
            else
                ((float *)out)[(col + i) * n + row] = v[i];
        }
    }
}

// ------------------------------------------------------------------ repack
// Nibble e of the 16-code subblock (e = 0..15) sits, in the plain NVFP4
// layout, at nibble e of its 8 bytes (byte e/2, low nibble for even e), and
// in the CKE layout at byte e % 8, low nibble for e < 8. Both directions
// move the codes through that index map, one thread per 64-weight block.
__device__ __forceinline__ void adjacent_to_split(uint32_t a0, uint32_t a1, uint32_t &c0, uint32_t &c1) {
    const uint64_t a = (uint64_t)a0 | ((uint64_t)a1 << 32);
    uint64_t c = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        c |= ((a >> (4 * i)) & 15u) << (8 * i);            // weight i -> byte i, low
        c |= ((a >> (4 * (i + 8))) & 15u) << (8 * i + 4);  // weight i + 8 -> byte i, high
    }
    c0 = (uint32_t)c;
    c1 = (uint32_t)(c >> 32);
}

__device__ __forceinline__ void split_to_adjacent(uint32_t c0, uint32_t c1, uint32_t &a0, uint32_t &a1) {
    const uint64_t c = (uint64_t)c0 | ((uint64_t)c1 << 32);
    uint64_t a = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a |= ((c >> (8 * i)) & 15u) << (4 * i);
        a |= ((c >> (8 * i + 4)) & 15u) << (4 * (i + 8));
    }
    a0 = (uint32_t)a;
    a1 = (uint32_t)(a >> 32);
}

// codes u8 [n][k/2] (16-byte aligned rows of k/2 bytes), scales u8 [n][k/16]
// -> CKE blocks [n][k/64][36].
__global__ __launch_bounds__(256) void k_nvfp4_to_cke(const uint8_t *__restrict__ codes,
                                                      const uint8_t *__restrict__ scales, int64_t nblocks,
                                                      uint8_t *__restrict__ out) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= nblocks) return;
    const u32x4 lo = ld16(codes + 32 * t), hi = ld16(codes + 32 * t + 16);
    const uint32_t a[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    uint32_t o[9];
    o[0] = (uint32_t)scales[4 * t] | ((uint32_t)scales[4 * t + 1] << 8) | ((uint32_t)scales[4 * t + 2] << 16) |
           ((uint32_t)scales[4 * t + 3] << 24);
#pragma unroll
    for (int j = 0; j < 4; ++j) adjacent_to_split(a[2 * j], a[2 * j + 1], o[1 + 2 * j], o[2 + 2 * j]);
    uint32_t *dst = reinterpret_cast<uint32_t *>(out + kBlockBytes * t);
#pragma unroll
    for (int i = 0; i < 9; ++i) dst[i] = o[i];
}

__global__ __launch_bounds__(256) void k_cke_to_nvfp4(const uint8_t *__restrict__ blocks, int64_t nblocks,
                                                      uint8_t *__restrict__ codes, uint8_t *__restrict__ scales) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= nblocks) return;
    const Blk b = load_blk(blocks + kBlockBytes * t);
    uint32_t a[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) split_to_adjacent(b.d[1 + 2 * j], b.d[2 + 2 * j], a[2 * j], a[2 * j + 1]);
    *reinterpret_cast<u32x4 *>(codes + 32 * t) = u32x4{a[0], a[1], a[2], a[3]};
    *reinterpret_cast<u32x4 *>(codes + 32 * t + 16) = u32x4{a[4], a[5], a[6], a[7]};
#pragma unroll
    for (int j = 0; j < 4; ++j) scales[4 * t + j] = (uint8_t)(b.d[0] >> (8 * j));
}

template <typename K, typename... A>
hipError_t launch1d(K kern, int64_t threads, hipStream_t s, A... args) {
    if (threads <= 0) return hipSuccess;
    hipLaunchKernelGGL(kern, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, args...);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_cke(const qbn_tensor &w, const void *x, int x_dtype, float *y, hipStream_t s) {
    return x_dtype == QBN_BF16 ? run_gemv<__bf16>(w, (const __bf16 *)x, y, s)
                               : run_gemv<float>(w, (const float *)x, y, s);
}

hipError_t launch_dequant_cke(const qbn_tensor &w, void *out, int out_dtype, int out_layout, hipStream_t s) {
    const int64_t threads = w.n * (w.k / 16);
    const uint8_t *d = (const uint8_t *)w.data;
    const bool bf = out_dtype == QBN_BF16;
    if (out_layout == 0)
        return bf ? launch1d(k_dequant_cke<true, 0>, threads, s, d, w.scale2, w.n, w.k, out)
                  : launch1d(k_dequant_cke<false, 0>, threads, s, d, w.scale2, w.n, w.k, out);
    return bf ? launch1d(k_dequant_cke<true, 1>, threads, s, d, w.scale2, w.n, w.k, out)
              : launch1d(k_dequant_cke<false, 1>, threads, s, d, w.scale2, w.n, w.k, out);
}

hipError_t launch_repack_cke(const qbn_tensor &src, void *dst_data, void *dst_scales, hipStream_t s) {
    const int64_t nblocks = src.n * (src.k / 64);
    if (src.format == QBN_NVFP4)
        return launch1d(k_nvfp4_to_cke, nblocks, s, (const uint8_t *)src.data, (const uint8_t *)src.scales, nblocks,
                        (uint8_t *)dst_data);
    return launch1d(k_cke_to_nvfp4, nblocks, s, (const uint8_t *)src.data, nblocks, (uint8_t *)dst_data,
                    (uint8_t *)dst_scales);
}

}  // namespace qbn
