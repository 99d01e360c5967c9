/*
 * qbn.h - C ABI of the qbn library: fused dequantize-and-dot over packed
 * 4-bit block-quantized weights, bulk dequantization and bit-exact int4
 * layout repacks, for AMD Instinct MI355X (gfx950).
 *
 * Sources (page title, section):
 *  [FB] "Four Bits, Three Contracts: an interactive guide to MXFP4, NVFP4 and
 *       Q4_K" (shivasnotes.com, blog 6006)
 *  [WK] "Why 4-Bit Quantization Is King: Understanding Q4_K, MXFP4, and NVFP4"
 *       (shivasnotes.com, blog 5996)
 *  [BP] "Bit Packing Architecture" (aicassindra.com)
 *  [NV] "Chapter 7 - NVFP4: the native lane" (Muser book,
 *       highperformanceailab.com)
 *
 * Conventions shared by every call
 *  - The logical weight W is n x k: n output features (rows), k input
 *    features (the reduction dimension). W_hat is its dequantized value.
 *  - Every buffer pointer is a DEVICE pointer owned by the caller (the one
 *    exception: qbn_validate's result is a host int64); the library never
 *    frees or retains a caller's buffer.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL means the
 *    default stream). A call returns after enqueueing its kernels and
 *    allocates nothing. The one exception is qbn_validate, which waits for
 *    its scan and holds one int64 of device memory while it runs.
 *  - Every argument is checked on the host before anything is enqueued; a
 *    rejected call returns a nonzero qbn_status and enqueues nothing. A
 *    launch failure returns QBN_ERR_HIP; qbn_last_hip_error() gives the
 *    hipError_t of the calling thread's last failure.
 *  - All multi-byte fields are little-endian ([BP] "Endianness, views and
 *    padding"). Dimensions must be multiples of the format's block or pack
 *    size; callers pad and slice ([BP] same section).
 *  - The library holds no state besides the per-thread last error and is
 *    thread-safe.
 *
 * Formats (the `data` / `scales` / `zeros` buffers of a qbn_tensor)
 *  QBN_MXFP4 [FB] section 3: data u8 [n][k/2], two E2M1 codes per byte, low
 *            nibble = even element; scales u8 [n][k/32] E8M0 (2^(b-127)),
 *            groups of 32 along k. k % 32 == 0.
 *  QBN_NVFP4 [NV] sections 7.1-7.3, Figure 7.2: data u8 [n][k/2] as MXFP4;
 *            scales u8 [n][k/16] E4M3FN; scale2 = per-tensor binary32, finite
 *            and > 0. Dequantized value (e2m1 * e4m3fn) * scale2 in that
 *            order. k % 16 == 0.
 *  QBN_Q4_K  [FB] sections 5-6, [WK] section 4: data = [n][k/256] blocks of
 *            144 bytes: fp16 d (offset 0), fp16 dmin (2), 12 bytes of packed
 *            6-bit (scale, min) pairs (4), 128 code bytes (16); code byte
 *            32c+l holds output 64c+l (low nibble, sub-block 2c) and
 *            64c+32+l (high nibble, sub-block 2c+1);
 *            w = d*s_j*q - dmin*m_j. k % 256 == 0.
 *  QBN_Q4_0  [BP] "Real layouts compared": data = [n][k/32] blocks of 18
 *            bytes: fp16 d, then byte j = element j (low) | element j+16
 *            (high); w = d*(q-8). Blocks run along k inside each output row.
 *            k % 32 == 0.
 *  QBN_GPTQ4 [BP]: data int32 [k/8][n], packed along k, row 8r+j at bits 4j
 *            of word [r][n]; scales fp16 [k/group][n]; zeros u8 [k/group][n]
 *            holding LOGICAL zero points 0..15 (w = s*(q - z)).
 *            k % 8 == 0, group % 8 == 0, k % group == 0.
 *  QBN_AWQ4  [BP]: data int32 [k][n/8], packed along n, the word's slots hold
 *            columns 0,2,4,6,1,3,5,7 of its group of eight; scales and zeros
 *            as GPTQ4. n % 8 == 0, k % group == 0.
 *  QBN_NVFP4_CKE [WK] section 5 (CKE's NVFP4 storage block): data = [n][k/64]
 *            blocks of 36 bytes, 64 consecutive weights of a row each: bytes
 *            0..3 are the E4M3FN subscales of the block's four 16-weight
 *            subblocks, bytes 4+8j .. 4+8j+7 the codes of subblock j, whose
 *            byte i holds weight i (low nibble) and weight i+8 (high nibble):
 *            split-half order, not NVFP4's adjacent pairs. scales = NULL
 *            (ignored); scale2 as NVFP4; the same dequantized value
 *            (e2m1 * e4m3fn) * scale2. 4.5 bits per weight. k % 64 == 0.
 *
 * Alignment: MXFP4 / NVFP4 / Q4_K data 16-byte aligned; Q4_0 data 2-byte;
 * GPTQ4 / AWQ4 / NVFP4_CKE data 4-byte; fp16 scales 2-byte; GEMV x 16-byte and y 4-byte;
 * GEMM X 16-byte and Y 2-byte; dequantize outputs 16-byte. Scale bytes of MXFP4 / NVFP4
 * and zero points have no alignment requirement. A violation returns
 * QBN_ERR_ALIGN.
 */
#ifndef QBN_H
#define QBN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QBN_ABI_VERSION 2

/* Size, in int64 words, of the device status array of qbn_repack: word 0 is
 * the result, words 1..QBN_REPACK_SCAN_PARTS hold the refusal scan's
 * partial results. */
#define QBN_REPACK_SCAN_PARTS 64
#define QBN_REPACK_STATUS_WORDS (1 + QBN_REPACK_SCAN_PARTS)

/* Exported from libqbn.so even when built with hidden default visibility. */
#if defined(__GNUC__) || defined(__clang__)
#define QBN_API __attribute__((visibility("default")))
#else
#define QBN_API
#endif

typedef enum qbn_status {
    QBN_OK = 0,
    QBN_ERR_NULL = 1,        /* a required pointer is NULL */
    QBN_ERR_FORMAT = 2,      /* unknown format or dtype enum value */
    QBN_ERR_UNSUPPORTED = 3, /* known format, but not for this operation */
    QBN_ERR_SHAPE = 4,       /* negative size, or not a multiple of the block / pack / group size */
    QBN_ERR_ALIGN = 5,       /* a pointer or leading dimension breaks the alignment rule */
    QBN_ERR_SCALE2 = 6,      /* NVFP4 scale2 is not finite and > 0 */
    QBN_ERR_NAN_SCALE = 7,   /* qbn_validate found an invalid scale or metadata element (NaN encoding, ...) */
    QBN_ERR_DTYPE = 8,       /* unsupported activation / output dtype for this call */
    QBN_ERR_HIP = 9,         /* the HIP runtime rejected a launch or copy */
    QBN_ERR_GROUP = 10       /* group size invalid for the format or the repack */
} qbn_status;

typedef enum qbn_format {
    QBN_MXFP4 = 1,
    QBN_NVFP4 = 2,
    QBN_Q4_K = 3,
    QBN_Q4_0 = 4,
    QBN_GPTQ4 = 5,
    QBN_AWQ4 = 6,
    QBN_MXFP8 = 7, /* activations only (qbn_quantize_mx): E4M3FN elements, one E8M0 scale per 32 */
    QBN_NVFP4_CKE = 8 /* NVFP4 in 36-byte split-half blocks of 64 weights (layout above) */
} qbn_format;

typedef enum qbn_dtype {
    QBN_F32 = 0,  /* IEEE binary32 */
    QBN_BF16 = 1, /* bfloat16 (upper half of a binary32) */
    QBN_F16 = 2   /* IEEE binary16 (accepted by no call in this version) */
} qbn_dtype;

/* A quantized weight: plain sizes and caller-owned device pointers. */
typedef struct qbn_tensor {
    int32_t format;      /* qbn_format */
    int32_t group;       /* GPTQ4 / AWQ4: group length along k; otherwise ignored */
    int64_t n;           /* output features (rows of W) */
    int64_t k;           /* input features (reduction length) */
    const void *data;    /* packed codes / blocks, layout per format above */
    const void *scales;  /* MXFP4 / NVFP4 scale bytes; GPTQ4 / AWQ4 fp16 scales; else NULL */
    const void *zeros;   /* GPTQ4 / AWQ4 logical zero points u8 [k/group][n]; else NULL */
    float scale2;        /* NVFP4 per-tensor scale; ignored by other formats */
    int32_t reserved;    /* must be 0 */
} qbn_tensor;

/* Version of this ABI (QBN_ABI_VERSION) and sizeof(qbn_tensor), so that a
 * binding can check that its struct mirror matches. */
QBN_API int32_t qbn_abi_version(void);
QBN_API size_t qbn_tensor_struct_size(void);

/* Static text for a status code; never NULL. */
QBN_API const char *qbn_status_string(int32_t status);

/* hipError_t (as int) of the calling thread's last QBN_ERR_HIP, 0 if none. */
QBN_API int32_t qbn_last_hip_error(void);

/* Bytes of one part of a tensor of this format and shape:
 * part 0 = data, 1 = scales, 2 = zeros. Returns -1 for an invalid format,
 * part or shape, 0 for a part the format does not have. The per-weight
 * storage cost follows [FB] sections 3-5 and [NV] section 7.1:
 * MXFP4 17 bytes per 32 weights, NVFP4 9 per 16 (+4 per tensor for scale2,
 * not counted here), NVFP4_CKE 36 per 64, Q4_K 144 per 256, Q4_0 18 per 32. */
QBN_API int64_t qbn_bytes(int32_t format, int64_t n, int64_t k, int32_t group, int32_t part);

/* y[r] = sum_i W_hat[r][i] * x[i] for r in 0..n  (decode GEMV, batch 1).
 * Fused: W_hat is decoded in registers and never written to memory
 * ([WK] sections 1, 7 and 7d; [FB] section 8).
 * Formats: MXFP4, NVFP4 (either layout), Q4_K, and the integer int4 layouts ([BP] "Real
 * layouts compared"): Q4_0 (rows of 18-byte blocks, w = d * (q - 8)),
 * GPTQ4 and AWQ4 (the k x n logical matrix packed along k or along n,
 * w = s[k/group][r] * (q - z[k/group][r]), z the logical zero point).
 * x: QBN_F32 or QBN_BF16 [k]; y: QBN_F32 [n].
 * Accumulation is binary32 with a fixed, atomics-free reduction order, so
 * repeated calls give bit-identical y. Each y[r] satisfies
 * |y - y_exact| <= 1e-5 * sum_i |W_hat[r][i] x[i]| + 1e-6.
 * Scale bytes are not re-checked here: run qbn_validate once at load time. */
QBN_API int32_t qbn_quantized_gemv(const qbn_tensor *w, const void *x, int32_t x_dtype, void *y, int32_t y_dtype,
                           void *stream);

/* Q8_K activation quantization for the W4A8 route ([NV] section 7.4.2, the
 * activation grid; [WK] section 7, the W4A8 paragraph, and section 7c, the
 * activation sums): x [k] (QBN_F32 or QBN_BF16, finite values) is cut into
 * blocks of 256 elements; block b gets
 *   mx = its first element (lowest index) of largest magnitude, signed,
 *   iscale = RN32(-127 / mx),  d[b] = RN32(1 / iscale)     (float [k/256]),
 *   q[i] = RNE(RN32(x[i] * iscale)) clamped at 127         (int8 [k]),
 *   bsums[8b + j] = sum of the codes of elements 32j .. 32j+31 of the
 *                   block                                  (int32 [k/32]).
 * So x ~ d * q, d has the sign opposite to mx, and mx's own code is -127.
 * A block with |mx| < 2^-118 (all zeros included) gets d = 0 and codes 0.
 * k % 256 == 0 (QBN_ERR_SHAPE). Alignment: x and q 16 bytes, d 4, bsums 8.
 * Bit-exact and deterministic. */
QBN_API int32_t qbn_quantize_q8(const void *x, int32_t x_dtype, int64_t k, int8_t *q, float *d, int32_t *bsums,
                                void *stream);

/* Decode GEMV against Q8_K activations (q, d, bsums as written by
 * qbn_quantize_q8 for the same k), for r in 0..n:
 *
 * Q4_K, the W4A8 route ([WK] section 7, section 7b step 4, section 7c):
 *   y[r] = sum_i W_hat[r][i] * d[i / 256] * q[i],  y QBN_F32 [n], bsums
 *   required. W_hat is d*s_j*q - dmin*m_j taken exactly. Per sub-block the
 *   codes meet in 4 x int8 integer dots; per block the integer sums are
 *   scaled as d * sum_j s_j dot_j - dmin * sum_j m_j bsums_j in binary64
 *   (both products exact, one rounding), times d[b]; the lane sums are added
 *   in binary32 in a fixed order (repeated calls are bit-identical). Each
 *   y[r] satisfies |y - y_exact| <= 1e-5 * sum_i |W_hat[r][i] x_hat[i]| + 1e-6
 *   with x_hat = d[i / 256] * q[i].
 *
 * NVFP4, the integer-exact decode ([NV] section 7.4.2): k % 256 == 0;
 *   bsums unused (may be NULL). Per 256-block b of the row, the integer
 *   T_b = sum over its 16-groups of (sum Q1(code) * q) * Q9(scale), with
 *   Q1 = 2 * e2m1 and Q9 = 512 * e4m3fn, is formed exactly; then, blocks
 *   ascending from acc = +0, exactly these binary32 steps:
 *     c = fma(float(T_b), 2^-10, 0); c = fma(c, d[b], 0);
 *     c = fma(c, scale2, 0); acc = fma(1, c, acc);
 *   and y[r] = acc rounded to binary16 (nearest even): QBN_F16 [n] stores it,
 *   QBN_F32 [n] stores its binary32 value. The result is bit-exact and
 *   independent of the machine's reduction order.
 *
 * Alignment: q 16 bytes, d 4, bsums 8, y 4 (QBN_F32) or 2 (QBN_F16). */
QBN_API int32_t qbn_quantized_gemv_q8(const qbn_tensor *w, const int8_t *q, const float *d, const int32_t *bsums,
                                      void *y, int32_t y_dtype, void *stream);

/* Y[i][r] = sum_j X[i][j] * W_hat[r][j] for i in 0..m, r in 0..n  (prefill
 * GEMM with packed weights, [WK] sections 7 and 7d).
 * Formats: MXFP4. X: QBN_BF16 [m][ldx] row-major, ldx >= k, ldx % 8 == 0,
 * X 16-byte aligned; Y: QBN_BF16 [m][ldy], ldy >= n, Y 2-byte aligned. W_hat is expanded to bf16
 * exactly (E2M1 x 2^e is exact in bf16), products run on bf16 matrix cores
 * with binary32 accumulation, and Y is rounded to bf16 (nearest even).
 * Formats GPTQ4, AWQ4, Q4_0 ([BP] "Real layouts compared"; w = s(q - z),
 * d(q - 8)): the same X; Y QBN_BF16 or QBN_F32 ([m][ldy], 2- or 4-byte
 * aligned); k % 32 == 0 and, for GPTQ4 / AWQ4, group % 32 == 0
 * (QBN_ERR_GROUP). The codes are expanded to bf16 (q - z), exact, summed
 * against X on the bf16 matrix cores per 32-long sub-block of k, and each
 * group's sum is multiplied by its binary32 scale and added in binary32,
 * so every product is exact. Each Y entry satisfies
 * |y - y_exact| <= 1e-5 * sum_j |X[i][j] W_hat[r][j]| + 1e-6 before the bf16
 * rounding. */
QBN_API int32_t qbn_quantized_gemm(const qbn_tensor *w, int64_t m, const void *x, int32_t x_dtype, int64_t ldx, void *y,
                           int32_t y_dtype, int64_t ldy, void *stream);

/* MX activation quantization (the OCP MX contract named by [FB] section 3
 * and [WK] section 5): X [m][ldx] (QBN_F32 or QBN_BF16, finite values),
 * k % 32 == 0, ldx >= k, ldx % 4 == 0. Per 32 consecutive elements of a row:
 *   e = floor(log2 max|x|) - emax (emax 2 for E2M1, 8 for E4M3), clamped to
 *   [-127, 127] (-127 for an all-zero block); scales[i][b] = e + 127 (E8M0);
 *   each element is x * 2^-e rounded to the element grid, ties to even,
 *   magnitudes past the largest finite value saturating to it.
 * x_format QBN_MXFP4: E2M1 codes [m][k/2] (low nibble = even element),
 * codes 2-byte aligned; QBN_MXFP8: E4M3FN bytes [m][k], 4-byte aligned.
 * scales u8 [m][k/32]. x 16-byte (f32) or 8-byte (bf16) aligned. Bit-exact. */
QBN_API int32_t qbn_quantize_mx(const void *x, int32_t x_dtype, int64_t m, int64_t k, int64_t ldx, int32_t x_format,
                                void *codes, void *scales, void *stream);

/* Y[i][r] = sum_j X_hat[i][j] * W_hat[r][j]: MX-quantized activations times
 * MXFP4 weights on the gfx950 block-scaled FP4 matrix instruction
 * (v_mfma_scale_f32_32x32x64_f8f6f4), both E8M0 scales applied by the matrix
 * core ([WK] sections 5 and 7, the native FP4 path; [FB] section 3).
 * w: QBN_MXFP4 [n][k/2] + E8M0 [n][k/32]; x_format: QBN_MXFP4 (W4A4: E2M1
 * codes [m][k/2]), codes and scales [m][k/32] as written by qbn_quantize_mx,
 * codes 16-byte aligned. QBN_MXFP8 activations return QBN_ERR_UNSUPPORTED:
 * the instruction sums each run of 8 products aligned to the run's largest
 * and drops bits more than 13 below it, and E4M3 x E2M1 products exceed that
 * window, so the bound below would not hold ([WK] section 7: a W4A8 route
 * keeps the same numerical contract).
 * Y: QBN_BF16 (RNE of the binary32 sum) or QBN_F32, [m][ldy], ldy >= n.
 * Products are exact; the sum is binary32 in k-steps of 64, checked within
 * 1e-5 * sum |x_hat w_hat| + 1e-6 of the exact value (before the bf16
 * rounding). */
QBN_API int32_t qbn_quantized_gemm_mx(const qbn_tensor *w, int64_t m, int32_t x_format, const void *xcodes,
                                      const void *xscales, void *y, int32_t y_dtype, int64_t ldy, void *stream);

/* Materialize W_hat. out_layout 0: out [n][k] row-major; 1: out [k][n].
 * out_dtype QBN_F32: the exact binary32 value of each format's rule
 * (NVFP4 rounded once after the multiply by scale2, Q4_K rounded once
 * after the subtraction); QBN_BF16: that binary32 value rounded to bf16,
 * nearest even. Every weight format. Bit-exact with the definitions, including
 * negative zero; a scale byte that qbn_validate rejects decodes to NaN. */
QBN_API int32_t qbn_dequantize(const qbn_tensor *w, void *out, int32_t out_dtype, int32_t out_layout, void *stream);

/* GPTQ qzeros <-> logical zero points ([BP] "Real layouts compared";
 * "Repacking between formats", step 2). qzeros: int32 [groups][n/8], a 4-bit
 * stream along the output dimension (column 8c + j at bits 4j of word c);
 * version 1 (AutoGPTQ's pack step) stores z - 1, version 2 stores z.
 * Logical zero points: u8 [groups][n], as qbn_tensor.zeros takes them.
 * to_logical 1: src = qzeros, dst = zero points (version 1 reads a stored s
 * as s + 1, so 1..16); 0: src = zero points, dst = qzeros (version 1 stores
 * (z - 1) mod 16: zero point 0 is not representable and reads back as 16).
 * n % 8 == 0; qzeros 4-byte and zero points 8-byte aligned. Bit-exact. */
QBN_API int32_t qbn_gptq_qzeros(const void *src, void *dst, int64_t groups, int64_t n, int32_t version,
                                int32_t to_logical, void *stream);

/* GPTQ act-order resolution ([BP] "Real layouts compared": g_idx maps each
 * input row to its group; "Repacking between formats", step 3). g_idx int32
 * [k] (device). Writes perm int32 [k] (device): the source row placed at
 * each position, rows ordered by group with their original order inside a
 * group; qweight_out int32 [k/8][n] = qweight with its rows permuted alike
 * (a GPTQ4 tensor with contiguous groups: scales and zeros [k/group][n] are
 * unchanged). Apply perm to the activations with qbn_permute before the
 * GEMV. *status (device int32) receives 0, -1 (a g_idx outside
 * 0..k/group-1) or -2 (a group without exactly `group` rows); on an error
 * perm is the identity and qweight_out a plain copy. group % 8 == 0,
 * k % group == 0, k / group <= 8192; qweight_out must not alias qweight. */
QBN_API int32_t qbn_gptq_resolve_g_idx(const void *qweight, const int32_t *g_idx, int64_t k, int64_t n,
                                       int32_t group, void *qweight_out, int32_t *perm, int32_t *status,
                                       void *stream);

/* dst[i] = src[perm[i]] for i < count; dtype QBN_F32, QBN_BF16 or QBN_F16
 * (the activation permutation of an act-order layer). perm values must lie
 * in 0..count-1 (as qbn_gptq_resolve_g_idx writes them). Not in place. */
QBN_API int32_t qbn_permute(const void *src, const int32_t *perm, int64_t count, int32_t dtype, void *dst,
                            void *stream);

/* NVFP4 quantization (the encode step; [WK] section 5: x = q_E2M1 *
 * s_block(E4M3) * s_global; [NV] section 7.2: ModelOpt's ties-to-even E2M1
 * midpoints; [FB] section 2: the lowest code on a tie). X [m][ldx]
 * (QBN_F32 or QBN_BF16, finite), k % 16 == 0, scale2 finite and > 0 (the
 * caller's per-tensor scale). Per block of 16, in binary32:
 *   s = E4M3FN(amax / (6 * scale2)) (nearest, ties to even, <= 448),
 *   t = s * scale2, code = E2M1(x / t) (a t of 0 gives codes +0),
 * tie 0: ties to the even code; tie 1: ties to the lowest code; magnitudes
 * past 6 saturate. codes [m][k/2] (low nibble = even element, 8-byte
 * aligned), scales u8 [m][k/16]: a QBN_NVFP4 tensor with this scale2.
 * Bit-exact. */
QBN_API int32_t qbn_quantize_nvfp4(const void *x, int32_t x_dtype, int64_t m, int64_t k, int64_t ldx, float scale2,
                                   int32_t tie, void *codes, void *scales, void *stream);

/* Signed INT4 symmetric quantization ([WK] section 1): W [m][ldw] (QBN_F32
 * or QBN_BF16), per group of `group` (even) consecutive elements of a row,
 * s = amax / 7 (binary32; 0 for a zero group, whose codes are 0) and
 * q = clip(round_half_even(w / s), -8, 7). codes u8 [m][k/2]: two's-
 * complement nibbles, the earlier element in the low nibble; scales
 * binary32 [m][k/group]. Bit-exact. */
QBN_API int32_t qbn_quantize_int4_sym(const void *w, int32_t w_dtype, int64_t m, int64_t k, int64_t ldw,
                                      int32_t group, void *codes, float *scales, void *stream);

/* b-bit packing ([BP] "The packing arithmetic", "Odd widths"), 1 <= bits
 * <= 8, values u8 [count] (bits above `bits` ignored). lo_bits == 0: one
 * little-endian stream of 32-bit words, element i at bits [i*bits,
 * i*bits + bits) (fields straddle words when bits does not divide 32),
 * words_lo [ceil(count*bits/32)], the last word zero-padded. 0 < lo_bits <
 * bits: bit planes, the low lo_bits of each value in words_lo
 * [ceil(count*lo_bits/32)] and the high bits - lo_bits in words_hi, each a
 * stream as above (GGUF's Q6_K keeps 4 + 2). Bit-exact. */
QBN_API int32_t qbn_pack_bits(const void *values, int64_t count, int32_t bits, int32_t lo_bits, void *words_lo,
                              void *words_hi, void *stream);

/* The inverse of qbn_pack_bits: values u8 [count]. */
QBN_API int32_t qbn_unpack_bits(const void *words_lo, const void *words_hi, int64_t count, int32_t bits,
                                int32_t lo_bits, void *values, void *stream);

/* Bit-exact repack through the logical matrix ([BP] "Repacking between
 * formats"): the weight src is written into the buffers of the weight dst,
 * a complete tensor of the target format (format, group, scale2 and its
 * buffers, all checked as any input tensor) with the same n and k. The
 * buffers of dst are OUTPUTS: data always; scales / zeros as stated below.
 * Directions: GPTQ4 <-> AWQ4, GPTQ4 <-> Q4_0, AWQ4 <-> Q4_0, and
 * NVFP4 <-> NVFP4_CKE ([WK] section 5: split-half versus adjacent-pair
 * order of the same codes).
 *  - NVFP4 <-> NVFP4_CKE: k % 64 == 0. To CKE, dst->data receives the
 *    36-byte blocks; to NVFP4, dst->data the codes [n][k/2] and dst->scales
 *    the E4M3FN bytes [n][k/16]. scale2 is stored by neither layout: dst's
 *    is the caller's (checked, not written).
 *  - GPTQ4 <-> AWQ4: dst->group == src->group. dst->data receives the
 *    qweight; the scales and zeros keep their [k/group][n] layout and are
 *    copied into dst->scales / dst->zeros unless those are src's own buffers.
 *  - GPTQ4 / AWQ4 -> Q4_0: src->group % 32 == 0. dst->data receives
 *    [n][k/32] 18-byte blocks, the codes moved and d a bit copy of the group
 *    scale s[(32b)/group][n]. Q4_0 holds no zero point (it is fixed at 8),
 *    so the weights survive exactly only where every zero point is 8 ([BP]:
 *    the dequantized weights of source and target must be bit-identical).
 *  - Q4_0 -> GPTQ4 / AWQ4: dst->group % 32 == 0 and k % dst->group == 0.
 *    dst->scales (fp16 [k/group][n]) receives the d shared by the blocks of
 *    each group, dst->zeros (u8) the zero point 8; the weights survive
 *    exactly only where every block of a group has the same d.
 * Fail closed: the two Q4_0 directions first scan the source on the device.
 * status is a caller-owned DEVICE array of QBN_REPACK_STATUS_WORDS int64
 * (8-byte aligned), required for them and ignored (may be NULL) for the
 * others. status[0] receives -1 if every weight is representable, else the
 * smallest offending index (into the zero points [k/group][n] for GPTQ4 /
 * AWQ4 -> Q4_0, into the blocks [n][k/32] for Q4_0 ->), and then nothing is
 * written to dst; the other words are working space. Read status[0] after
 * the stream. No buffer of dst may overlap src's. */
QBN_API int32_t qbn_repack(const qbn_tensor *src, const qbn_tensor *dst, int64_t *status, void *stream);

/* qbn_repack for callers that cannot allocate device memory or a workspace
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same operation and argument rules, but the refusal scan's
 * QBN_REPACK_SCAN_PARTS partial results live in the library's own scratch,
 * a file-scope device array of QBN_REPACK_SCAN_PARTS int64 (512 bytes) that
 * each GPU holds until the process ends, so the caller passes only *result
 * (a DEVICE int64, 8-byte aligned; required for the Q4_0 directions, which
 * write -1 or the first offending index to it, unused by the others). The
 * scratch size does not depend on the tensor, so no size is refused for it.
 * The call allocates nothing. Calls that overlap on one GPU (other streams,
 * other threads) share that GPU's scratch and race on it: serialize them. */
QBN_API int32_t qbn_repack_noalloc(const qbn_tensor *src, const qbn_tensor *dst, int64_t *result, void *stream);

/* Load-time fail-closed scan ([NV] section 7.3: a NaN scale byte or an
 * inconsistent companion refuses the load; [FB] section 7). Synchronous: the
 * scan runs on `stream`, the call waits for it and returns QBN_OK if the
 * tensor is clean, QBN_ERR_NAN_SCALE if it is not; *first_bad (a HOST int64,
 * may be NULL) receives -1 or the smallest index of an invalid element:
 *  MXFP4: scale byte 0xFF (E8M0 NaN), index into scales;
 *  NVFP4: scale byte 0x7F or 0xFF (E4M3FN NaN), index into scales
 *         (scale2 itself is checked on the host, QBN_ERR_SCALE2);
 *  NVFP4_CKE: the same test on the subscales, index in [n][k/16] order
 *         (subscale j of block b of row r is r * (k/16) + 4b + j);
 *  Q4_K:  d or dmin not finite, index = block;
 *  Q4_0:  d not finite, or (group > 0) a block whose d differs from the
 *         first block of its group of group/32 blocks, index = block;
 *  GPTQ4 / AWQ4: scale not finite or zero point > 15, index into scales.
 * It allocates one int64 of device memory for the scan's result for the
 * duration of the call (so it cannot run under stream capture). */
QBN_API int32_t qbn_validate(const qbn_tensor *w, int64_t *first_bad, void *stream);

/* The same scan, asynchronous and allocation-free: *first_bad is a
 * caller-owned DEVICE int64 (8-byte aligned) that receives the result when
 * the stream reaches it; the call itself returns QBN_OK once enqueued. */
QBN_API int32_t qbn_validate_async(const qbn_tensor *w, int64_t *first_bad, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QBN_H */
