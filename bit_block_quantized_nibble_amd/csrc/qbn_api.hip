// C-ABI entry points of libqbn: host-side argument checks, then dispatch to
// the kernel launchers. Every check runs before anything is enqueued, so a
// rejected call leaves the stream untouched ("Four Bits, Three Contracts",
// sections 7 and 10: explicit rejection of unsupported cases; "Bit Packing
// Architecture", 'Endianness, views and padding': dimensions must be
// multiples of the pack and group sizes).
#include <math.h>
#include <stdint.h>

#include "qbn_launch.h"

namespace {

thread_local int32_t g_last_hip_error = 0;

// Largest element count a launch grid here can cover (256-thread blocks,
// 32-bit grid dimension), with a wide margin.
constexpr int64_t kMaxElems = (int64_t)1 << 40;

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

int32_t hip_status(hipError_t e) {
    if (e == hipSuccess) return QBN_OK;
    g_last_hip_error = (int32_t)e;
    return QBN_ERR_HIP;
}

// Weight formats a qbn_tensor may carry (QBN_MXFP8 is an activation format only).
bool known_format(int32_t f) { return (f >= QBN_MXFP4 && f <= QBN_AWQ4) || f == QBN_NVFP4_CKE; }

// Shape, group and pointer rules of a tensor; `need_buffers` is false only
// when the tensor is empty.
int32_t check_tensor(const qbn_tensor *w) {
    if (!w) return QBN_ERR_NULL;
    if (!known_format(w->format)) return QBN_ERR_FORMAT;
    if (w->reserved != 0) return QBN_ERR_FORMAT;
    if (w->n < 0 || w->k < 0) return QBN_ERR_SHAPE;
    if (w->n > kMaxElems || w->k > kMaxElems || (w->n > 0 && w->k > kMaxElems / w->n)) return QBN_ERR_SHAPE;
    switch (w->format) {
    case QBN_MXFP4:
        if (w->k % 32) return QBN_ERR_SHAPE;
        break;
    case QBN_NVFP4:
        if (w->k % 16) return QBN_ERR_SHAPE;
        if (!(isfinite(w->scale2) && w->scale2 > 0.0f)) return QBN_ERR_SCALE2;
        break;
    case QBN_NVFP4_CKE:
        if (w->k % 64) return QBN_ERR_SHAPE;
        if (!(isfinite(w->scale2) && w->scale2 > 0.0f)) return QBN_ERR_SCALE2;
        break;
    case QBN_Q4_K:
        if (w->k % 256) return QBN_ERR_SHAPE;
        break;
    case QBN_Q4_0:
        if (w->k % 32) return QBN_ERR_SHAPE;
        break;
    case QBN_GPTQ4:
    case QBN_AWQ4:
        if (w->group <= 0 || w->group % 8) return QBN_ERR_GROUP;
        if (w->k % 8 || w->k % w->group) return QBN_ERR_SHAPE;
        if (w->format == QBN_AWQ4 && w->n % 8) return QBN_ERR_SHAPE;
        break;
    }
    const bool empty = (w->n == 0 || w->k == 0);
    if (empty) return QBN_OK;
    if (!w->data) return QBN_ERR_NULL;
    switch (w->format) {
    case QBN_MXFP4:
    case QBN_NVFP4:
        if (!w->scales) return QBN_ERR_NULL;
        if (!aligned(w->data, 16)) return QBN_ERR_ALIGN;
        break;
    case QBN_Q4_K:
        if (!aligned(w->data, 16)) return QBN_ERR_ALIGN;
        break;
    case QBN_Q4_0:
        if (!aligned(w->data, 2)) return QBN_ERR_ALIGN;
        break;
    case QBN_NVFP4_CKE:
        if (!aligned(w->data, 4)) return QBN_ERR_ALIGN;
        break;
    case QBN_GPTQ4:
    case QBN_AWQ4:
        if (!w->scales || !w->zeros) return QBN_ERR_NULL;
        if (!aligned(w->data, 4) || !aligned(w->scales, 2)) return QBN_ERR_ALIGN;
        break;
    }
    return QBN_OK;
}

// Argument rules of the validation scan. For Q4_0, `group` selects the
// uniformity check (blocks of a group share d) and is not a tensor property.
int32_t check_validate(const qbn_tensor *w) {
    if (!w) return QBN_ERR_NULL;
    if (w->format == QBN_Q4_0 && w->group != 0) {
        if (w->group < 0 || w->group % 32) return QBN_ERR_GROUP;
        if (w->k % w->group) return QBN_ERR_SHAPE;
    }
    if (w->format == QBN_Q4_0) {
        qbn_tensor t = *w;
        t.group = 0;
        return check_tensor(&t);
    }
    return check_tensor(w);
}

// Argument rules of a repack of src into the tensor dst (both complete
// tensors of their formats, same n and k); *q4_0_dir tells whether the
// direction can refuse (GPTQ4 / AWQ4 <-> Q4_0).
int32_t check_repack(const qbn_tensor *src, const qbn_tensor *dst, bool *q4_0_dir) {
    int32_t st = check_tensor(src);
    if (st) return st;
    if (!dst) return QBN_ERR_NULL;
    if (!known_format(dst->format) || dst->reserved != 0) return QBN_ERR_FORMAT;
    const int32_t sf = src->format, df = dst->format;
    // NVFP4 <-> CKE split-half blocks: the codes and subscale bytes move, scale2 is unchanged
    const bool nv_src = sf == QBN_NVFP4 || sf == QBN_NVFP4_CKE;
    const bool nv_dst = df == QBN_NVFP4 || df == QBN_NVFP4_CKE;
    const bool src_int4 = sf == QBN_GPTQ4 || sf == QBN_AWQ4 || sf == QBN_Q4_0;
    const bool dst_int4 = df == QBN_GPTQ4 || df == QBN_AWQ4 || df == QBN_Q4_0;
    if (!((nv_src && nv_dst) || (src_int4 && dst_int4)) || sf == df) return QBN_ERR_UNSUPPORTED;
    if (dst->n != src->n || dst->k != src->k) return QBN_ERR_SHAPE;
    if (df == QBN_Q4_0 && src->group % 32) return QBN_ERR_GROUP;  // Q4_0 blocks of 32 need whole groups
    if (sf == QBN_Q4_0 && (dst->group <= 0 || dst->group % 32)) return QBN_ERR_GROUP;
    if (sf != QBN_Q4_0 && df != QBN_Q4_0 && !nv_src && dst->group != src->group) return QBN_ERR_GROUP;
    if (nv_src && src->k % 64) return QBN_ERR_SHAPE;
    st = check_tensor(dst);
    if (st) return st;
    *q4_0_dir = sf == QBN_Q4_0 || df == QBN_Q4_0;
    return QBN_OK;
}

}  // namespace

extern "C" {

int32_t qbn_abi_version(void) { return QBN_ABI_VERSION; }

size_t qbn_tensor_struct_size(void) { return sizeof(qbn_tensor); }

int32_t qbn_last_hip_error(void) { return g_last_hip_error; }

const char *qbn_status_string(int32_t status) {
    switch (status) {
    case QBN_OK: return "ok";
    case QBN_ERR_NULL: return "a required pointer is NULL";
    case QBN_ERR_FORMAT: return "unknown format or enum value";
    case QBN_ERR_UNSUPPORTED: return "format not supported by this operation";
    case QBN_ERR_SHAPE: return "shape is negative, too large, or not a multiple of the block/pack/group size";
    case QBN_ERR_ALIGN: return "pointer or leading dimension is not aligned as required";
    case QBN_ERR_SCALE2: return "NVFP4 scale2 must be finite and > 0";
    case QBN_ERR_NAN_SCALE: return "validation found an invalid scale or metadata element (a NaN encoding, a non-finite fp16, a zero point above 15 or a Q4_0 group whose blocks disagree)";
    case QBN_ERR_DTYPE: return "unsupported activation or output dtype";
    case QBN_ERR_HIP: return "HIP runtime error (see qbn_last_hip_error)";
    case QBN_ERR_GROUP: return "invalid group size";
    default: return "unknown status";
    }
}

int64_t qbn_bytes(int32_t format, int64_t n, int64_t k, int32_t group, int32_t part) {
    if (!known_format(format) || part < 0 || part > 2 || n < 0 || k < 0) return -1;
    if (n > kMaxElems || k > kMaxElems || (n > 0 && k > kMaxElems / n)) return -1;
    switch (format) {
    case QBN_MXFP4:
        if (k % 32) return -1;
        return part == 0 ? n * k / 2 : part == 1 ? n * (k / 32) : 0;
    case QBN_NVFP4:
        if (k % 16) return -1;
        return part == 0 ? n * k / 2 : part == 1 ? n * (k / 16) : 0;
    case QBN_Q4_K:
        if (k % 256) return -1;
        return part == 0 ? n * (k / 256) * 144 : 0;
    case QBN_Q4_0:
        if (k % 32) return -1;
        return part == 0 ? n * (k / 32) * 18 : 0;
    case QBN_NVFP4_CKE:
        if (k % 64) return -1;
        return part == 0 ? n * (k / 64) * 36 : 0;
    case QBN_GPTQ4:
    case QBN_AWQ4:
        if (group <= 0 || group % 8 || k % 8 || k % group) return -1;
        if (format == QBN_AWQ4 && n % 8) return -1;
        return part == 0 ? n * k / 2 : part == 1 ? 2 * n * (k / group) : n * (k / group);
    }
    return -1;
}

int32_t qbn_quantized_gemv(const qbn_tensor *w, const void *x, int32_t x_dtype, void *y, int32_t y_dtype,
                           void *stream) {
    int32_t st = check_tensor(w);
    if (st) return st;
    if (x_dtype < QBN_F32 || x_dtype > QBN_F16 || y_dtype < QBN_F32 || y_dtype > QBN_F16) return QBN_ERR_FORMAT;
    if ((x_dtype != QBN_F32 && x_dtype != QBN_BF16) || y_dtype != QBN_F32) return QBN_ERR_DTYPE;
    if (w->n == 0) return QBN_OK;
    if (!y) return QBN_ERR_NULL;
    if (!aligned(y, 4)) return QBN_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    if (w->k == 0) return hip_status(qbn::launch_fill_zero(y, 4 * w->n, s));
    if (!x) return QBN_ERR_NULL;
    if (!aligned(x, 16)) return QBN_ERR_ALIGN;
    const bool int4 = w->format == QBN_Q4_0 || w->format == QBN_GPTQ4 || w->format == QBN_AWQ4;
    if (w->format == QBN_NVFP4_CKE) return hip_status(qbn::launch_gemv_cke(*w, x, x_dtype, (float *)y, s));
    return hip_status(int4 ? qbn::launch_gemv_int4(*w, x, x_dtype, (float *)y, s)
                           : qbn::launch_gemv(*w, x, x_dtype, (float *)y, s));
}

int32_t qbn_quantize_q8(const void *x, int32_t x_dtype, int64_t k, int8_t *q, float *d, int32_t *bsums,
                        void *stream) {
    if (x_dtype < QBN_F32 || x_dtype > QBN_F16) return QBN_ERR_FORMAT;
    if (x_dtype != QBN_F32 && x_dtype != QBN_BF16) return QBN_ERR_DTYPE;
    if (k < 0 || k > kMaxElems || k % 256) return QBN_ERR_SHAPE;
    if (k == 0) return QBN_OK;
    if (!x || !q || !d || !bsums) return QBN_ERR_NULL;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(d, 4) || !aligned(bsums, 8)) return QBN_ERR_ALIGN;
    return hip_status(qbn::launch_quantize_q8(x, x_dtype, k, q, d, bsums, (hipStream_t)stream));
}

int32_t qbn_quantized_gemv_q8(const qbn_tensor *w, const int8_t *q, const float *d, const int32_t *bsums, void *y,
                              int32_t y_dtype, void *stream) {
    int32_t st = check_tensor(w);
    if (st) return st;
    const bool q4k = w->format == QBN_Q4_K;
    if (!q4k && w->format != QBN_NVFP4) return QBN_ERR_UNSUPPORTED;
    if (!q4k && w->k % 256) return QBN_ERR_SHAPE;  // one activation scale per 256
    if (y_dtype < QBN_F32 || y_dtype > QBN_F16) return QBN_ERR_FORMAT;
    if (y_dtype == QBN_BF16 || (q4k && y_dtype != QBN_F32)) return QBN_ERR_DTYPE;
    if (w->n == 0) return QBN_OK;
    if (!y) return QBN_ERR_NULL;
    const int64_t ysize = y_dtype == QBN_F16 ? 2 : 4;
    if (!aligned(y, (uintptr_t)ysize)) return QBN_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    if (w->k == 0) return hip_status(qbn::launch_fill_zero(y, ysize * w->n, s));
    if (!q || !d || (q4k && !bsums)) return QBN_ERR_NULL;
    if (!aligned(q, 16) || !aligned(d, 4) || (q4k && !aligned(bsums, 8))) return QBN_ERR_ALIGN;
    if (!q4k) return hip_status(qbn::launch_gemv_a16q8(*w, q, d, y, y_dtype, s));
    return hip_status(qbn::launch_gemv_q8(*w, q, d, bsums, (float *)y, s));
}

int32_t qbn_quantize_mx(const void *x, int32_t x_dtype, int64_t m, int64_t k, int64_t ldx, int32_t x_format,
                        void *codes, void *scales, void *stream) {
    if (x_format != QBN_MXFP4 && x_format != QBN_MXFP8) return x_format >= QBN_MXFP4 && x_format <= QBN_AWQ4
                                                                   ? QBN_ERR_UNSUPPORTED
                                                                   : QBN_ERR_FORMAT;
    if (x_dtype < QBN_F32 || x_dtype > QBN_F16) return QBN_ERR_FORMAT;
    if (x_dtype != QBN_F32 && x_dtype != QBN_BF16) return QBN_ERR_DTYPE;
    if (m < 0 || k < 0 || k % 32 || m > kMaxElems || k > kMaxElems || (m > 0 && k > kMaxElems / m))
        return QBN_ERR_SHAPE;
    if (m == 0 || k == 0) return QBN_OK;
    if (ldx < k || ldx > kMaxElems / m) return QBN_ERR_SHAPE;
    if (!x || !codes || !scales) return QBN_ERR_NULL;
    if (ldx % 4 || !aligned(x, x_dtype == QBN_F32 ? 16 : 8)) return QBN_ERR_ALIGN;
    if (!aligned(codes, x_format == QBN_MXFP8 ? 4 : 2)) return QBN_ERR_ALIGN;
    return hip_status(qbn::launch_quantize_mx(x, x_dtype, m, k, ldx, x_format, codes, scales, (hipStream_t)stream));
}

int32_t qbn_quantized_gemm_mx(const qbn_tensor *w, int64_t m, int32_t x_format, const void *xcodes,
                              const void *xscales, void *y, int32_t y_dtype, int64_t ldy, void *stream) {
    int32_t st = check_tensor(w);
    if (st) return st;
    if (w->format != QBN_MXFP4) return QBN_ERR_UNSUPPORTED;
    // MXFP8 activations are not taken: the FP8 x FP4 matrix instruction drops
    // product bits more than 13 below each run's largest, past the tolerance
    if (x_format != QBN_MXFP4)
        return (known_format(x_format) || x_format == QBN_MXFP8) ? QBN_ERR_UNSUPPORTED : QBN_ERR_FORMAT;
    if (y_dtype < QBN_F32 || y_dtype > QBN_F16) return QBN_ERR_FORMAT;
    if (y_dtype != QBN_F32 && y_dtype != QBN_BF16) return QBN_ERR_DTYPE;
    if (m < 0 || m > kMaxElems) return QBN_ERR_SHAPE;
    if (m == 0 || w->n == 0) return QBN_OK;
    if (ldy < w->n || ldy > kMaxElems / m) return QBN_ERR_SHAPE;
    if (!y) return QBN_ERR_NULL;
    const int ysz = y_dtype == QBN_F32 ? 4 : 2;
    if (!aligned(y, (uintptr_t)ysz)) return QBN_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    if (w->k == 0)
        return hip_status(ysz == 2 ? qbn::launch_fill_zero_2d_u16(y, m, w->n, ldy, s)
                                   : qbn::launch_fill_zero_2d_u16(y, m, 2 * w->n, 2 * ldy, s));
    if (m > kMaxElems / w->k) return QBN_ERR_SHAPE;
    if (!xcodes || !xscales) return QBN_ERR_NULL;
    if (!aligned(xcodes, 16)) return QBN_ERR_ALIGN;
    return hip_status(qbn::launch_gemm_mx(*w, m, xcodes, xscales, y, y_dtype, ldy, s));
}

int32_t qbn_quantized_gemm(const qbn_tensor *w, int64_t m, const void *x, int32_t x_dtype, int64_t ldx, void *y,
                           int32_t y_dtype, int64_t ldy, void *stream) {
    int32_t st = check_tensor(w);
    if (st) return st;
    const bool int4 = w->format == QBN_GPTQ4 || w->format == QBN_AWQ4 || w->format == QBN_Q4_0;
    if (w->format != QBN_MXFP4 && !int4) return QBN_ERR_UNSUPPORTED;
    if (x_dtype < QBN_F32 || x_dtype > QBN_F16 || y_dtype < QBN_F32 || y_dtype > QBN_F16) return QBN_ERR_FORMAT;
    if (x_dtype != QBN_BF16 || (y_dtype != QBN_BF16 && !(int4 && y_dtype == QBN_F32))) return QBN_ERR_DTYPE;
    if (int4 && w->format != QBN_Q4_0 && w->group % 32) return QBN_ERR_GROUP;  // scales per 32-k sub-block
    if (int4 && w->k % 32) return QBN_ERR_SHAPE;
    if (m < 0 || m > kMaxElems) return QBN_ERR_SHAPE;
    if (m == 0 || w->n == 0) return QBN_OK;
    if (ldy < w->n) return QBN_ERR_SHAPE;
    if (ldy > kMaxElems / m) return QBN_ERR_SHAPE;
    if (int4 && !qbn::gemm_int4_grid_fits(m, w->n)) return QBN_ERR_SHAPE;
    if (!y) return QBN_ERR_NULL;
    const int ysz = y_dtype == QBN_F32 ? 4 : 2;
    if (!aligned(y, (uintptr_t)ysz)) return QBN_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    if (w->k == 0)
        return hip_status(ysz == 2 ? qbn::launch_fill_zero_2d_u16(y, m, w->n, ldy, s)
                                   : qbn::launch_fill_zero_2d_u16(y, m, 2 * w->n, 2 * ldy, s));
    if (ldx < w->k || ldx % 8) return ldx < w->k ? QBN_ERR_SHAPE : QBN_ERR_ALIGN;
    if (ldx > kMaxElems / m) return QBN_ERR_SHAPE;
    if (!x) return QBN_ERR_NULL;
    if (!aligned(x, 16)) return QBN_ERR_ALIGN;
    if (int4) return hip_status(qbn::launch_gemm_int4(*w, m, x, ldx, y, y_dtype, ldy, s));
    return hip_status(qbn::launch_gemm(*w, m, x, ldx, y, ldy, s));
}

int32_t qbn_dequantize(const qbn_tensor *w, void *out, int32_t out_dtype, int32_t out_layout, void *stream) {
    int32_t st = check_tensor(w);
    if (st) return st;
    if (out_dtype < QBN_F32 || out_dtype > QBN_F16 || out_layout < 0 || out_layout > 1) return QBN_ERR_FORMAT;
    if (out_dtype != QBN_F32 && out_dtype != QBN_BF16) return QBN_ERR_DTYPE;
    if (w->n == 0 || w->k == 0) return QBN_OK;
    if (!out) return QBN_ERR_NULL;
    if (!aligned(out, 16)) return QBN_ERR_ALIGN;
    if (w->format == QBN_NVFP4_CKE)
        return hip_status(qbn::launch_dequant_cke(*w, out, out_dtype, out_layout, (hipStream_t)stream));
    return hip_status(qbn::launch_dequant(*w, out, out_dtype, out_layout, (hipStream_t)stream));
}

int32_t qbn_gptq_qzeros(const void *src, void *dst, int64_t groups, int64_t n, int32_t version, int32_t to_logical,
                        void *stream) {
    if (version != 1 && version != 2) return QBN_ERR_FORMAT;
    if (to_logical != 0 && to_logical != 1) return QBN_ERR_FORMAT;
    if (groups < 0 || n < 0 || groups > kMaxElems || n > kMaxElems || (n > 0 && groups > kMaxElems / n) || n % 8)
        return QBN_ERR_SHAPE;
    if (groups == 0 || n == 0) return QBN_OK;
    if (!src || !dst) return QBN_ERR_NULL;
    const void *packed = to_logical ? src : dst, *logical = to_logical ? dst : src;
    if (!aligned(packed, 4) || !aligned(logical, 8)) return QBN_ERR_ALIGN;
    return hip_status(qbn::launch_gptq_qzeros(src, dst, groups, n, version, to_logical, (hipStream_t)stream));
}

int32_t qbn_gptq_resolve_g_idx(const void *qweight, const int32_t *g_idx, int64_t k, int64_t n, int32_t group,
                               void *qweight_out, int32_t *perm, int32_t *status, void *stream) {
    if (k < 0 || n < 0 || k > kMaxElems || n > kMaxElems || (n > 0 && k > kMaxElems / n)) return QBN_ERR_SHAPE;
    if (group <= 0 || group % 8) return QBN_ERR_GROUP;
    if (k % 8 || k % group) return QBN_ERR_SHAPE;
    if (!qbn::gptq_groups_fit(k, group)) return QBN_ERR_SHAPE;
    if (!g_idx || !perm || !status || (k > 0 && n > 0 && (!qweight || !qweight_out))) return QBN_ERR_NULL;
    if (!aligned(g_idx, 4) || !aligned(perm, 4) || !aligned(status, 4)) return QBN_ERR_ALIGN;
    if (n > 0 && k > 0 && (!aligned(qweight, 4) || !aligned(qweight_out, 4))) return QBN_ERR_ALIGN;
    if (qweight_out == qweight && n > 0 && k > 0) return QBN_ERR_UNSUPPORTED;  // rows move: not in place
    return hip_status(qbn::launch_gptq_resolve_g_idx(qweight, g_idx, k, n, group, qweight_out, perm, status,
                                                     (hipStream_t)stream));
}

int32_t qbn_permute(const void *src, const int32_t *perm, int64_t count, int32_t dtype, void *dst, void *stream) {
    if (dtype < QBN_F32 || dtype > QBN_F16) return QBN_ERR_FORMAT;
    if (count < 0 || count > kMaxElems) return QBN_ERR_SHAPE;
    if (count == 0) return QBN_OK;
    if (!src || !perm || !dst) return QBN_ERR_NULL;
    const int eb = dtype == QBN_F32 ? 4 : 2;
    if (!aligned(src, (uintptr_t)eb) || !aligned(dst, (uintptr_t)eb) || !aligned(perm, 4)) return QBN_ERR_ALIGN;
    if (src == dst) return QBN_ERR_UNSUPPORTED;
    return hip_status(qbn::launch_permute(src, perm, count, eb, dst, (hipStream_t)stream));
}

int32_t qbn_quantize_nvfp4(const void *x, int32_t x_dtype, int64_t m, int64_t k, int64_t ldx, float scale2,
                           int32_t tie, void *codes, void *scales, void *stream) {
    if (x_dtype < QBN_F32 || x_dtype > QBN_F16 || (tie != 0 && tie != 1)) return QBN_ERR_FORMAT;
    if (x_dtype == QBN_F16) return QBN_ERR_DTYPE;
    if (!(isfinite(scale2) && scale2 > 0.0f)) return QBN_ERR_SCALE2;
    if (m < 0 || k < 0 || k % 16 || m > kMaxElems || k > kMaxElems || (m > 0 && k > kMaxElems / m)) return QBN_ERR_SHAPE;
    if (m == 0 || k == 0) return QBN_OK;
    if (ldx < k || ldx > kMaxElems / m) return QBN_ERR_SHAPE;
    if (!x || !codes || !scales) return QBN_ERR_NULL;
    if (!aligned(x, x_dtype == QBN_F32 ? 4 : 2) || !aligned(codes, 8)) return QBN_ERR_ALIGN;
    return hip_status(qbn::launch_quantize_nvfp4(x, x_dtype, m, k, ldx, scale2, tie, codes, scales,
                                                 (hipStream_t)stream));
}

int32_t qbn_quantize_int4_sym(const void *w, int32_t w_dtype, int64_t m, int64_t k, int64_t ldw, int32_t group,
                              void *codes, float *scales, void *stream) {
    if (w_dtype < QBN_F32 || w_dtype > QBN_F16) return QBN_ERR_FORMAT;
    if (w_dtype == QBN_F16) return QBN_ERR_DTYPE;
    if (group <= 0 || group % 2) return QBN_ERR_GROUP;
    if (m < 0 || k < 0 || k % group || m > kMaxElems || k > kMaxElems || (m > 0 && k > kMaxElems / m))
        return QBN_ERR_SHAPE;
    if (m == 0 || k == 0) return QBN_OK;
    if (ldw < k || ldw > kMaxElems / m) return QBN_ERR_SHAPE;
    if (!w || !codes || !scales) return QBN_ERR_NULL;
    if (!aligned(w, w_dtype == QBN_F32 ? 4 : 2) || !aligned(scales, 4)) return QBN_ERR_ALIGN;
    return hip_status(qbn::launch_quantize_int4_sym(w, w_dtype, m, k, ldw, group, codes, scales, (hipStream_t)stream));
}

int32_t qbn_pack_bits(const void *values, int64_t count, int32_t bits, int32_t lo_bits, void *words_lo,
                      void *words_hi, void *stream) {
    if (bits < 1 || bits > 8 || lo_bits < 0 || lo_bits >= bits) return QBN_ERR_FORMAT;
    if (count < 0 || count > kMaxElems) return QBN_ERR_SHAPE;
    if (count == 0) return QBN_OK;
    if (!values || !words_lo || (lo_bits > 0 && !words_hi)) return QBN_ERR_NULL;
    if (!aligned(words_lo, 4) || (lo_bits > 0 && !aligned(words_hi, 4))) return QBN_ERR_ALIGN;
    return hip_status(qbn::launch_pack_bits(values, count, bits, lo_bits, words_lo, words_hi, (hipStream_t)stream));
}

int32_t qbn_unpack_bits(const void *words_lo, const void *words_hi, int64_t count, int32_t bits, int32_t lo_bits,
                        void *values, void *stream) {
    if (bits < 1 || bits > 8 || lo_bits < 0 || lo_bits >= bits) return QBN_ERR_FORMAT;
    if (count < 0 || count > kMaxElems) return QBN_ERR_SHAPE;
    if (count == 0) return QBN_OK;
    if (!values || !words_lo || (lo_bits > 0 && !words_hi)) return QBN_ERR_NULL;
    if (!aligned(words_lo, 4) || (lo_bits > 0 && !aligned(words_hi, 4))) return QBN_ERR_ALIGN;
    return hip_status(qbn::launch_unpack_bits(words_lo, words_hi, count, bits, lo_bits, values, (hipStream_t)stream));
}

int32_t qbn_repack(const qbn_tensor *src, const qbn_tensor *dst, int64_t *status, void *stream) {
    bool q4_0_dir = false;
    int32_t st = check_repack(src, dst, &q4_0_dir);
    if (st) return st;
    if (q4_0_dir) {  // these directions can refuse, and report it in status[0]
        if (!status) return QBN_ERR_NULL;
        if (!aligned(status, 8)) return QBN_ERR_ALIGN;
    }
    hipStream_t s = (hipStream_t)stream;
    if (src->n == 0 || src->k == 0) return q4_0_dir ? hip_status(qbn::launch_fill_i64(status, -1, 1, s)) : QBN_OK;
    if (src->format == QBN_NVFP4 || src->format == QBN_NVFP4_CKE)
        return hip_status(qbn::launch_repack_cke(*src, (void *)dst->data, (void *)dst->scales, s));
    return hip_status(qbn::launch_repack(*src, *dst, q4_0_dir ? status + 1 : nullptr, q4_0_dir ? status : nullptr, s));
}

int32_t qbn_repack_noalloc(const qbn_tensor *src, const qbn_tensor *dst, int64_t *result, void *stream) {
    bool q4_0_dir = false;
    int32_t st = check_repack(src, dst, &q4_0_dir);
    if (st) return st;
    if (q4_0_dir) {
        if (!result) return QBN_ERR_NULL;
        if (!aligned(result, 8)) return QBN_ERR_ALIGN;
    }
    hipStream_t s = (hipStream_t)stream;
    if (src->n == 0 || src->k == 0) return q4_0_dir ? hip_status(qbn::launch_fill_i64(result, -1, 1, s)) : QBN_OK;
    if (src->format == QBN_NVFP4 || src->format == QBN_NVFP4_CKE)
        return hip_status(qbn::launch_repack_cke(*src, (void *)dst->data, (void *)dst->scales, s));
    int64_t *parts = nullptr;
    if (q4_0_dir) {
        const hipError_t e = qbn::repack_scratch(&parts);
        if (e != hipSuccess) return hip_status(e);
    }
    return hip_status(qbn::launch_repack(*src, *dst, parts, q4_0_dir ? result : nullptr, s));
}

int32_t qbn_validate_async(const qbn_tensor *w, int64_t *first_bad, void *stream) {
    const int32_t st = check_validate(w);
    if (st) return st;
    if (!first_bad) return QBN_ERR_NULL;
    if (!aligned(first_bad, 8)) return QBN_ERR_ALIGN;
    return hip_status(qbn::launch_validate(*w, first_bad, (hipStream_t)stream));
}

int32_t qbn_validate(const qbn_tensor *w, int64_t *first_bad, void *stream) {
    int32_t st = check_validate(w);  // every argument error is reported before anything is allocated
    if (st) return st;
    int64_t *dev = nullptr;
    hipError_t e = hipMalloc((void **)&dev, sizeof(int64_t));
    if (e != hipSuccess) return hip_status(e);
    hipStream_t s = (hipStream_t)stream;
    int64_t found = -1;
    e = qbn::launch_validate(*w, dev, s);
    if (e == hipSuccess) e = hipMemcpyAsync(&found, dev, sizeof(int64_t), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    const hipError_t ef = hipFree(dev);
    if (e == hipSuccess) e = ef;
    if (e != hipSuccess) return hip_status(e);
    if (first_bad) *first_bad = found;
    return found >= 0 ? QBN_ERR_NAN_SCALE : QBN_OK;
}

}  // extern "C"
