// Internal launch entry points, one per kernel family. Arguments have been
// validated by the C-ABI layer (qbn_api.hip) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qbn.h"

namespace qbn {

hipError_t launch_gemv(const qbn_tensor &w, const void *x, int x_dtype, float *y, hipStream_t s);
hipError_t launch_gemv_cke(const qbn_tensor &w, const void *x, int x_dtype, float *y, hipStream_t s);
hipError_t launch_dequant_cke(const qbn_tensor &w, void *out, int out_dtype, int out_layout, hipStream_t s);
hipError_t launch_repack_cke(const qbn_tensor &src, void *dst_data, void *dst_scales, hipStream_t s);
hipError_t launch_gemv_int4(const qbn_tensor &w, const void *x, int x_dtype, float *y, hipStream_t s);
hipError_t launch_gptq_qzeros(const void *src, void *dst, int64_t groups, int64_t n, int version, int to_logical,
                              hipStream_t s);
hipError_t launch_gptq_resolve_g_idx(const void *qweight, const int32_t *g_idx, int64_t k, int64_t n, int64_t group,
                                     void *qweight_out, int32_t *perm, int32_t *status, hipStream_t s);
hipError_t launch_permute(const void *src, const int32_t *perm, int64_t count, int elem_bytes, void *dst,
                          hipStream_t s);
bool gptq_groups_fit(int64_t k, int64_t group);
hipError_t launch_quantize_nvfp4(const void *x, int x_dtype, int64_t m, int64_t k, int64_t ldx, float scale2, int tie,
                                 void *codes, void *scales, hipStream_t s);
hipError_t launch_quantize_int4_sym(const void *w, int w_dtype, int64_t m, int64_t k, int64_t ldw, int64_t group,
                                    void *codes, float *scales, hipStream_t s);
hipError_t launch_pack_bits(const void *values, int64_t count, int bits, int lo, void *words_lo, void *words_hi,
                            hipStream_t s);
hipError_t launch_unpack_bits(const void *words_lo, const void *words_hi, int64_t count, int bits, int lo,
                              void *values, hipStream_t s);
hipError_t launch_gemm(const qbn_tensor &w, int64_t m, const void *x, int64_t ldx, void *y, int64_t ldy,
                       hipStream_t s);
hipError_t launch_gemm_int4(const qbn_tensor &w, int64_t m, const void *x, int64_t ldx, void *y, int y_dtype,
                            int64_t ldy, hipStream_t s);
bool gemm_int4_grid_fits(int64_t m, int64_t n);
hipError_t launch_dequant(const qbn_tensor &w, void *out, int out_dtype, int out_layout, hipStream_t s);
// int4 repacks. The Q4_0 directions first run a refusal scan whose
// QBN_REPACK_SCAN_PARTS workgroups write their partial minima to parts[];
// the repack kernels reduce them, write *result (-1 or the first
// unrepresentable index) and write nothing on a refusal. parts and result
// are unused (may be NULL) by the other directions.
hipError_t launch_repack(const qbn_tensor &src, const qbn_tensor &dst, int64_t *parts, int64_t *result,
                         hipStream_t s);
// The device address of this GPU's file-scope scratch for parts[] (resolved
// once per device).
hipError_t repack_scratch(int64_t **parts);
hipError_t launch_fill_i64(int64_t *p, int64_t v, int64_t count, hipStream_t s);
hipError_t launch_scan_zero_points(const uint8_t *zeros, int64_t count, int64_t *parts, hipStream_t s);
hipError_t launch_scan_q4_0_groups(const uint8_t *blocks, int64_t n, int64_t k, int64_t group, int64_t *parts,
                                   hipStream_t s);
hipError_t launch_validate(const qbn_tensor &w, int64_t *first_bad, hipStream_t s);
hipError_t launch_quantize_q8(const void *x, int x_dtype, int64_t k, int8_t *q, float *d, int32_t *bsums,
                              hipStream_t s);
hipError_t launch_gemv_q8(const qbn_tensor &w, const int8_t *q, const float *d, const int32_t *bsums, float *y,
                          hipStream_t s);
hipError_t launch_gemv_a16q8(const qbn_tensor &w, const int8_t *q, const float *d, void *y, int y_dtype,
                             hipStream_t s);
hipError_t launch_quantize_mx(const void *x, int x_dtype, int64_t m, int64_t k, int64_t ldx, int x_format,
                              void *codes, void *scales, hipStream_t s);
hipError_t launch_gemm_mx(const qbn_tensor &w, int64_t m, const void *xcodes, const void *xscales, void *y,
                          int y_dtype, int64_t ldy, hipStream_t s);
hipError_t launch_fill_zero(void *out, int64_t bytes, hipStream_t s);
hipError_t launch_fill_zero_2d_u16(void *out, int64_t rows, int64_t cols, int64_t ld, hipStream_t s);

}  // namespace qbn
