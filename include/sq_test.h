/*
 * sq_test.h - coverage entry points of the W8A8 library (libsq.so).
 *
 * The tiled int8 / e4m3 GEMM picks its block shape from the problem shape.
 * These calls are the GEMM entry points of sq.h with that choice forced, so
 * that tests reach every block shape on small problems.  Every shape gives
 * the same bits (the integer sums do not depend on the order of their
 * terms, the e4m3 sums are formed block by block in the same order, and the
 * epilogue is per element).  Same arguments, checks and results as the
 * sq.h entry point of the same name, plus:
 *   tile  -1 the library's choice; 0, 1, 2 the block shapes 256 x 256,
 *         256 x 128, 128 x 128 (for M > 32; with M <= 32 the decode kernel
 *         runs either way); for sq_gemm_i8_dequant_tile also 3, 128 x 128
 *         tiles of eight waves in K-split pairs (K % 128 == 0; other K run
 *         the 256 x 128 shape).  Other values return SQ_ERR_ARG.
 * Defined by the same passages as their sq.h counterparts: the SmoothQuant
 * tutorial page's Y = diag(dX) X_int8 W_int8 diag(dW); the LLM.int8()
 * explainer's §2.1 (int32 sums, outer-product dequant) and §2.2
 * (decomposition); the SmoothQuant encyclopedia page's INT8 or FP8 units.
 */
#ifndef SQ_TEST_H
#define SQ_TEST_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int sq_gemm_i8_dequant_tile(const int8_t *xq, const int8_t *wq, int64_t M, int64_t N,
                            int64_t K, const float *x_scale, int x_scale_per_row,
                            const float *w_scale, void *y, int y_dt, int32_t *acc_out,
                            void *stream, int tile);

int sq_gemm_fp8_dequant_tile(const uint8_t *xq, const uint8_t *wq, int64_t M, int64_t N,
                             int64_t K, const float *x_scale, int x_scale_per_row,
                             const float *w_scale, void *y, int y_dt, void *stream, int tile);

int sq_int8_mixed_matmul_tile(const void *x, int64_t M, int64_t K, const int8_t *wq,
                              const float *w_scale, const void *w_f16, int64_t N,
                              float threshold, void *workspace, size_t workspace_bytes, void *y,
                              int y_dt, int32_t *acc_out, int32_t *n_outliers_out, void *stream,
                              int tile);

/*
 * The fused norm -> int8 quantizer of sq.h with its kernel forced:
 *   kernel  -1 the library's choice; 0 the block-per-row kernel; 1 the
 *           wave-per-row kernel (built for K = 2048, 3072, ..., 8192; other
 *           K run the block-per-row kernel).  Other values return
 *           SQ_ERR_ARG.  Both kernels give the same bits (exact row sums,
 *           the same per-element operations).
 * Defined by the passage of its sq.h counterpart: the SmoothQuant tutorial
 * page's section on folding the smoothing into LayerNorm.
 */
int sq_norm_quantize_act_kernel(const void *x, int dt, int64_t M, int64_t K, int norm,
                                const float *gamma, const float *beta, float eps, int mode,
                                const float *static_scale, int8_t *xq, float *x_scale,
                                void *stream, int kernel);

#ifdef __cplusplus
}
#endif

#endif /* SQ_TEST_H */
