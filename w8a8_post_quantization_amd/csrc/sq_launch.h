// Internal launchers behind the C ABI (include/sq.h).  Arguments arrive
// validated; each launcher only enqueues kernels on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sq {

void launch_absmax(const void *x, int dt, int64_t rows, int64_t cols, int accumulate,
                   float *amax, hipStream_t stream);

void launch_compute_scales(const float *act_amax, const float *w_amax, int64_t K, float alpha,
                           float *s, float *inv_s, float *static_scale, hipStream_t stream);

// Per-row quantization of fl(fl(x * row_mul[r]) * mul[k]) (row_mul and mul
// may be NULL; row_mul only with dynamic steps): a3 uses it for weights
// (row_mul: the next layer's folded 1/s), a4 for activations (either mode),
// a6 for the outlier-masked rows.
void launch_quant_rows(const void *x, int dt, int64_t rows, int64_t K, const float *mul,
                       int dynamic, const float *static_scale, int8_t *q, float *scale,
                       hipStream_t stream, const float *row_mul = nullptr);

// e4m3 codes (OCP e4m3fn), 448 in place of 127; per-row or static steps.
void launch_quant_rows_fp8(const void *x, int dt, int64_t rows, int64_t K, const float *mul,
                           int dynamic, const float *static_scale, uint8_t *q, float *scale,
                           hipStream_t stream);
// {a/qmax, qmax/a} with a = max(max_j fl(act_amax_j * inv_s_j), 1e-8).
void launch_static_scale(const float *act_amax, const float *inv_s, int64_t K, float qmax,
                         float *out, hipStream_t stream);

// e4m3 x e4m3 -> fp32 GEMM, y = fl(acc * fl(dx * dw)); K % 128 == 0.
void launch_gemm_fp8(const uint8_t *xq, const uint8_t *wq, int64_t M, int64_t N, int64_t K,
                     const float *x_scale, int per_row, const float *w_scale, void *y, int y_dt,
                     hipStream_t stream);

struct SideTerm {  // LLM.int8() fp16 side product over outlier columns
    const uint16_t *x16;   // [M, K]
    const uint16_t *w16;   // [N, K]
    const int32_t *idx;    // device list of outlier columns, ascending
    const int32_t *count;  // device |O|
};

void launch_gemm(const int8_t *xq, const int8_t *wq, int64_t M, int64_t N, int64_t K,
                 const float *x_scale, int per_row, const float *w_scale, void *y, int y_dt,
                 int32_t *acc_out, const SideTerm *side, hipStream_t stream);

// LLM.int8() preparation: column abs-max of x into colmax, then the mask
// (1.0 keep / 0.0 outlier), the ascending O list and its count (also into
// count_out when that is not null).
void launch_outlier_prep(const void *x, int64_t M, int64_t K, float threshold, float *colmax,
                         float *mask, int32_t *idx, int32_t *count, int32_t *count_out,
                         hipStream_t stream);

// Folding 1/s into the norm's parameters, and the fused fp16 norm ->
// int8 row quantizer (K <= 16384).
void launch_fold_norm(const float *gamma, const float *beta, const float *s, int64_t K,
                      float *gamma_out, float *beta_out, hipStream_t stream);
void launch_norm_quant(const void *x, int64_t M, int64_t K, int norm, const float *gamma,
                       const float *beta, float eps, int dynamic, const float *static_scale,
                       int8_t *q, float *scale, hipStream_t stream);

// Tiny device-to-device copies done by a kernel (no copy-engine or memset
// nodes, so the calls stay capturable in a HIP graph).
void launch_copy_f32(const float *src, float *dst, hipStream_t stream);

}  // namespace sq
