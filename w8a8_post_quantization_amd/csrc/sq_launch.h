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

// LLM.int8() outlier columns for the masked row quantizer (launch_quant_rows
// with ol): the multiplier of column j is 1, or 0 when the column abs-max
// mul[j] reaches thr.  Extra blocks of the same launch write the 0/1 mask,
// the ascending list of outlier columns and its length (count, and
// count_out when not null), and, when |O| <= cap, the side operands
// xo[t M + m] = x[m, idx[t]] and wo[t N + n] = w16[n, idx[t]] as fp32.
constexpr int kSideColsMax = 128;  // largest cap
struct OutlierList {
    int on;
    float thr;
    float *mask;
    int32_t *idx;
    int32_t *count;
    int32_t *count_out;
    const uint16_t *w16;  // [N, K] fp16
    int64_t M, N;
    float *xo;            // [cap, M]
    float *wo;            // [cap, N]
    int cap;              // <= kSideColsMax
    int blocks;           // the extra blocks (set by the launcher)
};

// Per-row quantization of fl(fl(x * row_mul[r]) * mul[k]) (row_mul and mul
// may be NULL; row_mul only with dynamic steps): a3 uses it for weights
// (row_mul: the next layer's folded 1/s), a4 for activations (either mode),
// a6 (ol not null, dynamic) for the outlier-masked rows, mul = the column
// abs-max.
void launch_quant_rows(const void *x, int dt, int64_t rows, int64_t K, const float *mul,
                       int dynamic, const float *static_scale, int8_t *q, float *scale,
                       hipStream_t stream, const float *row_mul = nullptr,
                       const OutlierList *ol = nullptr);

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
                     hipStream_t stream, int force_tile = -1);

struct SideTerm {  // LLM.int8() fp16 side product over outlier columns
    const uint16_t *x16;   // [M, K]
    const uint16_t *w16;   // [N, K]
    const int32_t *idx;    // device list of outlier columns, ascending
    const int32_t *count;  // device |O|
    const float *xo;       // [cap, M]: x[m, idx[t]] at t M + m when |O| <= cap
    const float *wo;       // [cap, N]: w[n, idx[t]] at t N + n when |O| <= cap
    int cap;
};


// force_tile: -1 the launcher's choice; 0, 1, 2 the tiled kernels' block
// shape 256 x 256, 256 x 128, 128 x 128 (M > 32; the coverage entry points
// of sq_test.h), all giving the same bits.
void launch_gemm(const int8_t *xq, const int8_t *wq, int64_t M, int64_t N, int64_t K,
                 const float *x_scale, int per_row, const float *w_scale, void *y, int y_dt,
                 int32_t *acc_out, const SideTerm *side, hipStream_t stream,
                 int force_tile = -1);



// Folding 1/s into the norm's parameters, and the fused fp16 norm ->
// int8 row quantizer (K <= 16384).  force_kernel: -1 the launcher's choice,
// 0 the block-per-row kernel, 1 the wave-per-row kernel (K <= 8192).
void launch_fold_norm(const float *gamma, const float *beta, const float *s, int64_t K,
                      float *gamma_out, float *beta_out, hipStream_t stream);
void launch_norm_quant(const void *x, int64_t M, int64_t K, int norm, const float *gamma,
                       const float *beta, float eps, int dynamic, const float *static_scale,
                       int8_t *q, float *scale, hipStream_t stream, int force_kernel = -1);

// Tiny device-to-device copies done by a kernel (no copy-engine or memset
// nodes, so the calls stay capturable in a HIP graph).
void launch_copy_f32(const float *src, float *dst, hipStream_t stream);

}  // namespace sq
