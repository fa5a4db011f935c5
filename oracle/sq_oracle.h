/*
 * CPU ORACLE for the SmoothQuant W8A8 linear-layer path and the LLM.int8()
 * mixed decomposition.  TEST INFRASTRUCTURE ONLY: only the tests, the smoke
 * check and the benchmark's CPU-baseline leg may load it.  The product path
 * never calls it, and it shares no code, header or table with the GPU path.
 *
 * Plain C11, built with -O2 -std=c11 -ffp-contract=off -fno-fast-math.
 * Every floating-point step is one IEEE-754 binary32 operation with
 * round-to-nearest-even unless a step says "double".  OpenMP is used only
 * over independent output rows; each output element is computed by one
 * thread in a fixed order, so results do not depend on the thread count.
 *
 * Pages cited (titles as printed on them):
 *   [SQ-tutorial] "大语言模型量化技术（四）：SmoothQuant" (wangyu.me)
 *   [SQ-practice] "大模型量化困局与SmoothQuant的破局思路" (lpnh.cn)
 *   [SQ-ondevice] "如何通过 SmoothQuant 解决激活值离群点难题" (tbr8.org)
 *   [SQ-wiki]     "SmoothQuant" encyclopedia entry (newton.com.tw)
 *   [INT8-expl]   LLM.int8() explainer (xdnf.cn), "8 位推理为什么在 6.7B 处突然崩掉"
 *
 * Parity status of each function is stated beside it; "pinned" means a
 * CPU test checks it against something other than itself (a printed worked
 * example, a closed form, an invariant or a library routine).
 *
 * Layouts: row-major.  X is [M, K] (tokens x input channels), W is [N, K]
 * (output x input channels, the nn.Linear layout), Y is [M, N].
 * Element-type codes: 0 = fp32, 1 = fp16, 2 = bf16 (16-bit values are passed
 * as their raw uint16 bit patterns).
 */
#ifndef SQ_ORACLE_H
#define SQ_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#define ORC_F32 0
#define ORC_F16 1
#define ORC_BF16 2

#define ORC_PER_TENSOR_STATIC 0
#define ORC_PER_TOKEN_DYNAMIC 1

/* Threads used by the parallel loops (OpenMP); n <= 0 leaves it unchanged. */
int orc_set_num_threads(int n);

/* Exact widening and round-to-nearest-even narrowing of 16-bit floats
 * (IEEE-754 binary16; bfloat16 = upper half of binary32).  Pinned against
 * numpy/torch conversions. */
float orc_f16_to_f32(uint16_t h);
float orc_bf16_to_f32(uint16_t b);
uint16_t orc_f32_to_f16(float f);
uint16_t orc_f32_to_bf16(float f);

/* Round half to even, the rounding the quantizer uses. Pinned (ties). */
float orc_round_half_even(float v);

/* Per-channel abs-max: amax[c] = max_r |x[r, c]|; with accumulate != 0 the
 * result is max(amax[c], that) (a running max over calibration batches).
 * [SQ-tutorial] section 缩放因子, definition of x_j and w_j;
 * [SQ-practice] §3.2 calibration code; [SQ-ondevice] §3 step 1 and 2.
 * Pinned: numpy abs().max(axis=0). */
void orc_absmax_cols(const void *x, int dt, int64_t rows, int64_t cols,
                     int accumulate, float *amax);

/* Smoothing factors.  s_j = max(xc^alpha / wc^(1-alpha), 1e-5) with
 * xc = max(x_j, 1e-5), wc = max(w_j, 1e-5), the power and quotient in double
 * and rounded once to fp32; inv_s_j = fl(1 / s_j).
 * If static_scale != NULL: a = max(max_j fl(x_j * inv_s_j), 1e-8),
 * static_scale[0] = fl(a / 127) (step), static_scale[1] = fl(127 / a).
 * [SQ-tutorial] section 缩放因子 (equation for s_j and the three alpha cases);
 * [SQ-practice] §2.1 formula and §3.2 clamps; [SQ-ondevice] §3 step 3.
 * Pinned: worked example of [SQ-tutorial] 缩放的效果, alpha = 0 and 1 closed
 * forms, alpha = 0.5 balance, smoothed-max closed form. */
void orc_compute_scales(const float *act_amax, const float *w_amax, int64_t K,
                        float alpha, float *s, float *inv_s, float *static_scale);

/* Weight smoothing W'[n, k] = fl(W[n, k] * s[k]) (s == NULL: W' = W).
 * [SQ-tutorial] SmoothQuant 的原理 (SW scales weight channel j by s_j);
 * [SQ-ondevice] §3 step 4; [SQ-practice] §3.3 apply code.
 * Pinned: column max of W' equals fl(s_j * w_j). */
void orc_smooth_weights_f32(const void *w, int dt, int64_t N, int64_t K,
                            const float *s, float *w_smoothed);

/* Symmetric abs-max int8 quantization of each row of an fp32 matrix:
 * a = max(max_k |v|, 1e-8); step = fl(a / 127); inv = fl(127 / a);
 * q = clamp(round_half_even(fl(v * inv)), -127, 127).
 * [INT8-expl] §2.1 quantize_absmax / quantize_vectorwise;
 * [SQ-tutorial] 缩放的效果 (step = max / 127, round).
 * Pinned: worked example, ties, clamp, zero row, error bound. */
void orc_quantize_rows_f32(const float *v, int64_t rows, int64_t K, int8_t *q,
                           float *step);

/* a3: per-output-channel int8 weights of W' (above).  wq [N, K], w_scale [N]
 * holds the per-row step.  [SQ-tutorial] 为什么激活不能用逐通道量化 (weights
 * per output channel, dequant diag(delta_W) on the right). */
void orc_smooth_weights(const void *w, int dt, int64_t N, int64_t K,
                        const float *s, int8_t *wq, float *w_scale);

/* a3 with the next layer's smoothing folded into this layer's output
 * channels: W''[n, k] = fl(fl(W[n, k] * row_mul[n]) * s[k]) (row_mul == NULL:
 * no row factor; s == NULL: no column factor), then the row quantizer above.
 * [SQ-tutorial] 融入前序线性层的权重: down_proj's input channel j is shrunk by
 * 1/s_j by multiplying up_proj's output channel j by 1/s_j (likewise v_proj
 * for o_proj), so row_mul is the next layer's inv_s; this layer's own input
 * smoothing s still scales its columns.  The row factor is applied first
 * (the fold rewrites the stored weight, the smoothing then acts on it).
 * Pinned: row_mul = 1 gives a3; power-of-two row_mul gives a3's codes with
 * the steps scaled exactly; dequantized W'' against diag(r) W diag(s). */
void orc_fold_smooth_weights(const void *w, int dt, int64_t N, int64_t K,
                             const float *row_mul, const float *s, int8_t *wq,
                             float *w_scale);

/* a4: xs = fl(X * inv_s) (inv_s == NULL: xs = X), then
 *   mode PER_TOKEN_DYNAMIC: the row quantizer above, x_scale[M];
 *   mode PER_TENSOR_STATIC: q = clamp(rhe(fl(xs * static_scale[1]))),
 *                           x_scale[0] = static_scale[0].
 * [SQ-tutorial] 为什么激活不能用逐通道量化 (per-tensor or per-token only);
 * [SQ-practice] §3.3 (divide activations by s) and §7.3 (static vs dynamic);
 * [SQ-ondevice] §3 (X_new = X / s). */
void orc_quantize_act(const void *x, int dt, int64_t M, int64_t K,
                      const float *inv_s, int mode, const float *static_scale,
                      int8_t *xq, float *x_scale);

/* a5: acc[m, n] = sum_k xq[m, k] * wq[n, k] (exact integer sum, checked in
 * int64 and stored as int32); y = fl(fl((float)acc) * fl(dx_m * dw_n)) in
 * fp32, then narrowed RNE to y_dt.  dx_m = x_scale[per_row ? m : 0].
 * [SQ-tutorial] equation Y = diag(delta_X) X W diag(delta_W);
 * [INT8-expl] §2.1 (int32 accumulation; outer-product c_x (x) c_w dequant).
 * Pinned: int32 against numpy int64 matmul; unit scales give (float)acc;
 * fp32 y within 1 ulp-ish of the double product.
 * Returns the number of sums that did not fit int32 (0 expected). */
int64_t orc_gemm_i8_dequant(const int8_t *xq, const int8_t *wq, int64_t M,
                            int64_t N, int64_t K, const float *x_scale,
                            int per_row, const float *w_scale, void *y,
                            int y_dt, int32_t *acc_out);

/* The same definition evaluated at sampled (row, col) pairs only; y and acc
 * receive one element per pair (y in y_dt encoding). */
void orc_gemm_i8_dequant_at(const int8_t *xq, const int8_t *wq, int64_t K,
                            const float *x_scale, int per_row,
                            const float *w_scale, int y_dt, const int64_t *rows,
                            const int64_t *cols, int64_t n, void *y,
                            int32_t *acc);

/* LLM.int8() outlier columns: idx receives, ascending, every column j with
 * some |X[m, j]| >= threshold (X fp16).  Returns |O|.
 * [INT8-expl] §2.2 (columns whose magnitude exceeds the threshold form O)
 * and §4.1 (any value above the threshold marks the dimension).
 * Pinned: numpy brute force. */
int64_t orc_outlier_columns(const uint16_t *x_f16, int64_t M, int64_t K,
                            float threshold, int32_t *idx);

/* LLM.int8() mixed matmul ([INT8-expl] §2.2 decomposition):
 *  O from orc_outlier_columns; X~ = X with O columns zeroed; xq/x_scale =
 *  per-token dynamic quantization of X~ (no smoothing); acc = xq . wq^T;
 *  side[m, n] = sum over o in O ascending of fl(X[m,o] * W16[n,o]) in fp32
 *  starting from 0; y = fl(fl((float)acc * fl(dx_m * dw_n)) + side), then
 *  narrowed RNE to y_dt.  wq / w_scale are the weights' per-output-channel
 *  int8 form (orc_smooth_weights with s == NULL, over all K).
 *  Optional outputs (NULL to skip): acc_out [M,N], xq_out [M,K],
 *  x_scale_out [M], idx_out [K] (first |O| used).  Returns |O|.
 * Pinned: threshold +inf equals the plain vector-wise path; threshold tiny
 * (every column in O) equals the fp32-accumulated fp16 product within its
 * error bound. */
int64_t orc_int8_mixed_matmul(const uint16_t *x_f16, int64_t M, int64_t K,
                              const int8_t *wq, const float *w_scale,
                              const uint16_t *w_f16, int64_t N, float threshold,
                              void *y, int y_dt, int32_t *acc_out,
                              int8_t *xq_out, float *x_scale_out,
                              int32_t *idx_out);

/* Mixed matmul at sampled (row, col) pairs, given the full O list and the
 * quantized X~ (as produced by the call above on the same inputs). */
void orc_int8_mixed_at(const uint16_t *x_f16, int64_t K, const int8_t *xq,
                       const float *x_scale, const int8_t *wq,
                       const float *w_scale, const uint16_t *w_f16,
                       const int32_t *idx, int64_t n_idx, int y_dt,
                       const int64_t *rows, const int64_t *cols, int64_t n,
                       void *y, int32_t *acc);

/* fp64 references ([SQ-tutorial] SmoothQuant 的原理: (XS^-1)(SW) = XW in
 * the reals).  y64 [M, N] = X W^T in double; ys64 = (X diag(s)^-1)(diag(s) W)^T
 * in double, with X/s and W*s each formed in double.  Pinned: the invariant
 * ys64 = y64 to 1e-9 relative, and y64 against numpy float64 matmul. */
void orc_matmul_f64(const void *x, int xdt, const void *w, int wdt, int64_t M,
                    int64_t N, int64_t K, double *y64);
void orc_smoothed_matmul_f64(const void *x, int xdt, const void *w, int wdt,
                             const float *s, int64_t M, int64_t N, int64_t K,
                             double *ys64);

/* ------------------------------------------------------------------------
 * Folding the smoothing into the preceding norm, and the fused
 * norm -> int8 quantizer.
 *
 * [SQ-tutorial] section 融入 LayerNorm: the norm before q/k/v (and before
 * gate/up) computes y_j = (x_j - mu) / sigma * gamma_j + beta_j; dividing
 * its parameters once, gamma'_j = gamma_j / s_j and beta'_j = beta_j / s_j,
 * makes it emit y_j / s_j, the smoothed activation a4 would otherwise form.
 */
#define ORC_NORM_LAYER 0
#define ORC_NORM_RMS 1

/* gamma_out[j] = fl(gamma[j] / s[j]); beta_out[j] = fl(beta[j] / s[j]) when
 * beta != NULL.  Pinned: exact for power-of-two s; the folded norm equals
 * the unfolded one divided by s within rounding. */
void orc_fold_norm(const float *gamma, const float *beta, const float *s,
                   int64_t K, float *gamma_out, float *beta_out);

/* Row statistics of fp16 rows (x_f16 [M, K] raw bits), computed exactly:
 * every fp16 value times 2^24 is an integer below 2^40, so
 *   S1 = sum_j x_j 2^24 (int64) and S2 = sum_j (x_j 2^24)^2 (128-bit)
 * are exact in any order.  Then, in double:
 *   LAYER: mu = S1 / (K 2^24); var = (K S2 - S1^2) / (K^2 2^48)
 *          (the population variance, mean of (x - mu)^2, exactly);
 *   RMS:   mu = 0;           var = S2 / (K 2^48)      (mean of x^2);
 *   rstd = 1 / sqrt(var + eps);
 * and mu, rstd rounded to fp32.  The 128-bit integers are converted to
 * double as fl(hi 2^64 + fl(lo)) (hi, lo the 64-bit halves).
 * Pinned: mu, var against exact rational arithmetic; rstd against
 * 1/sqrt in double; invariance of the layer norm under x -> 2x (eps = 0). */
void orc_norm_stats(const uint16_t *x_f16, int64_t M, int64_t K, int norm,
                    float eps, float *mu, float *rstd);

/* Fused norm + int8 quantization of fp16 rows.  Per element, in fp32:
 *   LAYER: y = fl(fl(fl(x - mu) * rstd) * gamma_j)  (+ beta_j, one more fl)
 *   RMS:   y = fl(fl(x * rstd) * gamma_j)           (+ beta_j if given)
 * with (mu, rstd) from orc_norm_stats; gamma / beta are the folded
 * parameters (orc_fold_norm) or the plain ones.  Then, as orc_quantize_act:
 * PER_TOKEN_DYNAMIC quantizes each row with its own step (x_scale[M]),
 * PER_TENSOR_STATIC uses static_scale (x_scale[0] = static_scale[0]).
 * y_out (optional, [M, K] fp32) receives y.  [SQ-tutorial] 融入 LayerNorm
 * (the norm and its folded parameters) and 为什么激活不能用逐通道量化
 * (per-token / per-tensor activation quantization).
 * Pinned: y against the fp64 norm; constant rows give y = beta exactly. */
void orc_norm_quantize(const uint16_t *x_f16, int64_t M, int64_t K, int norm,
                       const float *gamma, const float *beta, float eps,
                       int mode, const float *static_scale, int8_t *xq,
                       float *x_scale, float *y_out);

/* ------------------------------------------------------------------
 * FP8 (e4m3) variant of the same path.  [SQ-wiki] 技術原理與特性: a
 * SmoothQuant-quantized model can run on INT8 or FP8 compute units.  The
 * scale semantics are those of the int8 path with 448, the largest finite
 * e4m3 value, in place of 127 (reading: the page gives no FP8 details).
 *
 * Format (OCP e4m3fn): sign, 4 exponent bits with bias 7, 3 mantissa bits;
 * exponent 0 holds the subnormals m 2^-9; 0x7F and 0xFF are NaN; no
 * infinities; the largest finite value is 1.75 2^8 = 448.
 * Pinned: decode of all 256 codes and encode of |v| <= 448 against torch's
 * float8_e4m3fn conversion; round trip of every finite code; ties. */
float orc_fp8_decode(uint8_t b);
/* |v| <= 448 (callers clamp): the nearest e4m3 value, ties to the even
 * code (the even mantissa). */
uint8_t orc_fp8_encode(float v);

/* Row quantizer to e4m3: a = max(max_k |v|, 1e-8); step = fl(a / 448);
 * inv = fl(448 / a); q = encode(clamp(fl(v * inv), -448, 448)).
 * Pinned: the row maximum lands on +-448; zero rows; the relative
 * reconstruction error of normal values is at most 2^-4. */
void orc_quantize_rows_fp8(const float *v, int64_t rows, int64_t K, uint8_t *q,
                           float *step);
/* a3 in e4m3: w' = fl(W * s) (s may be NULL), per output channel. */
void orc_smooth_weights_fp8(const void *w, int dt, int64_t N, int64_t K,
                            const float *s, uint8_t *wq, float *w_scale);
/* a4 in e4m3: xs = fl(X * inv_s) (inv_s may be NULL); PER_TOKEN_DYNAMIC:
 * the row quantizer above; PER_TENSOR_STATIC: encode(clamp(fl(xs *
 * static_scale[1]), -448, 448)) and x_scale[0] = static_scale[0]. */
void orc_quantize_act_fp8(const void *x, int dt, int64_t M, int64_t K,
                          const float *inv_s, int mode, const float *static_scale,
                          uint8_t *xq, float *x_scale);
/* The per-tensor static step for a largest code qmax (127 for int8, 448 for
 * e4m3): a = max(max_j fl(x_j * inv_s_j), 1e-8) (inv_s may be NULL);
 * out = {fl(a / qmax), fl(qmax / a)}. */
void orc_static_scale(const float *act_amax, const float *inv_s, int64_t K,
                      float qmax, float *out);
/* e4m3 GEMM: acc[m, n] = sum_k dec(xq[m, k]) dec(wq[n, k]) in double, which
 * is exact (every product is a multiple of 2^-18 below 2^18, so K <= 2^16
 * terms need fewer than 53 bits); y = fl(fl32(acc) * fl(dx_m * dw_n)),
 * narrowed RNE.  acc_out (double [M, N]) or NULL receives acc.
 * Pinned: acc against numpy's fp64 product on integer-valued codes. */
void orc_gemm_fp8_dequant(const uint8_t *xq, const uint8_t *wq, int64_t M, int64_t N,
                          int64_t K, const float *x_scale, int per_row,
                          const float *w_scale, void *y, int y_dt, double *acc_out);
/* The same at the n (row, col) pairs given (large shapes, sampled). */
void orc_gemm_fp8_dequant_at(const uint8_t *xq, const uint8_t *wq, int64_t K,
                             const float *x_scale, int per_row, const float *w_scale,
                             int y_dt, const int64_t *rows, const int64_t *cols,
                             int64_t n, void *y, double *acc_out);

#endif
