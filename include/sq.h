/*
 * sq.h - C ABI of the MI355X (gfx950) W8A8 SmoothQuant linear-layer library.
 *
 * The library implements, as hand-written HIP kernels, the per-layer path of
 * SmoothQuant W8A8 post-training quantization and LLM.int8()'s mixed
 * decomposition.  Pages defining each operation (titles as printed):
 *   [SQ-tutorial] "大语言模型量化技术（四）：SmoothQuant" (wangyu.me)
 *   [SQ-practice] "大模型量化困局与SmoothQuant的破局思路" (lpnh.cn)
 *   [SQ-ondevice] "如何通过 SmoothQuant 解决激活值离群点难题" (tbr8.org)
 *   [INT8-expl]   LLM.int8() explainer (xdnf.cn)
 *   [SQ-wiki]     "SmoothQuant" encyclopedia entry (newton.com.tw)
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers owned by the caller (allocated with
 *    hipMalloc or by a framework); the library never allocates, frees or
 *    keeps them.  Tensors are dense and row-major.
 *  - Layouts: X is [M, K] (tokens x input channels, K contiguous), W is
 *    [N, K] (output x input channels, the nn.Linear layout), Y is [M, N].
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is enqueued on it; the library never synchronizes, so results are
 *    ready once the stream is.  Calls that share output buffers must be
 *    ordered by the caller.
 *  - Every call returns an sq_status.  Argument errors are found on the host
 *    before anything is enqueued and leave all outputs untouched.  A failed
 *    launch returns SQ_ERR_HIP (hipGetLastError after the launch).
 *  - Sizes are int64_t; 0 rows/tokens/outputs is allowed and enqueues
 *    nothing (except where stated).  A row length or inner dimension K of 0
 *    with at least one row (or output) is rejected with SQ_ERR_SHAPE before
 *    any pointer is used: there is no row to quantize and no sum to form.
 *    Row strides must be multiples of 16
 *    bytes and int8 / 16-bit / fp32 tensor pointers 16-byte aligned, so the
 *    kernels can move 16-byte vectors: K % 16 == 0 for int8 operands,
 *    cols % 8 == 0 (16-bit) or cols % 4 == 0 (fp32) for reductions.
 *  - Floating point: fp32 arithmetic, IEEE round-to-nearest-even, no
 *    contraction of a*b+c into fma, denormals kept.  Inputs must be finite.
 */
#ifndef SQ_H
#define SQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SQ_OK = 0,
    SQ_ERR_NULL = 1,        /* a required pointer is NULL */
    SQ_ERR_SHAPE = 2,       /* negative size or unsupported divisibility */
    SQ_ERR_DTYPE = 3,       /* element type not allowed for this argument */
    SQ_ERR_ALIGN = 4,       /* pointer not 16-byte aligned */
    SQ_ERR_ARG = 5,         /* alpha outside [0,1], threshold <= 0 or NaN, bad mode */
    SQ_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than required */
    SQ_ERR_UNSUPPORTED = 7, /* combination not implemented */
    SQ_ERR_HIP = 8          /* the HIP runtime reported an error */
} sq_status;

typedef enum { SQ_F32 = 0, SQ_F16 = 1, SQ_BF16 = 2 } sq_dtype;

typedef enum { SQ_PER_TENSOR_STATIC = 0, SQ_PER_TOKEN_DYNAMIC = 1 } sq_qmode;

typedef enum { SQ_NORM_LAYER = 0, SQ_NORM_RMS = 1 } sq_norm;

/* Human-readable name of a status code (static string). */
const char *sq_status_str(int status);

/* Library ABI version (major * 100 + minor). */
int sq_version(void);

/*
 * a1 - per-channel abs-max (calibration statistics).
 * [SQ-tutorial] 缩放因子: x_j = max_i |X_ij| (activations, over all tokens) and
 * w_j = max over output channels of |W| in input channel j; [SQ-practice] §3.2
 * and [SQ-ondevice] §3 compute both as column maxima.
 *   x        [rows, cols] of dt (SQ_F32, SQ_F16 or SQ_BF16)
 *   amax_out [cols] fp32: amax_out[c] = max_r |x[r, c]|.  With accumulate != 0
 *            the result is max(previous amax_out[c], that) - a running max over
 *            calibration batches; amax_out must then hold non-negative values.
 *            rows == 0 gives 0 (or leaves the running max unchanged).
 * Exact (a max of magnitudes has no rounding).  cols*size(dt) % 16 == 0.
 */
int sq_absmax_reduce(const void *x, int dt, int64_t rows, int64_t cols,
                     int accumulate, float *amax_out, void *stream);

/*
 * a2 - smoothing factors.  [SQ-tutorial] 缩放因子, s_j = x_j^alpha / w_j^(1-alpha);
 * clamps from [SQ-practice] §3.2.
 *   act_amax, w_amax [K] fp32 (from a1)
 *   s, inv_s         [K] fp32 out: xc = max(x_j, 1e-5), wc = max(w_j, 1e-5),
 *                    s_j = max(xc^alpha / wc^(1-alpha), 1e-5) (powers and
 *                    quotient in double, rounded once), inv_s_j = fl(1 / s_j).
 *   static_scale     [2] fp32 out or NULL: the per-tensor static activation
 *                    step {step, 1/step}: a = max(max_j fl(x_j * inv_s_j), 1e-8),
 *                    step = fl(a / 127), inv = fl(127 / a).  Since rounding is
 *                    monotone, a is the max of |fl(X * inv_s)| over the
 *                    calibration data.
 *   alpha in [0, 1].
 */
int sq_compute_scales(const float *act_amax, const float *w_amax, int64_t K,
                      float alpha, float *s, float *inv_s, float *static_scale,
                      void *stream);

/*
 * a3 - weight smoothing + per-output-channel int8.  [SQ-tutorial]
 * SmoothQuant 的原理 (SW: weight input channel j times s_j) and
 * 为什么激活不能用逐通道量化 (weights quantized per output channel);
 * quantizer of [INT8-expl] §2.1 (scale 127/max, round, clip to +-127).
 *   w       [N, K] of dt
 *   s       [K] fp32, or NULL for s = 1 (plain per-channel quantization)
 *   wq      [N, K] int8 out: w' = fl(W * s); a_n = max(max_k |w'|, 1e-8);
 *           q = clamp(round_half_even(fl(w' * fl(127 / a_n))), -127, 127)
 *   w_scale [N] fp32 out: fl(a_n / 127)
 * K % 16 == 0; K > 0 when N > 0.
 */
int sq_smooth_weights(const void *w, int dt, int64_t N, int64_t K,
                      const float *s, int8_t *wq, float *w_scale, void *stream);

/*
 * a4 - fused smoothing and activation int8 quantization.  xs = fl(X * inv_s)
 * ([SQ-ondevice] §3: X / s at inference; [SQ-practice] §3.3), then
 *   SQ_PER_TOKEN_DYNAMIC: per row a = max(max_k |xs|, 1e-8),
 *       x_scale[m] = fl(a / 127), q = clamp(rhe(fl(xs * fl(127 / a))), +-127)
 *   SQ_PER_TENSOR_STATIC: q = clamp(rhe(fl(xs * static_scale[1])), +-127),
 *       x_scale[0] = static_scale[0]
 * ([SQ-tutorial] 为什么激活不能用逐通道量化: per-tensor or per-token only).
 *   x            [M, K] of dt
 *   inv_s        [K] fp32 or NULL (no smoothing, e.g. folded upstream)
 *   static_scale [2] fp32 {step, 1/step} (static mode only, else ignored)
 *   xq           [M, K] int8 out; x_scale [M] (dynamic) or [1] (static) out
 *                (with M == 0 in dynamic mode nothing is written and x_scale
 *                may be NULL; in static mode x_scale[0] is still set)
 * K % 16 == 0; K > 0 when M > 0.
 */
int sq_quantize_act(const void *x, int dt, int64_t M, int64_t K,
                    const float *inv_s, int mode, const float *static_scale,
                    int8_t *xq, float *x_scale, void *stream);

/*
 * a3 with the next layer's smoothing folded into this layer's output
 * channels.  [SQ-tutorial] 融入前序线性层的权重 and its table of fold
 * positions: down_proj's input channel j must shrink by 1/s_j, which is done
 * by multiplying up_proj's output channel j by 1/s_j (o_proj's smoothing
 * likewise goes into v_proj); this layer's own input smoothing s still
 * scales its columns.
 *   w        [N, K] of dt (e.g. up_proj or v_proj)
 *   row_mul  [N] fp32 (the next layer's inv_s), or NULL (= sq_smooth_weights)
 *   s        [K] fp32, or NULL (this layer's columns unscaled)
 *   wq, w_scale as sq_smooth_weights, of w''[n, k] = fl(fl(w * row_mul[n]) * s[k]).
 * The next layer then quantizes its input with inv_s = NULL (the division
 * already happened here).  K % 16 == 0 (K > 0 when N > 0); row_mul 4-byte
 * aligned.
 */
int sq_smooth_weights_folded(const void *w, int dt, int64_t N, int64_t K,
                             const float *row_mul, const float *s, int8_t *wq,
                             float *w_scale, void *stream);

/*
 * Per-tensor static step for a largest code qmax: a = max(max_j
 * fl(act_amax_j * inv_s_j), 1e-8) (inv_s NULL: act_amax_j), static_scale =
 * {fl(a / qmax), fl(qmax / a)}.  qmax = 127 gives a2's int8 step, 448 the
 * e4m3 one.  [SQ-practice] §7.3 (static steps fixed after calibration).
 *   act_amax [K], inv_s [K] or NULL, static_scale [2] out; qmax > 0 finite.
 */
int sq_static_scale(const float *act_amax, const float *inv_s, int64_t K, float qmax,
                    float *static_scale, void *stream);

/*
 * f4 - the FP8 (OCP e4m3fn) form of a3 and a4.  [SQ-wiki] 技術原理與特性:
 * the quantized model can use INT8 or FP8 compute units.  Same definitions
 * as the int8 entry points with 448 (the largest finite e4m3 value) in place
 * of 127: step = fl(a / 448), q = e4m3(clamp(fl(v * fl(448 / a)), -448, 448)),
 * rounding to nearest even; codes are bytes (sign, 4 exponent bits with bias
 * 7, 3 mantissa bits; 0x7F / 0xFF are NaN and never produced).
 *   sq_smooth_weights_fp8: w [N, K] of dt, s [K] or NULL -> wq [N, K] e4m3,
 *                          w_scale [N].
 *   sq_quantize_act_fp8:   x [M, K] of dt, inv_s [K] or NULL, mode and
 *                          static_scale as sq_quantize_act (the static pair
 *                          from sq_static_scale with qmax 448) -> xq [M, K]
 *                          e4m3, x_scale [M] or [1].
 * K % 16 == 0; K > 0 when there are rows.
 */
int sq_smooth_weights_fp8(const void *w, int dt, int64_t N, int64_t K, const float *s,
                          uint8_t *wq, float *w_scale, void *stream);
int sq_quantize_act_fp8(const void *x, int dt, int64_t M, int64_t K, const float *inv_s,
                        int mode, const float *static_scale, uint8_t *xq, float *x_scale,
                        void *stream);

/*
 * f4 - e4m3 x e4m3 GEMM on the matrix cores' FP8 path ([SQ-wiki]
 * 技術原理與特性: INT8 or FP8 units) with a5's dequant epilogue.
 *   xq [M, K] e4m3, wq [N, K] e4m3 (from the _fp8 quantizers)
 *   x_scale, x_scale_per_row, w_scale, y, y_dt as sq_gemm_i8_dequant:
 *   y = fl(acc * fl(x_scale[m] * w_scale[n])) narrowed RNE, where acc is
 *   sum_k dec(xq[m,k]) dec(wq[n,k]) as the matrix cores form it: products
 *   are exact, each block of 64 consecutive k is aligned to its largest
 *   product with limited precision below it, and the blocks are added in
 *   fp32 (|acc - exact| <= 2^-9 sum_blocks max|p| + K 2^-24 sum|p|,
 *   measured well inside on this GPU).  Results are deterministic.
 * K % 128 == 0 (K > 0).
 */
int sq_gemm_fp8_dequant(const uint8_t *xq, const uint8_t *wq, int64_t M, int64_t N,
                        int64_t K, const float *x_scale, int x_scale_per_row,
                        const float *w_scale, void *y, int y_dt, void *stream);

/*
 * a5 - int8 x int8 -> int32 GEMM with the outer-product dequant epilogue.
 * [SQ-tutorial] Y = diag(delta_X) X_int8 W_int8 diag(delta_W);
 * [INT8-expl] §2.1 (int32 accumulation, c_x (x) c_w).
 *   xq [M, K] int8, wq [N, K] int8
 *   x_scale: [M] fp32 if x_scale_per_row != 0, else [1] (per-tensor)
 *   w_scale: [N] fp32
 *   y  [M, N] of y_dt out: acc = sum_k xq[m,k] * wq[n,k] (exact int32),
 *      y = fl(fl((float)acc) * fl(x_scale[m] * w_scale[n])) narrowed RNE.
 *   acc_out [M, N] int32 out or NULL (the integer sums, for checking).
 * K % 16 == 0, K > 0 when M, N > 0; |acc| must fit int32 (holds for
 * K <= 133143).  M <= 32 uses
 * the skinny (decode) kernel, larger M the tiled MFMA kernel; both give the
 * same bits.
 */
int sq_gemm_i8_dequant(const int8_t *xq, const int8_t *wq, int64_t M,
                       int64_t N, int64_t K, const float *x_scale,
                       int x_scale_per_row, const float *w_scale, void *y,
                       int y_dt, int32_t *acc_out, void *stream);

/*
 * a6 - LLM.int8() mixed-precision matmul ([INT8-expl] §2.2 decomposition;
 * §4.1: a dimension is an outlier when any value reaches the threshold).
 *   x         [M, K] fp16 activations
 *   wq, w_scale  [N, K] int8 and [N] fp32: the weights' per-output-channel
 *             int8 form over ALL K (sq_smooth_weights with s = NULL)
 *   w_f16     [N, K] fp16 original weights (read only in outlier columns)
 *   threshold > 0 (may be +inf: no outliers)
 *   y         [M, N] of y_dt out:
 *     O = ascending { j : some |x[m, j]| >= threshold };
 *     X~ = x with the O columns zeroed, quantized per token (a4 dynamic,
 *     no smoothing); acc = X~q . wq^T;
 *     side = sum over o in O ascending of fl(x[m,o] * w[n,o]) in fp32 from 0;
 *     y = fl(fl((float)acc * fl(dx_m * dw_n)) + side), narrowed RNE.
 *   acc_out   [M, N] int32 out or NULL: the int8 sums acc (for checking).
 *   n_outliers_out  device int32 out or NULL: |O|.
 *   workspace       device memory of at least
 *                   sq_int8_mixed_matmul_workspace(M, N, K) bytes, 256-byte
 *                   aligned.  On return it holds, with R(b) = b rounded up
 *                   to a multiple of 256, C = min(K, SQ_MIXED_SIDE_COLS)
 *                   and parts back to back:
 *                     X~q [M, K] int8 at 0;
 *                     the row steps dx [M] fp32 at R(M K);
 *                     the column maxima of |x| [K] fp32, R(4 M) further;
 *                     the column mask [K] fp32 (1 kept, 0 outlier), R(4 K)
 *                     further; the O list [K] int32 (its first |O| entries,
 *                     ascending), R(4 K) further; |O| int32, R(4 K) further;
 *                     when |O| <= C, the side operands as fp32, their first
 *                     |O| rows: x[m, O_t] at [t, m] of a [C, M] array 256
 *                     bytes further, w[n, O_t] at [t, n] of a [C, N] array
 *                     R(4 C M) further (not written when |O| > C: the side
 *                     product then reads x and w_f16 directly).
 * K % 16 == 0; K > 0 when M, N > 0.
 */
#define SQ_MIXED_SIDE_COLS 128
size_t sq_int8_mixed_matmul_workspace(int64_t M, int64_t N, int64_t K);
int sq_int8_mixed_matmul(const void *x, int64_t M, int64_t K, const int8_t *wq,
                         const float *w_scale, const void *w_f16, int64_t N,
                         float threshold, void *workspace,
                         size_t workspace_bytes, void *y, int y_dt,
                         int32_t *acc_out, int32_t *n_outliers_out, void *stream);

/*
 * sq_int8_mixed_matmul for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation, arguments and results, with no
 * workspace argument.  The decomposition's intermediates live in a device
 * array of SQ_MIXED_SCRATCH_BYTES that the library holds on every GPU it
 * runs on until the process ends; the call allocates nothing.
 *   Returns SQ_ERR_WORKSPACE when sq_int8_mixed_matmul_workspace(M, N, K)
 *   exceeds SQ_MIXED_SCRATCH_BYTES (M = 2048, N = K = 4096 needs about
 *   11.6 MB; with N = K = 4096 up to 6810 rows fit),
 *   SQ_ERR_HIP when the array's device address cannot be obtained (looked up
 *   once per GPU, with that GPU current, on the first call there).
 * Every call on a GPU uses that GPU's one array: calls that overlap on one
 * GPU (other streams, other threads) race and must be ordered by the
 * caller.  The array keeps the last call's intermediates (laid out as the
 * workspace above); each call rewrites everything it reads.
 */
#define SQ_MIXED_SCRATCH_BYTES (32u << 20)
int sq_int8_mixed_matmul_noalloc(const void *x, int64_t M, int64_t K, const int8_t *wq,
                                 const float *w_scale, const void *w_f16, int64_t N,
                                 float threshold, void *y, int y_dt, int32_t *acc_out,
                                 int32_t *n_outliers_out, void *stream);

/*
 * Folding the smoothing into the norm that precedes the layer
 * ([SQ-tutorial] section 融入 LayerNorm: the norm's output times 1/s_j is
 * obtained by dividing its parameters once).
 *   gamma, beta  [K] fp32 in (beta may be NULL: no shift)
 *   s            [K] fp32 smoothing factors (sq_compute_scales)
 *   gamma_out    [K] fp32 out: fl(gamma_j / s_j)
 *   beta_out     [K] fp32 out: fl(beta_j / s_j); required iff beta != NULL
 * Outputs may alias their inputs.  Pointers 4-byte aligned.
 */
int sq_fold_norm(const float *gamma, const float *beta, const float *s, int64_t K,
                 float *gamma_out, float *beta_out, void *stream);

/*
 * Fused norm + int8 quantization of fp16 rows: the norm of [SQ-tutorial]
 * 融入 LayerNorm, y_j = (x_j - mu) / sigma * gamma_j + beta_j, with the
 * folded parameters (sq_fold_norm) it emits the smoothed activation, which
 * is quantized in the same pass as sq_quantize_act does (per token or per
 * tensor) - the residual row is read once and only int8 is written.
 *   x      [M, K] fp16 (dt must be SQ_F16), finite
 *   norm   SQ_NORM_LAYER: mu = mean_j x_j, sigma^2 = mean_j (x_j - mu)^2;
 *          SQ_NORM_RMS:   mu = 0,          sigma^2 = mean_j x_j^2
 *          The sums are exact (every fp16 value times 2^24 is an integer);
 *          in double: mu = S1 / (K 2^24), sigma^2 from the exact integers,
 *          rstd = 1 / sqrt(sigma^2 + eps); then mu, rstd rounded to fp32.
 *   gamma  [K] fp32 (16-byte aligned); beta [K] fp32 or NULL (no shift)
 *   eps    >= 0, finite
 *   per element in fp32: n = fl(fl(x - mu) * rstd) (LAYER) or fl(x * rstd)
 *          (RMS), y = fl(n * gamma_j), then y = fl(y + beta_j) if beta
 *   mode / static_scale / xq / x_scale: as sq_quantize_act, applied to y
 * K % 16 == 0, 16 <= K <= 16384 when M > 0 (else SQ_ERR_SHAPE /
 * SQ_ERR_UNSUPPORTED).
 */
int sq_norm_quantize_act(const void *x, int dt, int64_t M, int64_t K, int norm,
                         const float *gamma, const float *beta, float eps, int mode,
                         const float *static_scale, int8_t *xq, float *x_scale,
                         void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SQ_H */
