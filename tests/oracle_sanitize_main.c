/* Every oracle function on small and edge-case inputs, built with
 * -fsanitize=address,undefined (no recovery) by tests/test_oracle_sanitize.py:
 * an out-of-bounds access, a use of freed memory, a leak or undefined
 * behaviour in the oracle stops this program with a non-zero status.
 * Test infrastructure only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "sq_oracle.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double urand(void) { /* xorshift64*: inputs only */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (double)((rng_state * 0x2545F4914F6CDD1Dull) >> 11) / 9007199254740992.0;
}
static float nrand(float scale) { return (float)((urand() * 2.0 - 1.0) * scale); }

static void run_shape(int64_t M, int64_t N, int64_t K) {
    float *x = malloc((size_t)(M * K + 1) * sizeof(float));
    float *w = malloc((size_t)(N * K + 1) * sizeof(float));
    uint16_t *x16 = malloc((size_t)(M * K + 1) * sizeof(uint16_t));
    uint16_t *w16 = malloc((size_t)(N * K + 1) * sizeof(uint16_t));
    for (int64_t i = 0; i < M * K; ++i) {
        x[i] = nrand(2.0f);
        if (i % 37 == 3) x[i] *= 20.0f; /* outlier-like values */
        x16[i] = orc_f32_to_f16(x[i]);
    }
    for (int64_t i = 0; i < N * K; ++i) {
        w[i] = nrand(0.05f);
        w16[i] = orc_f32_to_f16(w[i]);
    }
    float *xa = calloc((size_t)K + 1, sizeof(float)), *wa = calloc((size_t)K + 1, sizeof(float));
    orc_absmax_cols(x, ORC_F32, M, K, 0, xa);
    orc_absmax_cols(x16, ORC_F16, M, K, 1, xa);
    orc_absmax_cols(w, ORC_F32, N, K, 0, wa);
    float *s = malloc((size_t)(K + 1) * sizeof(float)), *inv = malloc((size_t)(K + 1) * sizeof(float));
    float st[2], st8[2];
    orc_compute_scales(xa, wa, K, 0.5f, s, inv, st);
    orc_static_scale(xa, inv, K, 448.0f, st8);
    orc_static_scale(xa, NULL, K, 127.0f, st8);

    float *ws32 = malloc((size_t)(N * K + 1) * sizeof(float));
    orc_smooth_weights_f32(w, ORC_F32, N, K, s, ws32);
    int8_t *wq = malloc((size_t)(N * K + 1)), *xq = malloc((size_t)(M * K + 1));
    float *wsc = malloc((size_t)(N + 1) * sizeof(float)), *xsc = malloc((size_t)(M + 1) * sizeof(float));
    orc_quantize_rows_f32(ws32, N, K, wq, wsc);
    orc_smooth_weights(w16, ORC_F16, N, K, s, wq, wsc);
    float *rm = malloc((size_t)(N + 1) * sizeof(float));
    for (int64_t n = 0; n < N; ++n) rm[n] = 0.5f + (float)urand();
    orc_fold_smooth_weights(w16, ORC_BF16, N, K, rm, s, wq, wsc);
    orc_fold_smooth_weights(w, ORC_F32, N, K, NULL, NULL, wq, wsc);
    orc_quantize_act(x, ORC_F32, M, K, inv, ORC_PER_TENSOR_STATIC, st, xq, xsc);
    orc_quantize_act(x16, ORC_F16, M, K, inv, ORC_PER_TOKEN_DYNAMIC, NULL, xq, xsc);

    const size_t MN = (size_t)(M * N > 3 ? M * N : 3); /* the sampled calls take 3 pairs */
    float *y = malloc(MN * sizeof(float));
    int32_t *acc = malloc(MN * sizeof(int32_t));
    orc_gemm_i8_dequant(xq, wq, M, N, K, xsc, 1, wsc, y, ORC_F32, acc);
    orc_gemm_i8_dequant(xq, wq, M, N, K, xsc, 0, wsc, y, ORC_BF16, NULL);
    int64_t rows[3] = {0, M > 1 ? M - 1 : 0, M / 2}, cols[3] = {N - 1, 0, N / 2};
    if (M > 0 && N > 0) orc_gemm_i8_dequant_at(xq, wq, K, xsc, 1, wsc, ORC_F16, rows, cols, 3, y, acc);

    int32_t *idx = malloc((size_t)(K + 1) * sizeof(int32_t));
    orc_outlier_columns(x16, M, K, 6.0f, idx);
    orc_int8_mixed_matmul(x16, M, K, wq, wsc, w16, N, 6.0f, y, ORC_F16, acc, xq, xsc, idx);
    int64_t no = orc_outlier_columns(x16, M, K, 6.0f, idx);
    if (M > 0 && N > 0)
        orc_int8_mixed_at(x16, K, xq, xsc, wq, wsc, w16, idx, no, ORC_F32, rows, cols, 3, y, acc);

    double *y64 = malloc((size_t)(M * N + 1) * sizeof(double));
    orc_matmul_f64(x16, ORC_F16, w, ORC_F32, M, N, K, y64);
    orc_smoothed_matmul_f64(x, ORC_F32, w16, ORC_F16, s, M, N, K, y64);

    float *g = malloc((size_t)(K + 1) * sizeof(float)), *b = malloc((size_t)(K + 1) * sizeof(float));
    float *g2 = malloc((size_t)(K + 1) * sizeof(float)), *b2 = malloc((size_t)(K + 1) * sizeof(float));
    for (int64_t k = 0; k < K; ++k) {
        g[k] = 1.0f + nrand(0.1f);
        b[k] = nrand(0.05f);
    }
    orc_fold_norm(g, b, s, K, g2, b2);
    orc_fold_norm(g, NULL, s, K, g2, NULL);
    float *mu = malloc((size_t)(M + 1) * sizeof(float)), *rs = malloc((size_t)(M + 1) * sizeof(float));
    float *yo = malloc((size_t)(M * K + 1) * sizeof(float));
    if (K > 0) {
        orc_norm_stats(x16, M, K, 0, 1e-5f, mu, rs);
        orc_norm_stats(x16, M, K, 1, 1e-6f, mu, rs);
        orc_norm_quantize(x16, M, K, 0, g2, b2, 1e-5f, ORC_PER_TOKEN_DYNAMIC, NULL, xq, xsc, yo);
        orc_norm_quantize(x16, M, K, 1, g2, NULL, 1e-6f, ORC_PER_TENSOR_STATIC, st, xq, xsc, NULL);
    }

    uint8_t *xq8 = malloc((size_t)(M * K + 1)), *wq8 = malloc((size_t)(N * K + 1));
    orc_quantize_rows_fp8(ws32, N, K, wq8, wsc);
    orc_smooth_weights_fp8(w16, ORC_F16, N, K, s, wq8, wsc);
    orc_quantize_act_fp8(x, ORC_F32, M, K, inv, ORC_PER_TOKEN_DYNAMIC, NULL, xq8, xsc);
    orc_quantize_act_fp8(x16, ORC_F16, M, K, NULL, ORC_PER_TENSOR_STATIC, st8, xq8, xsc);
    double *a64 = malloc(MN * sizeof(double));
    orc_gemm_fp8_dequant(xq8, wq8, M, N, K, xsc, 0, wsc, y, ORC_F32, a64);
    orc_gemm_fp8_dequant(xq8, wq8, M, N, K, xsc, 0, wsc, y, ORC_BF16, NULL);
    if (M > 0 && N > 0)
        orc_gemm_fp8_dequant_at(xq8, wq8, K, xsc, 0, wsc, ORC_F16, rows, cols, 3, y, a64);

    free(x); free(w); free(x16); free(w16); free(xa); free(wa); free(s); free(inv);
    free(ws32); free(wq); free(xq); free(wsc); free(xsc); free(rm); free(y); free(acc);
    free(idx); free(y64); free(g); free(b); free(g2); free(b2); free(mu); free(rs); free(yo);
    free(xq8); free(wq8); free(a64);
}

int main(void) {
    /* scalar conversions over every 16-bit pattern and the e4m3 codes */
    for (uint32_t h = 0; h < 65536; ++h) {
        volatile float a = orc_f16_to_f32((uint16_t)h), b = orc_bf16_to_f32((uint16_t)h);
        (void)orc_f32_to_f16(a);
        (void)orc_f32_to_bf16(b);
        (void)orc_round_half_even(a);
    }
    for (int c = 0; c < 256; ++c) {
        float v = orc_fp8_decode((uint8_t)c);
        if (v == v) (void)orc_fp8_encode(v);
    }
    const int64_t shapes[][3] = {{1, 1, 16}, {3, 5, 48}, {17, 9, 64}, {0, 4, 32}, {4, 0, 32},
                                 {2, 3, 0}, {33, 65, 160}, {5, 7, 2064}};
    for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i)
        run_shape(shapes[i][0], shapes[i][1], shapes[i][2]);
    puts("oracle sanitizer run ok");
    return 0;
}
