/*
 * CPU ORACLE (test infrastructure only; see sq_oracle.h for the contract,
 * the page citations and the pins).  Written from the pages' definitions,
 * one obvious loop per definition, no blocking or fusion.
 */
#include "sq_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/* ---------------------------------------------------------------- floats */

static uint32_t f32_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}
static float bits_f32(uint32_t u) {
    float f;
    memcpy(&f, &u, 4);
    return f;
}

float orc_f16_to_f32(uint16_t h) {
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    uint32_t e = (h >> 10) & 0x1fu;
    uint32_t m = h & 0x3ffu;
    if (e == 0x1f) return bits_f32(sign | 0x7f800000u | (m << 13)); /* inf/nan */
    if (e != 0) return bits_f32(sign | ((e + 112u) << 23) | (m << 13));
    /* zero or subnormal: m * 2^-24, exact in binary32 */
    float v = (float)m * 5.9604644775390625e-8f;
    return sign ? -v : v;
}

float orc_bf16_to_f32(uint16_t b) { return bits_f32((uint32_t)b << 16); }

uint16_t orc_f32_to_f16(float f) {
    uint32_t x = f32_bits(f);
    uint32_t sign = (x >> 16) & 0x8000u;
    uint32_t ax = x & 0x7fffffffu;
    if (ax > 0x7f800000u) return (uint16_t)(sign | 0x7e00u); /* nan */
    uint32_t E = ax >> 23;                                   /* biased exponent */
    if (E >= 143u) return (uint16_t)(sign | 0x7c00u);        /* >= 2^16: inf */
    if (E >= 113u) {                                         /* f16 normal range */
        uint32_t m = ax & 0x7fffffu;
        uint32_t h = ((E - 112u) << 10) | (m >> 13);
        uint32_t rem = m & 0x1fffu;
        if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h++; /* carry may give inf */
        return (uint16_t)(sign | h);
    }
    if (E < 102u) return (uint16_t)sign; /* below half the smallest subnormal */
    /* f16 subnormal: value / 2^-24 = m * 2^(E - 126), shift in [14, 24] */
    uint32_t m = (ax & 0x7fffffu) | 0x800000u;
    uint32_t shift = 126u - E;
    uint32_t n = m >> shift;
    uint32_t rem = m & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1u);
    if (rem > half || (rem == half && (n & 1u))) n++;
    return (uint16_t)(sign | n);
}

uint16_t orc_f32_to_bf16(float f) {
    uint32_t x = f32_bits(f);
    if ((x & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((x >> 16) | 0x40u);
    uint32_t lsb = (x >> 16) & 1u;
    return (uint16_t)((x + 0x7fffu + lsb) >> 16);
}

static float load_elem(const void *p, int dt, int64_t i) {
    if (dt == ORC_F32) return ((const float *)p)[i];
    if (dt == ORC_F16) return orc_f16_to_f32(((const uint16_t *)p)[i]);
    return orc_bf16_to_f32(((const uint16_t *)p)[i]);
}

static void store_elem(void *p, int dt, int64_t i, float v) {
    if (dt == ORC_F32)
        ((float *)p)[i] = v;
    else if (dt == ORC_F16)
        ((uint16_t *)p)[i] = orc_f32_to_f16(v);
    else
        ((uint16_t *)p)[i] = orc_f32_to_bf16(v);
}

/* Round half to even written from its definition: take the nearest integer,
 * and on an exact .5 tie the even one.  For |v| >= 2^23 every binary32 value
 * is already an integer; below that v - floor(v) is exact. */
float orc_round_half_even(float v) {
    if (!(fabsf(v) < 8388608.0f)) return v;
    float fl = floorf(v);
    float frac = v - fl;
    if (frac > 0.5f) return fl + 1.0f;
    if (frac < 0.5f) return fl;
    /* tie: fl is an integer below 2^23, so its parity is exact */
    return (fmodf(fl, 2.0f) == 0.0f) ? fl : fl + 1.0f;
}

static int8_t clamp_i8(float r) {
    if (r > 127.0f) return 127;
    if (r < -127.0f) return -127;
    return (int8_t)r;
}

/* ------------------------------------------------------------ a1: amax */

void orc_absmax_cols(const void *x, int dt, int64_t rows, int64_t cols,
                     int accumulate, float *amax) {
    /* amax[c] = max over rows of |x[r, c]|, rows visited in order for each
     * column; threads own disjoint column ranges. */
    const int64_t chunk = 256;
#pragma omp parallel for schedule(static)
    for (int64_t c0 = 0; c0 < cols; c0 += chunk) {
        const int64_t c1 = c0 + chunk < cols ? c0 + chunk : cols;
        float m[256];
        for (int64_t c = c0; c < c1; ++c) m[c - c0] = 0.0f;
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t c = c0; c < c1; ++c) {
                float a = fabsf(load_elem(x, dt, r * cols + c));
                if (a > m[c - c0]) m[c - c0] = a;
            }
        for (int64_t c = c0; c < c1; ++c) {
            float v = m[c - c0];
            if (accumulate && amax[c] > v) v = amax[c];
            amax[c] = v;
        }
    }
}

/* ---------------------------------------------------------- a2: scales */

void orc_compute_scales(const float *act_amax, const float *w_amax, int64_t K,
                        float alpha, float *s, float *inv_s, float *static_scale) {
    const double a = (double)alpha;
    for (int64_t j = 0; j < K; ++j) {
        float xc = act_amax[j] > 1e-5f ? act_amax[j] : 1e-5f;
        float wc = w_amax[j] > 1e-5f ? w_amax[j] : 1e-5f;
        double q = pow((double)xc, a) / pow((double)wc, 1.0 - a);
        float sj = (float)q;
        if (!(sj > 1e-5f)) sj = 1e-5f;
        s[j] = sj;
        inv_s[j] = 1.0f / sj;
    }
    if (static_scale) {
        float m = 0.0f;
        for (int64_t j = 0; j < K; ++j) {
            float v = act_amax[j] * inv_s[j];
            if (v > m) m = v;
        }
        if (!(m > 1e-8f)) m = 1e-8f;
        static_scale[0] = m / 127.0f;
        static_scale[1] = 127.0f / m;
    }
}

/* ---------------------------------------------------- a3: weights */

void orc_smooth_weights_f32(const void *w, int dt, int64_t N, int64_t K,
                            const float *s, float *w_smoothed) {
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            float v = load_elem(w, dt, n * K + k);
            w_smoothed[n * K + k] = s ? v * s[k] : v;
        }
}

static void quantize_row(const float *v, int64_t K, int8_t *q, float *step) {
    float a = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        float t = fabsf(v[k]);
        if (t > a) a = t;
    }
    if (!(a > 1e-8f)) a = 1e-8f;
    float inv = 127.0f / a;
    *step = a / 127.0f;
    for (int64_t k = 0; k < K; ++k) q[k] = clamp_i8(orc_round_half_even(v[k] * inv));
}

void orc_quantize_rows_f32(const float *v, int64_t rows, int64_t K, int8_t *q,
                           float *step) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) quantize_row(v + r * K, K, q + r * K, &step[r]);
}

void orc_smooth_weights(const void *w, int dt, int64_t N, int64_t K,
                        const float *s, int8_t *wq, float *w_scale) {
#pragma omp parallel
    {
        float *row = (float *)malloc((size_t)K * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t k = 0; k < K; ++k) {
                float v = load_elem(w, dt, n * K + k);
                row[k] = s ? v * s[k] : v;
            }
            quantize_row(row, K, wq + n * K, &w_scale[n]);
        }
        free(row);
    }
}

void orc_fold_smooth_weights(const void *w, int dt, int64_t N, int64_t K,
                             const float *row_mul, const float *s, int8_t *wq,
                             float *w_scale) {
#pragma omp parallel
    {
        float *row = (float *)malloc((size_t)K * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t k = 0; k < K; ++k) {
                float v = load_elem(w, dt, n * K + k);
                if (row_mul) v = v * row_mul[n];
                row[k] = s ? v * s[k] : v;
            }
            quantize_row(row, K, wq + n * K, &w_scale[n]);
        }
        free(row);
    }
}

/* ------------------------------------------------- a4: activations */

void orc_quantize_act(const void *x, int dt, int64_t M, int64_t K,
                      const float *inv_s, int mode, const float *static_scale,
                      int8_t *xq, float *x_scale) {
    if (mode == ORC_PER_TENSOR_STATIC) x_scale[0] = static_scale[0];
#pragma omp parallel
    {
        float *row = (float *)malloc((size_t)K * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t m = 0; m < M; ++m) {
            for (int64_t k = 0; k < K; ++k) {
                float v = load_elem(x, dt, m * K + k);
                row[k] = inv_s ? v * inv_s[k] : v;
            }
            if (mode == ORC_PER_TOKEN_DYNAMIC) {
                quantize_row(row, K, xq + m * K, &x_scale[m]);
            } else {
                float inv = static_scale[1];
                for (int64_t k = 0; k < K; ++k)
                    xq[m * K + k] = clamp_i8(orc_round_half_even(row[k] * inv));
            }
        }
        free(row);
    }
}

/* ------------------------------------------------------- a5: GEMM */

static int64_t dot_i8(const int8_t *a, const int8_t *b, int64_t K) {
    int64_t acc = 0;
    for (int64_t k = 0; k < K; ++k) acc += (int64_t)a[k] * (int64_t)b[k];
    return acc;
}

static float dequant(int32_t acc, float dx, float dw) {
    float c = dx * dw;
    return (float)acc * c;
}

int64_t orc_gemm_i8_dequant(const int8_t *xq, const int8_t *wq, int64_t M,
                            int64_t N, int64_t K, const float *x_scale,
                            int per_row, const float *w_scale, void *y,
                            int y_dt, int32_t *acc_out) {
    int64_t overflow = 0;
#pragma omp parallel for schedule(static) reduction(+ : overflow)
    for (int64_t m = 0; m < M; ++m) {
        float dx = x_scale[per_row ? m : 0];
        for (int64_t n = 0; n < N; ++n) {
            int64_t a = dot_i8(xq + m * K, wq + n * K, K);
            if (a > INT32_MAX || a < INT32_MIN) overflow++;
            int32_t acc = (int32_t)a;
            if (acc_out) acc_out[m * N + n] = acc;
            if (y) store_elem(y, y_dt, m * N + n, dequant(acc, dx, w_scale[n]));
        }
    }
    return overflow;
}

void orc_gemm_i8_dequant_at(const int8_t *xq, const int8_t *wq, int64_t K,
                            const float *x_scale, int per_row,
                            const float *w_scale, int y_dt, const int64_t *rows,
                            const int64_t *cols, int64_t n, void *y,
                            int32_t *acc) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        int64_t m = rows[i], c = cols[i];
        int32_t a = (int32_t)dot_i8(xq + m * K, wq + c * K, K);
        if (acc) acc[i] = a;
        if (y) store_elem(y, y_dt, i, dequant(a, x_scale[per_row ? m : 0], w_scale[c]));
    }
}

/* ------------------------------------------------ a6: LLM.int8() */

int64_t orc_outlier_columns(const uint16_t *x_f16, int64_t M, int64_t K,
                            float threshold, int32_t *idx) {
    int64_t count = 0;
    for (int64_t j = 0; j < K; ++j) {
        int hit = 0;
        for (int64_t m = 0; m < M && !hit; ++m)
            if (fabsf(orc_f16_to_f32(x_f16[m * K + j])) >= threshold) hit = 1;
        if (hit) idx[count++] = (int32_t)j;
    }
    return count;
}

static float side_sum(const uint16_t *x_f16, const uint16_t *w_f16, int64_t K,
                      int64_t m, int64_t n, const int32_t *idx, int64_t n_idx) {
    float side = 0.0f;
    for (int64_t t = 0; t < n_idx; ++t) {
        int64_t o = idx[t];
        float p = orc_f16_to_f32(x_f16[m * K + o]) * orc_f16_to_f32(w_f16[n * K + o]);
        side = side + p;
    }
    return side;
}

int64_t orc_int8_mixed_matmul(const uint16_t *x_f16, int64_t M, int64_t K,
                              const int8_t *wq, const float *w_scale,
                              const uint16_t *w_f16, int64_t N, float threshold,
                              void *y, int y_dt, int32_t *acc_out,
                              int8_t *xq_out, float *x_scale_out,
                              int32_t *idx_out) {
    int32_t *idx = (int32_t *)malloc((size_t)(K > 0 ? K : 1) * sizeof(int32_t));
    int8_t *xq = (int8_t *)malloc((size_t)(M * K > 0 ? M * K : 1));
    float *xs = (float *)malloc((size_t)(M > 0 ? M : 1) * sizeof(float));
    char *in_o = (char *)calloc((size_t)(K > 0 ? K : 1), 1);
    int64_t n_idx = orc_outlier_columns(x_f16, M, K, threshold, idx);
    for (int64_t t = 0; t < n_idx; ++t) in_o[idx[t]] = 1;

#pragma omp parallel
    {
        float *row = (float *)malloc((size_t)(K > 0 ? K : 1) * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t m = 0; m < M; ++m) {
            for (int64_t k = 0; k < K; ++k)
                row[k] = in_o[k] ? 0.0f : orc_f16_to_f32(x_f16[m * K + k]);
            quantize_row(row, K, xq + m * K, &xs[m]);
        }
        free(row);
    }

#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int32_t acc = (int32_t)dot_i8(xq + m * K, wq + n * K, K);
            if (acc_out) acc_out[m * N + n] = acc;
            float side = side_sum(x_f16, w_f16, K, m, n, idx, n_idx);
            if (y) store_elem(y, y_dt, m * N + n, dequant(acc, xs[m], w_scale[n]) + side);
        }

    if (xq_out) memcpy(xq_out, xq, (size_t)(M * K));
    if (x_scale_out) memcpy(x_scale_out, xs, (size_t)M * sizeof(float));
    if (idx_out) memcpy(idx_out, idx, (size_t)n_idx * sizeof(int32_t));
    free(idx);
    free(xq);
    free(xs);
    free(in_o);
    return n_idx;
}

void orc_int8_mixed_at(const uint16_t *x_f16, int64_t K, const int8_t *xq,
                       const float *x_scale, const int8_t *wq,
                       const float *w_scale, const uint16_t *w_f16,
                       const int32_t *idx, int64_t n_idx, int y_dt,
                       const int64_t *rows, const int64_t *cols, int64_t n,
                       void *y, int32_t *acc) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        int64_t m = rows[i], c = cols[i];
        int32_t a = (int32_t)dot_i8(xq + m * K, wq + c * K, K);
        if (acc) acc[i] = a;
        float side = side_sum(x_f16, w_f16, K, m, c, idx, n_idx);
        if (y) store_elem(y, y_dt, i, dequant(a, x_scale[m], w_scale[c]) + side);
    }
}

/* -------------------------------------------------- fp64 references */

void orc_matmul_f64(const void *x, int xdt, const void *w, int wdt, int64_t M,
                    int64_t N, int64_t K, double *y64) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += (double)load_elem(x, xdt, m * K + k) * (double)load_elem(w, wdt, n * K + k);
            y64[m * N + n] = acc;
        }
}

void orc_smoothed_matmul_f64(const void *x, int xdt, const void *w, int wdt,
                             const float *s, int64_t M, int64_t N, int64_t K,
                             double *ys64) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double xs = (double)load_elem(x, xdt, m * K + k) / (double)s[k];
                double ws = (double)s[k] * (double)load_elem(w, wdt, n * K + k);
                acc += xs * ws;
            }
            ys64[m * N + n] = acc;
        }
}

/* ------------------------------------------- norm folding and fused norm */

void orc_fold_norm(const float *gamma, const float *beta, const float *s,
                   int64_t K, float *gamma_out, float *beta_out) {
    for (int64_t j = 0; j < K; ++j) {
        gamma_out[j] = gamma[j] / s[j];
        if (beta) beta_out[j] = beta[j] / s[j];
    }
}

typedef unsigned __int128 u128;

static double u128_to_double(u128 v) {
    const uint64_t hi = (uint64_t)(v >> 64), lo = (uint64_t)v;
    return (double)hi * 18446744073709551616.0 + (double)lo;
}

static void row_stats(const uint16_t *x, int64_t K, int norm, float eps, float *mu32,
                      float *rstd32) {
    int64_t s1 = 0;
    u128 s2 = 0;
    for (int64_t j = 0; j < K; ++j) {
        /* x * 2^24 is an integer below 2^40: exact in double and in int64 */
        const int64_t xi = (int64_t)((double)orc_f16_to_f32(x[j]) * 16777216.0);
        const uint64_t a = (uint64_t)(xi < 0 ? -xi : xi);
        s1 += xi;
        s2 += (u128)a * a;
    }
    const double kd = (double)K;
    double mu = 0.0, var;
    if (norm == ORC_NORM_LAYER) {
        mu = (double)s1 / (kd * 16777216.0);
        const u128 sq1 = (u128)(s1 < 0 ? -s1 : s1) * (u128)(s1 < 0 ? -s1 : s1);
        const u128 v = (u128)K * s2 - sq1; /* K S2 >= S1^2 (Cauchy-Schwarz) */
        var = u128_to_double(v) / (kd * kd * 281474976710656.0);
    } else {
        var = u128_to_double(s2) / (kd * 281474976710656.0);
    }
    *mu32 = (float)mu;
    *rstd32 = (float)(1.0 / sqrt(var + (double)eps));
}

void orc_norm_stats(const uint16_t *x_f16, int64_t M, int64_t K, int norm,
                    float eps, float *mu, float *rstd) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) row_stats(x_f16 + m * K, K, norm, eps, &mu[m], &rstd[m]);
}

void orc_norm_quantize(const uint16_t *x_f16, int64_t M, int64_t K, int norm,
                       const float *gamma, const float *beta, float eps,
                       int mode, const float *static_scale, int8_t *xq,
                       float *x_scale, float *y_out) {
    if (mode == ORC_PER_TENSOR_STATIC) x_scale[0] = static_scale[0];
#pragma omp parallel
    {
        float *row = (float *)malloc((size_t)K * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t m = 0; m < M; ++m) {
            const uint16_t *x = x_f16 + m * K;
            float mu, rstd;
            row_stats(x, K, norm, eps, &mu, &rstd);
            for (int64_t j = 0; j < K; ++j) {
                const float v = orc_f16_to_f32(x[j]);
                const float n = norm == ORC_NORM_LAYER ? (v - mu) * rstd : v * rstd;
                float y = n * gamma[j];
                if (beta) y = y + beta[j];
                row[j] = y;
            }
            if (y_out) memcpy(y_out + m * K, row, (size_t)K * sizeof(float));
            if (mode == ORC_PER_TOKEN_DYNAMIC) {
                quantize_row(row, K, xq + m * K, &x_scale[m]);
            } else {
                const float inv = static_scale[1];
                for (int64_t j = 0; j < K; ++j)
                    xq[m * K + j] = clamp_i8(orc_round_half_even(row[j] * inv));
            }
        }
        free(row);
    }
}

/* ------------------------------------------------ f4: FP8 (e4m3) */

float orc_fp8_decode(uint8_t b) {
    int e = (b >> 3) & 15, m = b & 7;
    if (e == 15 && m == 7) return NAN;
    float v = e == 0 ? ldexpf((float)m, -9) : ldexpf((float)(8 + m), e - 10);
    return (b & 0x80) ? -v : v;
}

uint8_t orc_fp8_encode(float v) {
    uint8_t sign = signbit(v) ? 0x80 : 0;
    double a = fabs((double)v);
    if (a >= 448.0) return sign | 0x7E;
    /* codes 0 .. 126 increase with their value: find lo with
     * dec(lo) <= a < dec(lo + 1) */
    int lo = 0, hi = 126;
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if ((double)orc_fp8_decode((uint8_t)mid) <= a) lo = mid;
        else hi = mid;
    }
    if ((double)orc_fp8_decode((uint8_t)hi) <= a) lo = hi;
    if (lo == 126) return sign | 126;
    double dl = a - (double)orc_fp8_decode((uint8_t)lo);
    double dh = (double)orc_fp8_decode((uint8_t)(lo + 1)) - a;
    int c = dl < dh ? lo : dh < dl ? lo + 1 : (lo % 2 == 0 ? lo : lo + 1);
    return sign | (uint8_t)c;
}

static uint8_t fp8_clamp_encode(float z) {
    if (z > 448.0f) z = 448.0f;
    if (z < -448.0f) z = -448.0f;
    return orc_fp8_encode(z);
}

static void quantize_row_fp8(const float *v, int64_t K, uint8_t *q, float *step) {
    float a = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        float t = fabsf(v[k]);
        if (t > a) a = t;
    }
    if (!(a > 1e-8f)) a = 1e-8f;
    float inv = 448.0f / a;
    *step = a / 448.0f;
    for (int64_t k = 0; k < K; ++k) q[k] = fp8_clamp_encode(v[k] * inv);
}

void orc_quantize_rows_fp8(const float *v, int64_t rows, int64_t K, uint8_t *q,
                           float *step) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) quantize_row_fp8(v + r * K, K, q + r * K, &step[r]);
}

void orc_smooth_weights_fp8(const void *w, int dt, int64_t N, int64_t K,
                            const float *s, uint8_t *wq, float *w_scale) {
#pragma omp parallel
    {
        float *row = (float *)malloc((size_t)K * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t k = 0; k < K; ++k) {
                float v = load_elem(w, dt, n * K + k);
                row[k] = s ? v * s[k] : v;
            }
            quantize_row_fp8(row, K, wq + n * K, &w_scale[n]);
        }
        free(row);
    }
}

void orc_quantize_act_fp8(const void *x, int dt, int64_t M, int64_t K,
                          const float *inv_s, int mode, const float *static_scale,
                          uint8_t *xq, float *x_scale) {
    if (mode == ORC_PER_TENSOR_STATIC) x_scale[0] = static_scale[0];
#pragma omp parallel
    {
        float *row = (float *)malloc((size_t)K * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t m = 0; m < M; ++m) {
            for (int64_t k = 0; k < K; ++k) {
                float v = load_elem(x, dt, m * K + k);
                row[k] = inv_s ? v * inv_s[k] : v;
            }
            if (mode == ORC_PER_TOKEN_DYNAMIC) {
                quantize_row_fp8(row, K, xq + m * K, &x_scale[m]);
            } else {
                for (int64_t k = 0; k < K; ++k)
                    xq[m * K + k] = fp8_clamp_encode(row[k] * static_scale[1]);
            }
        }
        free(row);
    }
}

void orc_static_scale(const float *act_amax, const float *inv_s, int64_t K,
                      float qmax, float *out) {
    float a = 0.0f;
    for (int64_t j = 0; j < K; ++j) {
        float t = inv_s ? act_amax[j] * inv_s[j] : act_amax[j];
        if (t > a) a = t;
    }
    if (!(a > 1e-8f)) a = 1e-8f;
    out[0] = a / qmax;
    out[1] = qmax / a;
}

/* The 256 decoded values, filled (from orc_fp8_decode) before any
 * parallel region reads them. */
static double fp8_table[256];
static void fp8_table_init(void) {
    for (int i = 0; i < 256; ++i) fp8_table[i] = (double)orc_fp8_decode((uint8_t)i);
}

/* The exact sum of the products in double: every e4m3 product is a multiple
 * of 2^-18 below 2^18, so K <= 2^16 terms need fewer than 53 bits and no
 * addition rounds. */
static double dot_fp8(const uint8_t *a, const uint8_t *b, int64_t K) {
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k) s += fp8_table[a[k]] * fp8_table[b[k]];
    return s;
}

void orc_gemm_fp8_dequant(const uint8_t *xq, const uint8_t *wq, int64_t M, int64_t N,
                          int64_t K, const float *x_scale, int per_row,
                          const float *w_scale, void *y, int y_dt, double *acc_out) {
    fp8_table_init();
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float dx = x_scale[per_row ? m : 0];
        for (int64_t n = 0; n < N; ++n) {
            double acc = dot_fp8(xq + m * K, wq + n * K, K);
            if (acc_out) acc_out[m * N + n] = acc;
            float c = dx * w_scale[n];
            if (y) store_elem(y, y_dt, m * N + n, (float)acc * c);
        }
    }
}

void orc_gemm_fp8_dequant_at(const uint8_t *xq, const uint8_t *wq, int64_t K,
                             const float *x_scale, int per_row, const float *w_scale,
                             int y_dt, const int64_t *rows, const int64_t *cols,
                             int64_t n, void *y, double *acc_out) {
    fp8_table_init();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        int64_t m = rows[i], c = cols[i];
        double acc = dot_fp8(xq + m * K, wq + c * K, K);
        if (acc_out) acc_out[i] = acc;
        float cc = x_scale[per_row ? m : 0] * w_scale[c];
        if (y) store_elem(y, y_dt, i, (float)acc * cc);
    }
}
