// C ABI of the library (include/sq.h): argument validation on the host,
// then kernel launches on the caller's stream.  No allocation, no
// synchronization, no state besides the kernels themselves.
#include "../../include/sq.h"
#include "../../include/sq_test.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>

#include "sq_launch.h"

namespace {

inline bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }
inline size_t esize(int dt) { return dt == SQ_F32 ? 4 : 2; }
inline bool valid_dt(int dt) { return dt == SQ_F32 || dt == SQ_F16 || dt == SQ_BF16; }
inline hipStream_t st(void *s) { return reinterpret_cast<hipStream_t>(s); }
constexpr int64_t kMaxDim = 0x7fffffff;

int finish() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? SQ_OK : SQ_ERR_HIP;
}

inline size_t round256(size_t b) { return (b + 255) & ~size_t(255); }

struct MixedWs {
    size_t xq, xs, colmax, mask, idx, count, xo, wo, total;
    int cap;  // outlier columns the compact side operands hold
};

// Device memory for sq_int8_mixed_matmul_noalloc: one array per GPU, held
// until the process ends.  Its name is a host-side stand-in for the device
// symbol: host code uses only the per-device address that
// hipGetSymbolAddress returns for it (scratch_ptr below).
static __device__ __align__(256) char scratch[SQ_MIXED_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_dev[kMaxDevices];  // per-device address of `scratch`, once looked up

// The current device's address of `scratch` (looked up once per device with
// that device current), or null with *err set on failure.
void *scratch_ptr(int *err) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *err = SQ_ERR_HIP;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_dev[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            *err = SQ_ERR_HIP;
            return nullptr;
        }
        scratch_dev[dev] = ptr;
    }
    return scratch_dev[dev];
}

static_assert(SQ_MIXED_SIDE_COLS <= sq::kSideColsMax, "side operand columns");

MixedWs mixed_layout(int64_t M, int64_t N, int64_t K) {
    MixedWs w{};
    w.cap = (int)(K < SQ_MIXED_SIDE_COLS ? K : SQ_MIXED_SIDE_COLS);
    size_t off = 0;
    w.xq = off; off += round256((size_t)M * (size_t)K);
    w.xs = off; off += round256((size_t)M * 4);
    w.colmax = off; off += round256((size_t)K * 4);
    w.mask = off; off += round256((size_t)K * 4);
    w.idx = off; off += round256((size_t)K * 4);
    w.count = off; off += 256;
    w.xo = off; off += round256((size_t)w.cap * (size_t)M * 4);
    w.wo = off; off += round256((size_t)w.cap * (size_t)N * 4);
    w.total = off;
    return w;
}

}  // namespace

extern "C" {

const char *sq_status_str(int status) {
    switch (status) {
        case SQ_OK: return "SQ_OK";
        case SQ_ERR_NULL: return "SQ_ERR_NULL: a required pointer is NULL";
        case SQ_ERR_SHAPE: return "SQ_ERR_SHAPE: negative size or unsupported divisibility";
        case SQ_ERR_DTYPE: return "SQ_ERR_DTYPE: element type not allowed";
        case SQ_ERR_ALIGN: return "SQ_ERR_ALIGN: pointer not 16-byte aligned";
        case SQ_ERR_ARG: return "SQ_ERR_ARG: invalid scalar argument";
        case SQ_ERR_WORKSPACE: return "SQ_ERR_WORKSPACE: workspace missing or too small";
        case SQ_ERR_UNSUPPORTED: return "SQ_ERR_UNSUPPORTED: combination not implemented";
        case SQ_ERR_HIP: return "SQ_ERR_HIP: the HIP runtime reported an error";
        default: return "unknown sq_status";
    }
}

int sq_version(void) { return 103; }

int sq_absmax_reduce(const void *x, int dt, int64_t rows, int64_t cols, int accumulate,
                     float *amax_out, void *stream) {
    if (!valid_dt(dt)) return SQ_ERR_DTYPE;
    if (rows < 0 || cols < 0 || rows > kMaxDim || cols > kMaxDim) return SQ_ERR_SHAPE;
    if ((cols * (int64_t)esize(dt)) % 16 != 0) return SQ_ERR_SHAPE;
    if (cols == 0) return SQ_OK;
    if (!amax_out || (rows > 0 && !x)) return SQ_ERR_NULL;
    if (!aligned(x, 16) || !aligned(amax_out, 4)) return SQ_ERR_ALIGN;
    sq::launch_absmax(x, dt, rows, cols, accumulate, amax_out, st(stream));
    return finish();
}

int sq_compute_scales(const float *act_amax, const float *w_amax, int64_t K, float alpha,
                      float *s, float *inv_s, float *static_scale, void *stream) {
    if (K < 0 || K > kMaxDim) return SQ_ERR_SHAPE;
    if (!(alpha >= 0.0f && alpha <= 1.0f)) return SQ_ERR_ARG;
    if (K > 0 && (!act_amax || !w_amax || !s || !inv_s)) return SQ_ERR_NULL;
    if (!aligned(act_amax, 4) || !aligned(w_amax, 4) || !aligned(s, 4) || !aligned(inv_s, 4) ||
        !aligned(static_scale, 4))
        return SQ_ERR_ALIGN;
    if (K == 0 && !static_scale) return SQ_OK;
    sq::launch_compute_scales(act_amax, w_amax, K, alpha, s, inv_s, static_scale, st(stream));
    return finish();
}

int sq_smooth_weights(const void *w, int dt, int64_t N, int64_t K, const float *s, int8_t *wq,
                      float *w_scale, void *stream) {
    if (!valid_dt(dt)) return SQ_ERR_DTYPE;
    if (N < 0 || K < 0 || N > kMaxDim || K > kMaxDim || K % 16 != 0) return SQ_ERR_SHAPE;
    if (N == 0) return SQ_OK;
    if (K == 0) return SQ_ERR_SHAPE;  // rows of no elements are rejected
    if (!w_scale || !w || !wq) return SQ_ERR_NULL;
    if (!aligned(w, 16) || !aligned(wq, 16) || !aligned(s, 16) || !aligned(w_scale, 4))
        return SQ_ERR_ALIGN;
    sq::launch_quant_rows(w, dt, N, K, s, 1, nullptr, wq, w_scale, st(stream));
    return finish();
}

int sq_smooth_weights_folded(const void *w, int dt, int64_t N, int64_t K, const float *row_mul,
                             const float *s, int8_t *wq, float *w_scale, void *stream) {
    if (!valid_dt(dt)) return SQ_ERR_DTYPE;
    if (N < 0 || K < 0 || N > kMaxDim || K > kMaxDim || K % 16 != 0) return SQ_ERR_SHAPE;
    if (N == 0) return SQ_OK;
    if (K == 0) return SQ_ERR_SHAPE;  // rows of no elements are rejected
    if (!w_scale || !w || !wq) return SQ_ERR_NULL;
    if (!aligned(w, 16) || !aligned(wq, 16) || !aligned(s, 16) || !aligned(row_mul, 4) ||
        !aligned(w_scale, 4))
        return SQ_ERR_ALIGN;
    sq::launch_quant_rows(w, dt, N, K, s, 1, nullptr, wq, w_scale, st(stream), row_mul);
    return finish();
}

int sq_smooth_weights_fp8(const void *w, int dt, int64_t N, int64_t K, const float *s,
                          uint8_t *wq, float *w_scale, void *stream) {
    if (!valid_dt(dt)) return SQ_ERR_DTYPE;
    if (N < 0 || K < 0 || N > kMaxDim || K > kMaxDim || K % 16 != 0) return SQ_ERR_SHAPE;
    if (N == 0) return SQ_OK;
    if (K == 0) return SQ_ERR_SHAPE;  // rows of no elements are rejected
    if (!w_scale || !w || !wq) return SQ_ERR_NULL;
    if (!aligned(w, 16) || !aligned(wq, 16) || !aligned(s, 16) || !aligned(w_scale, 4))
        return SQ_ERR_ALIGN;
    sq::launch_quant_rows_fp8(w, dt, N, K, s, 1, nullptr, wq, w_scale, st(stream));
    return finish();
}

int sq_quantize_act_fp8(const void *x, int dt, int64_t M, int64_t K, const float *inv_s,
                        int mode, const float *static_scale, uint8_t *xq, float *x_scale,
                        void *stream) {
    if (!valid_dt(dt)) return SQ_ERR_DTYPE;
    if (mode != SQ_PER_TENSOR_STATIC && mode != SQ_PER_TOKEN_DYNAMIC) return SQ_ERR_ARG;
    if (M < 0 || K < 0 || M > kMaxDim || K > kMaxDim || K % 16 != 0) return SQ_ERR_SHAPE;
    if (M == 0 && mode == SQ_PER_TOKEN_DYNAMIC) return SQ_OK;
    if (M > 0 && K == 0) return SQ_ERR_SHAPE;  // rows of no elements are rejected
    if (!x_scale || (mode == SQ_PER_TENSOR_STATIC && !static_scale)) return SQ_ERR_NULL;
    if (M > 0 && (!x || !xq)) return SQ_ERR_NULL;
    if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(inv_s, 16) || !aligned(x_scale, 4) ||
        !aligned(static_scale, 4))
        return SQ_ERR_ALIGN;
    sq::launch_quant_rows_fp8(x, dt, M, K, inv_s, mode == SQ_PER_TOKEN_DYNAMIC, static_scale, xq,
                              x_scale, st(stream));
    return finish();
}

int sq_static_scale(const float *act_amax, const float *inv_s, int64_t K, float qmax,
                    float *static_scale, void *stream) {
    if (!(qmax > 0.0f) || !(qmax < 3.0e38f)) return SQ_ERR_ARG;
    if (K < 0 || K > kMaxDim) return SQ_ERR_SHAPE;
    if (!static_scale || (K > 0 && !act_amax)) return SQ_ERR_NULL;
    if (!aligned(act_amax, 4) || !aligned(inv_s, 4) || !aligned(static_scale, 4))
        return SQ_ERR_ALIGN;
    sq::launch_static_scale(act_amax, inv_s, K, qmax, static_scale, st(stream));
    return finish();
}

int sq_quantize_act(const void *x, int dt, int64_t M, int64_t K, const float *inv_s, int mode,
                    const float *static_scale, int8_t *xq, float *x_scale, void *stream) {
    if (!valid_dt(dt)) return SQ_ERR_DTYPE;
    if (mode != SQ_PER_TENSOR_STATIC && mode != SQ_PER_TOKEN_DYNAMIC) return SQ_ERR_ARG;
    if (M < 0 || K < 0 || M > kMaxDim || K > kMaxDim || K % 16 != 0) return SQ_ERR_SHAPE;
    if (M == 0 && mode == SQ_PER_TOKEN_DYNAMIC) return SQ_OK;  // no rows, no steps
    if (M > 0 && K == 0) return SQ_ERR_SHAPE;  // rows of no elements are rejected
    if (!x_scale || (mode == SQ_PER_TENSOR_STATIC && !static_scale)) return SQ_ERR_NULL;
    if (M > 0 && (!x || !xq)) return SQ_ERR_NULL;
    if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(inv_s, 16) || !aligned(x_scale, 4) ||
        !aligned(static_scale, 4))
        return SQ_ERR_ALIGN;
    sq::launch_quant_rows(x, dt, M, K, inv_s, mode == SQ_PER_TOKEN_DYNAMIC, static_scale, xq,
                          x_scale, st(stream));
    return finish();
}

int sq_gemm_i8_dequant_tile(const int8_t *xq, const int8_t *wq, int64_t M, int64_t N, int64_t K,
                            const float *x_scale, int x_scale_per_row, const float *w_scale,
                            void *y, int y_dt, int32_t *acc_out, void *stream, int tile) {
    if (tile < -1 || tile > 3) return SQ_ERR_ARG;
    if (!valid_dt(y_dt)) return SQ_ERR_DTYPE;
    if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim || K % 16 != 0)
        return SQ_ERR_SHAPE;
    if (K > 133143) return SQ_ERR_UNSUPPORTED;  // 127*127*K must fit int32
    if (M == 0 || N == 0) return SQ_OK;
    if (K == 0) return SQ_ERR_SHAPE;  // an empty inner dimension
    if (!x_scale || !w_scale || !y || !xq || !wq) return SQ_ERR_NULL;
    if (!aligned(xq, 16) || !aligned(wq, 16) || !aligned(x_scale, 4) || !aligned(w_scale, 4) ||
        !aligned(y, esize(y_dt)) || !aligned(acc_out, 4))
        return SQ_ERR_ALIGN;
    sq::launch_gemm(xq, wq, M, N, K, x_scale, x_scale_per_row ? 1 : 0, w_scale, y, y_dt,
                    acc_out, nullptr, st(stream), tile);
    return finish();
}

int sq_gemm_i8_dequant(const int8_t *xq, const int8_t *wq, int64_t M, int64_t N, int64_t K,
                       const float *x_scale, int x_scale_per_row, const float *w_scale, void *y,
                       int y_dt, int32_t *acc_out, void *stream) {
    return sq_gemm_i8_dequant_tile(xq, wq, M, N, K, x_scale, x_scale_per_row, w_scale, y, y_dt,
                                   acc_out, stream, -1);
}

int sq_gemm_fp8_dequant_tile(const uint8_t *xq, const uint8_t *wq, int64_t M, int64_t N,
                             int64_t K, const float *x_scale, int x_scale_per_row,
                             const float *w_scale, void *y, int y_dt, void *stream, int tile) {
    if (tile < -1 || tile > 2) return SQ_ERR_ARG;
    if (!valid_dt(y_dt)) return SQ_ERR_DTYPE;
    if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim || K % 128 != 0)
        return SQ_ERR_SHAPE;
    if (M == 0 || N == 0) return SQ_OK;
    if (K == 0) return SQ_ERR_SHAPE;
    if (!x_scale || !w_scale || !y || !xq || !wq) return SQ_ERR_NULL;
    if (!aligned(xq, 16) || !aligned(wq, 16) || !aligned(x_scale, 4) || !aligned(w_scale, 4) ||
        !aligned(y, esize(y_dt)))
        return SQ_ERR_ALIGN;
    sq::launch_gemm_fp8(xq, wq, M, N, K, x_scale, x_scale_per_row ? 1 : 0, w_scale, y, y_dt,
                        st(stream), tile);
    return finish();
}

int sq_gemm_fp8_dequant(const uint8_t *xq, const uint8_t *wq, int64_t M, int64_t N, int64_t K,
                        const float *x_scale, int x_scale_per_row, const float *w_scale,
                        void *y, int y_dt, void *stream) {
    return sq_gemm_fp8_dequant_tile(xq, wq, M, N, K, x_scale, x_scale_per_row, w_scale, y, y_dt,
                                    stream, -1);
}

int sq_fold_norm(const float *gamma, const float *beta, const float *s, int64_t K,
                 float *gamma_out, float *beta_out, void *stream) {
    if (K < 0 || K > kMaxDim) return SQ_ERR_SHAPE;
    if (K == 0) return SQ_OK;
    if (!gamma || !s || !gamma_out || (beta && !beta_out)) return SQ_ERR_NULL;
    if (!aligned(gamma, 4) || !aligned(beta, 4) || !aligned(s, 4) || !aligned(gamma_out, 4) ||
        !aligned(beta_out, 4))
        return SQ_ERR_ALIGN;
    sq::launch_fold_norm(gamma, beta, s, K, gamma_out, beta ? beta_out : nullptr, st(stream));
    return finish();
}

int sq_norm_quantize_act(const void *x, int dt, int64_t M, int64_t K, int norm,
                         const float *gamma, const float *beta, float eps, int mode,
                         const float *static_scale, int8_t *xq, float *x_scale, void *stream) {
    return sq_norm_quantize_act_kernel(x, dt, M, K, norm, gamma, beta, eps, mode, static_scale,
                                       xq, x_scale, stream, -1);
}

int sq_norm_quantize_act_kernel(const void *x, int dt, int64_t M, int64_t K, int norm,
                                const float *gamma, const float *beta, float eps, int mode,
                                const float *static_scale, int8_t *xq, float *x_scale,
                                void *stream, int kernel) {
    if (kernel < -1 || kernel > 1) return SQ_ERR_ARG;
    if (dt != SQ_F16) return SQ_ERR_DTYPE;
    if (norm != SQ_NORM_LAYER && norm != SQ_NORM_RMS) return SQ_ERR_ARG;
    if (mode != SQ_PER_TENSOR_STATIC && mode != SQ_PER_TOKEN_DYNAMIC) return SQ_ERR_ARG;
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return SQ_ERR_ARG;
    if (M < 0 || K < 0 || M > kMaxDim || K > kMaxDim || K % 16 != 0) return SQ_ERR_SHAPE;
    if (M > 0 && K == 0) return SQ_ERR_SHAPE;  // the mean of an empty row is undefined
    if (K > 16384) return SQ_ERR_UNSUPPORTED;
    if (M == 0 && mode == SQ_PER_TOKEN_DYNAMIC) return SQ_OK;  // no rows, no steps
    if (!x_scale || (mode == SQ_PER_TENSOR_STATIC && !static_scale)) return SQ_ERR_NULL;
    if (M == 0) {  // the per-tensor step is still reported
        if (!aligned(x_scale, 4) || !aligned(static_scale, 4)) return SQ_ERR_ALIGN;
        sq::launch_copy_f32(static_scale, x_scale, st(stream));
        return finish();
    }
    if (!x || !xq || !gamma) return SQ_ERR_NULL;
    if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(gamma, 16) || !aligned(beta, 16) ||
        !aligned(x_scale, 4) || !aligned(static_scale, 4))
        return SQ_ERR_ALIGN;
    sq::launch_norm_quant(x, M, K, norm, gamma, beta, eps, mode == SQ_PER_TOKEN_DYNAMIC,
                          static_scale, xq, x_scale, st(stream), kernel);
    return finish();
}

size_t sq_int8_mixed_matmul_workspace(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0) return 0;
    return mixed_layout(M, N, K).total;
}

}  // extern "C"

namespace {

// Arguments checked except the workspace; runs the three steps of the
// decomposition with their buffers in `ws` (laid out by mixed_layout).
int mixed_checked(const void *x, int64_t M, int64_t K, const int8_t *wq, const float *w_scale,
                  const void *w_f16, int64_t N, float threshold, char *ws, void *y, int y_dt,
                  int32_t *acc_out, int32_t *n_outliers_out, hipStream_t s, int tile) {
    const MixedWs L = mixed_layout(M, N, K);
    auto *xq = reinterpret_cast<int8_t *>(ws + L.xq);
    auto *xs = reinterpret_cast<float *>(ws + L.xs);
    auto *colmax = reinterpret_cast<float *>(ws + L.colmax);
    auto *mask = reinterpret_cast<float *>(ws + L.mask);
    auto *idx = reinterpret_cast<int32_t *>(ws + L.idx);
    auto *count = reinterpret_cast<int32_t *>(ws + L.count);
    auto *xo = reinterpret_cast<float *>(ws + L.xo);
    auto *wo = reinterpret_cast<float *>(ws + L.wo);
    // column abs-max, then the masked row quantizer; extra blocks of that
    // launch write the mask, the outlier list, |O| and (|O| <= cap) the
    // outlier columns of x and w, gathered once for the GEMM's side term
    sq::launch_absmax(x, SQ_F16, M, K, 0, colmax, s);
    sq::OutlierList ol{};
    ol.on = 1; ol.thr = threshold; ol.mask = mask; ol.idx = idx; ol.count = count;
    ol.count_out = n_outliers_out; ol.w16 = static_cast<const uint16_t *>(w_f16);
    ol.M = M; ol.N = N; ol.xo = xo; ol.wo = wo; ol.cap = L.cap;
    sq::launch_quant_rows(x, SQ_F16, M, K, colmax, 1, nullptr, xq, xs, s, nullptr, &ol);
    const sq::SideTerm side{static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(w_f16),
                            idx, count, xo, wo, L.cap};
    sq::launch_gemm(xq, wq, M, N, K, xs, 1, w_scale, y, y_dt, acc_out, &side, s, tile);
    return finish();
}

// The checks both LLM.int8() entry points share (all but the workspace).
int mixed_args(const void *x, int64_t M, int64_t K, const int8_t *wq, const float *w_scale,
               const void *w_f16, int64_t N, float threshold, void *y, int y_dt,
               int32_t *acc_out, int32_t *n_outliers_out, bool *nothing) {
    *nothing = false;
    if (!valid_dt(y_dt)) return SQ_ERR_DTYPE;
    if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim || K % 16 != 0)
        return SQ_ERR_SHAPE;
    if (K > 133143) return SQ_ERR_UNSUPPORTED;
    if (!(threshold > 0.0f)) return SQ_ERR_ARG;  // also rejects NaN
    if (M == 0 || N == 0) {
        *nothing = true;
        return SQ_OK;
    }
    if (K == 0) return SQ_ERR_SHAPE;  // an empty inner dimension
    if (!x || !wq || !w_scale || !w_f16 || !y) return SQ_ERR_NULL;
    if (!aligned(x, 16) || !aligned(wq, 16) || !aligned(w_f16, 16) || !aligned(w_scale, 4) ||
        !aligned(y, esize(y_dt)) || !aligned(acc_out, 4) || !aligned(n_outliers_out, 4))
        return SQ_ERR_ALIGN;
    return SQ_OK;
}

}  // namespace

extern "C" {

int sq_int8_mixed_matmul_tile(const void *x, int64_t M, int64_t K, const int8_t *wq,
                              const float *w_scale, const void *w_f16, int64_t N,
                              float threshold, void *workspace, size_t workspace_bytes, void *y,
                              int y_dt, int32_t *acc_out, int32_t *n_outliers_out, void *stream,
                              int tile) {
    if (tile < -1 || tile > 2) return SQ_ERR_ARG;
    bool nothing = false;
    int st_ = mixed_args(x, M, K, wq, w_scale, w_f16, N, threshold, y, y_dt, acc_out,
                         n_outliers_out, &nothing);
    if (st_ != SQ_OK || nothing) return st_;
    if (!workspace || workspace_bytes < mixed_layout(M, N, K).total) return SQ_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return SQ_ERR_ALIGN;
    return mixed_checked(x, M, K, wq, w_scale, w_f16, N, threshold,
                         static_cast<char *>(workspace), y, y_dt, acc_out, n_outliers_out,
                         st(stream), tile);
}

int sq_int8_mixed_matmul(const void *x, int64_t M, int64_t K, const int8_t *wq,
                         const float *w_scale, const void *w_f16, int64_t N, float threshold,
                         void *workspace, size_t workspace_bytes, void *y, int y_dt,
                         int32_t *acc_out, int32_t *n_outliers_out, void *stream) {
    return sq_int8_mixed_matmul_tile(x, M, K, wq, w_scale, w_f16, N, threshold, workspace,
                                     workspace_bytes, y, y_dt, acc_out, n_outliers_out, stream,
                                     -1);
}

int sq_int8_mixed_matmul_noalloc(const void *x, int64_t M, int64_t K, const int8_t *wq,
                                 const float *w_scale, const void *w_f16, int64_t N,
                                 float threshold, void *y, int y_dt, int32_t *acc_out,
                                 int32_t *n_outliers_out, void *stream) {
    bool nothing = false;
    int st_ = mixed_args(x, M, K, wq, w_scale, w_f16, N, threshold, y, y_dt, acc_out,
                         n_outliers_out, &nothing);
    if (st_ != SQ_OK || nothing) return st_;
    if (mixed_layout(M, N, K).total > (size_t)SQ_MIXED_SCRATCH_BYTES) return SQ_ERR_WORKSPACE;
    int err = SQ_OK;
    void *ws = scratch_ptr(&err);
    if (!ws) return err;
    return mixed_checked(x, M, K, wq, w_scale, w_f16, N, threshold, static_cast<char *>(ws), y,
                         y_dt, acc_out, n_outliers_out, st(stream), -1);
}

}  // extern "C"
