// Column reductions and the smoothing-factor kernels.
//
// absmax_cols: per-channel abs-max of a row-major [rows, cols] matrix
// ("x_j = max_i |X_ij|" and the weight-side w_j of the SmoothQuant tutorial
// page, section 缩放因子; the calibration code of the lpnh.cn write-up §3.2).
// Each thread owns one 16-byte column vector and keeps a running max over a
// strided slab of rows; a block folds its row groups through LDS and merges
// into the output with one atomicMax per column on the float bit pattern
// (non-negative floats order like their unsigned bits).  Reads are
// coalesced row segments of 256 bytes to 1 KB; the kernel is HBM-bound.
//
// compute_scales: s_j = max(max(x_j,1e-5)^a / max(w_j,1e-5)^(1-a), 1e-5),
// powers and quotient in double rounded once; inv_s = fl(1/s); optional
// static per-tensor step from max_j fl(x_j * inv_s_j).
#include "sq_device.h"
#include "sq_launch.h"

namespace sq {

__global__ void fill_zero_u32(uint32_t *p, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// Block = 256 / CVB row groups x CVB column vectors: a wave reads 64 / CVB
// row segments of 16 CVB bytes per load, thread (g, c) keeps the max of
// column vector c over rows r0 + g, r0 + g + RG, ... of the block's slab,
// with U loads in flight.
constexpr int kCvb = 16;           // column vectors per block (direct path)
constexpr int kRg = 256 / kCvb;    // row groups per block (direct path)

// DIRECT: one block per column slab covers every row (at most 16 per
// thread), so the block's maxima are the results: stored (or merged with
// the running max) without atomics, and the output needs no zero fill.
template <int DT, bool DIRECT, int CVB = kCvb, int U = 4, bool NTL = true>
__global__ __launch_bounds__(256) void absmax_cols_kernel(const uint4 *__restrict__ x,
                                                          int64_t rows, int64_t cols,
                                                          int64_t rows_per_block,
                                                          uint32_t *__restrict__ out,
                                                          int accumulate) {
    constexpr int V = Vec<DT>::n;
    constexpr int RG = 256 / CVB;
    static_assert(CVB == 16 || CVB == 32 || CVB == 64, "column vectors per block");
    __shared__ float red[RG][CVB * V + 1];
    const int tid = threadIdx.x, c = tid % CVB, g = tid / CVB;
    const int64_t cvec = cols / V;
    const int64_t cv = (int64_t)blockIdx.x * CVB + c;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
    const int64_t r1 = r0 + rows_per_block < rows ? r0 + rows_per_block : rows;

    float m[V];
#pragma unroll
    for (int i = 0; i < V; ++i) m[i] = 0.0f;

    if (cv < cvec) {
        const uint4 *p = x + cv;
        int64_t r = r0 + g;
        for (; r + (U - 1) * RG < r1; r += U * RG) {
            uint4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = ld16<NTL>(p + (r + u * RG) * cvec);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float f[V];
                widen16<DT>(v[u], f);
#pragma unroll
                for (int i = 0; i < V; ++i) m[i] = fmaxf(m[i], fabsf(f[i]));
            }
        }
        for (; r < r1; r += RG) {
            float f[V];
            widen16<DT>(ld16<NTL>(p + r * cvec), f);
#pragma unroll
            for (int i = 0; i < V; ++i) m[i] = fmaxf(m[i], fabsf(f[i]));
        }
    }
#pragma unroll
    for (int i = 0; i < V; ++i) red[g][c * V + i] = m[i];
    __syncthreads();
    for (int t = tid; t < CVB * V; t += 256) {
        float v = red[0][t];
#pragma unroll
        for (int k = 1; k < RG; ++k) v = fmaxf(v, red[k][t]);
        const int64_t col = (int64_t)blockIdx.x * CVB * V + t;  // red[.][c*V + i] = column c*V + i
        if constexpr (DIRECT) {
            if (col < cols) out[col] = __float_as_uint(accumulate ? fmaxf(v, __uint_as_float(out[col])) : v);
        } else {
            if (col < cols && v > 0.0f) atomicMax(&out[col], __float_as_uint(v));
        }
    }
}

void launch_absmax(const void *x, int dt, int64_t rows, int64_t cols, int accumulate,
                   float *amax, hipStream_t stream) {
    if (cols == 0) return;
    auto *out = reinterpret_cast<uint32_t *>(amax);
    auto *xv = reinterpret_cast<const uint4 *>(x);
    const int V = dt == F32 ? 4 : 8;
    const int64_t cvec = cols / V;
    const int64_t bx = (cvec + kCvb - 1) / kCvb;
    if (rows > 0 && rows <= 16 * kRg) {
        // Few rows (the activations of a prefill batch): one block per
        // column slab, direct stores, no fill launch.
        dim3 grid((unsigned)bx, 1), block(256);
        // (At most 256 rows: plain loads, the input may be read again.)
        if (dt == F32)
            absmax_cols_kernel<F32, true, kCvb, 4, false><<<grid, block, 0, stream>>>(
                xv, rows, cols, rows, out, accumulate);
        else if (dt == F16)
            absmax_cols_kernel<F16, true, kCvb, 4, false><<<grid, block, 0, stream>>>(
                xv, rows, cols, rows, out, accumulate);
        else
            absmax_cols_kernel<BF16, true, kCvb, 4, false><<<grid, block, 0, stream>>>(
                xv, rows, cols, rows, out, accumulate);
        return;
    }
    if (!accumulate)
        fill_zero_u32<<<dim3((unsigned)((cols + 255) / 256)), dim3(256), 0, stream>>>(
            reinterpret_cast<uint32_t *>(amax), cols);
    if (rows == 0) return;
    // At most 2048 blocks - one round at 8 blocks per CU, so no block of a
    // second round streams its slab alone at the end - with at least 64
    // rows per block: the blocks of one column slab merge with one
    // atomicMax per column each, so their number is kept small.
    auto shape = [&](int64_t cvb, int64_t &gx, int64_t &gy, int64_t &rpb) {
        gx = (cvec + cvb - 1) / cvb;
        gy = 2048 / gx;
        const int64_t max_by = (rows + 63) / 64;
        if (gy > max_by) gy = max_by;
        if (gy > 65535) gy = 65535;
        if (gy < 1) gy = 1;
        rpb = (rows + gy - 1) / gy;
        gy = (rows + rpb - 1) / rpb;
    };
    // 64 column vectors per block (a wave reads one 1 KB row segment per
    // load) with 8 loads in flight per thread where the rows are at least
    // 64 vectors wide and that still gives at least 1024 blocks: W [28672, 7168] fp16 63-64 us against 69 us with
    // 16 x 4 (four 256-byte segments per wave load).  Smaller inputs keep
    // 16 x 4, whose blocks are four times as many: X [2048, 4096] gets 1024
    // blocks instead of 256 (LLM.int8() outlier detection: 4 us less).
    int64_t gx, gy, rpb;
    shape(64, gx, gy, rpb);
    const bool wide = cvec >= 64 && gx * gy >= 1024;
    if (!wide) shape(kCvb, gx, gy, rpb);
    dim3 grid((unsigned)gx, (unsigned)gy), block(256);
    // Inputs larger than the caches are loaded nontemporally; smaller ones
    // stay cached for the kernel that reads them next (LLM.int8()'s
    // quantizer after its outlier detection: 54.5 -> 52.8 us for the
    // 2048 x 4096 x 4096 call, with the quantizer's loads plain as well).
    const bool ntl = rows * cols * dt_bytes(dt) > kNtLoadBytes;
#define SQ_ABS(DTV)                                                                              \
    do {                                                                                         \
        if (wide && ntl)                                                                         \
            absmax_cols_kernel<DTV, false, 64, 8, true><<<grid, block, 0, stream>>>(             \
                xv, rows, cols, rpb, out, 0);                                                    \
        else if (wide)                                                                           \
            absmax_cols_kernel<DTV, false, 64, 8, false><<<grid, block, 0, stream>>>(            \
                xv, rows, cols, rpb, out, 0);                                                    \
        else if (ntl)                                                                            \
            absmax_cols_kernel<DTV, false, kCvb, 4, true><<<grid, block, 0, stream>>>(           \
                xv, rows, cols, rpb, out, 0);                                                    \
        else                                                                                     \
            absmax_cols_kernel<DTV, false, kCvb, 4, false><<<grid, block, 0, stream>>>(          \
                xv, rows, cols, rpb, out, 0);                                                    \
    } while (0)
    if (dt == F32) SQ_ABS(F32);
    else if (dt == F16) SQ_ABS(F16);
    else SQ_ABS(BF16);
#undef SQ_ABS
}

__global__ __launch_bounds__(256) void scales_kernel(const float *__restrict__ act_amax,
                                                     const float *__restrict__ w_amax,
                                                     int64_t K, double alpha,
                                                     float *__restrict__ s,
                                                     float *__restrict__ inv_s) {
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= K) return;
    const float xc = act_amax[j] > 1e-5f ? act_amax[j] : 1e-5f;
    const float wc = w_amax[j] > 1e-5f ? w_amax[j] : 1e-5f;
    const double q = pow((double)xc, alpha) / pow((double)wc, 1.0 - alpha);
    float sj = (float)q;
    if (!(sj > 1e-5f)) sj = 1e-5f;
    s[j] = sj;
    inv_s[j] = 1.0f / sj;
}

// One block: a = max(max_j fl(x_j * inv_s_j), 1e-8) (inv_s NULL: x_j);
// {a/qmax, qmax/a} (qmax 127 for int8 codes, 448 for e4m3).
__global__ __launch_bounds__(1024) void static_scale_kernel(const float *__restrict__ act_amax,
                                                            const float *__restrict__ inv_s,
                                                            int64_t K, float qmax,
                                                            float *__restrict__ out) {
    __shared__ float red[16];
    float m = 0.0f;
    if (inv_s)
        for (int64_t j = threadIdx.x; j < K; j += 1024) m = fmaxf(m, act_amax[j] * inv_s[j]);
    else
        for (int64_t j = threadIdx.x; j < K; j += 1024) m = fmaxf(m, act_amax[j]);
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float a = red[0];
        for (int i = 1; i < 16; ++i) a = fmaxf(a, red[i]);
        if (!(a > 1e-8f)) a = 1e-8f;
        out[0] = a / qmax;
        out[1] = qmax / a;
    }
}

void launch_compute_scales(const float *act_amax, const float *w_amax, int64_t K, float alpha,
                           float *s, float *inv_s, float *static_scale, hipStream_t stream) {
    if (K > 0)
        scales_kernel<<<dim3((unsigned)((K + 255) / 256)), dim3(256), 0, stream>>>(
            act_amax, w_amax, K, (double)alpha, s, inv_s);
    if (static_scale)
        static_scale_kernel<<<dim3(1), dim3(1024), 0, stream>>>(act_amax, inv_s, K, 127.0f,
                                                                 static_scale);
}

void launch_static_scale(const float *act_amax, const float *inv_s, int64_t K, float qmax,
                         float *out, hipStream_t stream) {
    static_scale_kernel<<<dim3(1), dim3(1024), 0, stream>>>(act_amax, inv_s, K, qmax, out);
}

__global__ void copy_f32_kernel(const float *src, float *dst) { *dst = *src; }

void launch_copy_f32(const float *src, float *dst, hipStream_t stream) {
    copy_f32_kernel<<<dim3(1), dim3(1), 0, stream>>>(src, dst);
}

}  // namespace sq
