// Row-wise int8 quantization with a per-channel multiplier fused into the
// read:  v = fl(x[r, k] * mul[k])  (mul = NULL: v = x), then
//   dynamic:  a = max(max_k |v|, 1e-8), step = fl(a/127),
//             q = clamp(round_half_even(fl(v * fl(127/a))), -127, 127)
//   static:   q = clamp(round_half_even(fl(v * static_scale[1])), -127, 127)
//
// One kernel serves three steps of the path:
//  - weight smoothing + per-output-channel int8 (mul = s; the SmoothQuant
//    tutorial page, SmoothQuant 的原理 and 为什么激活不能用逐通道量化),
//  - fused activation smoothing + per-token / per-tensor int8 (mul = 1/s;
//    X / s of the tbr8.org page §3, folded into the quantizer read),
//  - LLM.int8()'s row quantization with outlier columns zeroed (mul = the
//    0/1 column mask; the xdnf.cn explainer §2.2).  Multiplying by 1.0 is
//    exact and by 0.0 gives +-0, which quantizes to 0, the same as
//    removing the column.
//
// One 64-lane wave per row.  Each lane keeps its 16-byte vectors of the row
// in registers (up to 16 per lane: 8192 16-bit or 4096 fp32 elements), so
// HBM is read once and written once; longer rows re-read from L2.
#include "sq_device.h"
#include "sq_launch.h"

namespace sq {

constexpr int kMaxIt = 16;

template <int DT>
__device__ __forceinline__ void load_mul(const float *__restrict__ mul, int64_t e0, float *m) {
    constexpr int V = Vec<DT>::n;
    const float4 *p = reinterpret_cast<const float4 *>(mul + e0);
#pragma unroll
    for (int i = 0; i < V / 4; ++i) {
        float4 t = p[i];
        m[4 * i] = t.x;
        m[4 * i + 1] = t.y;
        m[4 * i + 2] = t.z;
        m[4 * i + 3] = t.w;
    }
}

template <int DT, bool HAS_MUL>
__device__ __forceinline__ void scaled(const uint4 &raw, const float *__restrict__ mul,
                                       int64_t e0, float *v) {
    constexpr int V = Vec<DT>::n;
    widen16<DT>(raw, v);
    if constexpr (HAS_MUL) {
        float m[V];
        load_mul<DT>(mul, e0, m);
#pragma unroll
        for (int i = 0; i < V; ++i) v[i] = v[i] * m[i];
    }
}

template <int DT>
__device__ __forceinline__ void store_q(int8_t *__restrict__ q, int64_t e0, const float *v,
                                        float inv) {
    if constexpr (Vec<DT>::n == 8) {
        uint2 o;
        o.x = pack4(quant_i8(v[0], inv), quant_i8(v[1], inv), quant_i8(v[2], inv),
                    quant_i8(v[3], inv));
        o.y = pack4(quant_i8(v[4], inv), quant_i8(v[5], inv), quant_i8(v[6], inv),
                    quant_i8(v[7], inv));
        *reinterpret_cast<uint2 *>(q + e0) = o;
    } else {
        *reinterpret_cast<uint32_t *>(q + e0) =
            pack4(quant_i8(v[0], inv), quant_i8(v[1], inv), quant_i8(v[2], inv),
                  quant_i8(v[3], inv));
    }
}

template <int DT, bool HAS_MUL, bool DYN, bool IN_REGS>
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint4 *__restrict__ x,
                                                         int64_t rows, int64_t K,
                                                         const float *__restrict__ mul,
                                                         const float *__restrict__ static_scale,
                                                         int8_t *__restrict__ q,
                                                         float *__restrict__ scale) {
    constexpr int V = Vec<DT>::n;
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (!DYN && blockIdx.x == 0 && threadIdx.x == 0) scale[0] = static_scale[0];
    if (r >= rows) return;
    const int64_t nvec = K / V;
    const uint4 *xr = x + r * nvec;
    int8_t *qr = q + r * K;

    if constexpr (DYN) {
        uint4 buf[IN_REGS ? kMaxIt : 1];
        float a = 0.0f;
        if constexpr (IN_REGS) {
#pragma unroll
            for (int it = 0; it < kMaxIt; ++it) {
                const int64_t vi = lane + (int64_t)it * kWave;
                if (vi < nvec) buf[it] = xr[vi];
            }
#pragma unroll
            for (int it = 0; it < kMaxIt; ++it) {
                const int64_t vi = lane + (int64_t)it * kWave;
                if (vi < nvec) {
                    float v[V];
                    scaled<DT, HAS_MUL>(buf[it], mul, vi * V, v);
#pragma unroll
                    for (int i = 0; i < V; ++i) a = fmaxf(a, fabsf(v[i]));
                }
            }
        } else {
            for (int64_t vi = lane; vi < nvec; vi += kWave) {
                float v[V];
                scaled<DT, HAS_MUL>(xr[vi], mul, vi * V, v);
#pragma unroll
                for (int i = 0; i < V; ++i) a = fmaxf(a, fabsf(v[i]));
            }
        }
        a = wave_max(a);
        if (!(a > 1e-8f)) a = 1e-8f;
        const float inv = 127.0f / a;
        if (lane == 0) scale[r] = a / 127.0f;
        if constexpr (IN_REGS) {
#pragma unroll
            for (int it = 0; it < kMaxIt; ++it) {
                const int64_t vi = lane + (int64_t)it * kWave;
                if (vi < nvec) {
                    float v[V];
                    scaled<DT, HAS_MUL>(buf[it], mul, vi * V, v);
                    store_q<DT>(qr, vi * V, v, inv);
                }
            }
        } else {
            for (int64_t vi = lane; vi < nvec; vi += kWave) {
                float v[V];
                scaled<DT, HAS_MUL>(xr[vi], mul, vi * V, v);
                store_q<DT>(qr, vi * V, v, inv);
            }
        }
    } else {
        const float inv = static_scale[1];
        for (int64_t vi = lane; vi < nvec; vi += kWave) {
            float v[V];
            scaled<DT, HAS_MUL>(xr[vi], mul, vi * V, v);
            store_q<DT>(qr, vi * V, v, inv);
        }
    }
}

template <int DT, bool HAS_MUL, bool DYN>
static void launch_q(const void *x, int64_t rows, int64_t K, const float *mul,
                     const float *static_scale, int8_t *q, float *scale, hipStream_t stream) {
    dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    auto *xv = reinterpret_cast<const uint4 *>(x);
    const bool in_regs = K / Vec<DT>::n <= (int64_t)kMaxIt * kWave;
    if (DYN && in_regs)
        quant_rows_kernel<DT, HAS_MUL, DYN, true>
            <<<grid, block, 0, stream>>>(xv, rows, K, mul, static_scale, q, scale);
    else
        quant_rows_kernel<DT, HAS_MUL, DYN, false>
            <<<grid, block, 0, stream>>>(xv, rows, K, mul, static_scale, q, scale);
}

template <int DT>
static void launch_dt(const void *x, int64_t rows, int64_t K, const float *mul, int dynamic,
                      const float *static_scale, int8_t *q, float *scale, hipStream_t stream) {
    if (mul) {
        if (dynamic) launch_q<DT, true, true>(x, rows, K, mul, static_scale, q, scale, stream);
        else launch_q<DT, true, false>(x, rows, K, mul, static_scale, q, scale, stream);
    } else {
        if (dynamic) launch_q<DT, false, true>(x, rows, K, mul, static_scale, q, scale, stream);
        else launch_q<DT, false, false>(x, rows, K, mul, static_scale, q, scale, stream);
    }
}

void launch_quant_rows(const void *x, int dt, int64_t rows, int64_t K, const float *mul,
                       int dynamic, const float *static_scale, int8_t *q, float *scale,
                       hipStream_t stream) {
    if (rows == 0) {
        if (!dynamic)  // the per-tensor step is still reported
            launch_copy_f32(static_scale, scale, stream);
        return;
    }
    if (dt == F32) launch_dt<F32>(x, rows, K, mul, dynamic, static_scale, q, scale, stream);
    else if (dt == F16) launch_dt<F16>(x, rows, K, mul, dynamic, static_scale, q, scale, stream);
    else launch_dt<BF16>(x, rows, K, mul, dynamic, static_scale, q, scale, stream);
}

}  // namespace sq
