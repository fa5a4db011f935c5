// Measured peaks (include/sq_peaks.h): matrix-core issue rate with no
// memory traffic, HBM read and 2:1 read:write stream rates, and the shader
// clock sustained under each.  Built into its own library; the quantization
// kernels do not use it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sq_peaks.h"

namespace {

typedef int int4v __attribute__((ext_vector_type(4)));
typedef int int8v __attribute__((ext_vector_type(8)));
typedef int int16v __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u4v __attribute__((ext_vector_type(4)));
typedef unsigned int u2v __attribute__((ext_vector_type(2)));

// Clock samples of the first wave of block 0 (lane 0 stores them).
struct Clock {
    uint64_t c0, r0;
    __device__ __forceinline__ void start() {
        c0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
    }
    __device__ __forceinline__ void stop(uint64_t *clk) const {
        const uint64_t c1 = __builtin_amdgcn_s_memtime();
        const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
        if (clk && blockIdx.x == 0 && threadIdx.x == 0) {
            clk[0] = c0;
            clk[1] = c1;
            clk[2] = r0;
            clk[3] = r1;
        }
    }
};

template <bool F8>
__global__ __launch_bounds__(256) void mfma_loop(int iters, int *sink, uint64_t *clk) {
    const int lane = threadIdx.x & 63;
    Clock ck;
    ck.start();
    if constexpr (F8) {
        // mixed e4m3 bit patterns of both signs; bit 3 of each byte cleared so
        // no byte is a NaN code (0x7f, 0xff): every value finite, |v| <= 240
        int8v a, b;
        for (int i = 0; i < 8; ++i) {
            a[i] = (int)(((unsigned)lane * 0x9e3779b1u + (unsigned)i * 0x7f4a7c15u) & 0xf7f7f7f7u);
            b[i] = (int)(((unsigned)lane * 0x85ebca6bu + (unsigned)i * 0xc2b2ae35u) & 0xf7f7f7f7u);
        }
        f32x16 acc[4];
        for (int c = 0; c < 4; ++c)
            for (int v = 0; v < 16; ++v) acc[c][v] = 0.0f;
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 0, 0, 0, 0,
                                                                         0, 0);
        }
        float s = 0.0f;
        for (int c = 0; c < 4; ++c)
            for (int v = 0; v < 16; ++v) s += acc[c][v];
        if (s != s) sink[0] = 1;  // never: finite operands, sums far below overflow
    } else {
        int4v a, b;
        for (int i = 0; i < 4; ++i) {  // mixed int8 bit patterns of both signs
            a[i] = (int)((unsigned)lane * 0x9e3779b1u + (unsigned)i * 0x7f4a7c15u);
            b[i] = (int)((unsigned)lane * 0x85ebca6bu + (unsigned)i * 0xc2b2ae35u);
        }
        int16v acc[4];
        for (int c = 0; c < 4; ++c)
            for (int v = 0; v < 16; ++v) acc[c][v] = c;
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[c], 0, 0, 0);
        }
        int s = 0;
        for (int c = 0; c < 4; ++c)
            for (int v = 0; v < 16; ++v) s ^= acc[c][v];
        if (s == 0x7eadbeef) sink[0] = 1;
    }
    ck.stop(clk);
}

__global__ __launch_bounds__(256) void read_stream(const u4v *__restrict__ x, int64_t n,
                                                   uint32_t *sink, uint64_t *clk) {
    Clock ck;
    ck.start();
    const int64_t stride = (int64_t)gridDim.x * 256 * 4;
    uint32_t f = 0;
    for (int64_t base = (int64_t)blockIdx.x * 256 * 4 + threadIdx.x; base < n; base += stride) {
        u4v v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = base + (int64_t)u * 256;
            v[u] = __builtin_nontemporal_load(x + (i < n ? i : n - 1));
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)  // clamped loads past the end are not folded
            f ^= base + (int64_t)u * 256 < n ? v[u].x ^ v[u].y ^ v[u].z ^ v[u].w : 0u;
    }
    // one word per block: the lanes' folds combined through LDS
    __shared__ uint32_t red[256];
    red[threadIdx.x] = f;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int i = 0; i < 256; ++i) t ^= red[i];
        sink[blockIdx.x] = t;
    }
    ck.stop(clk);
}

template <bool NTS>
__global__ __launch_bounds__(256) void rw_stream(const u4v *__restrict__ x, u2v *__restrict__ y,
                                                 int64_t n, uint64_t *clk) {
    Clock ck;
    ck.start();
    const int64_t stride = (int64_t)gridDim.x * 256 * 8;
    for (int64_t base = (int64_t)blockIdx.x * 256 * 8 + threadIdx.x; base < n; base += stride) {
        u4v v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t i = base + (int64_t)u * 256;
            v[u] = __builtin_nontemporal_load(x + (i < n ? i : n - 1));
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t i = base + (int64_t)u * 256;
            if (i < n) {
                const u2v o = {v[u].x ^ v[u].y, v[u].z ^ v[u].w};
                if constexpr (NTS) __builtin_nontemporal_store(o, y + i);
                else y[i] = o;
            }
        }
    }
    ck.stop(clk);
}

int status() { return (int)hipGetLastError(); }

}  // namespace

extern "C" int sqp_mfma_loop(int fp8, int iters, int blocks, int *sink, uint64_t *clk,
                             void *stream) {
    if (iters < 1 || blocks < 1 || !sink) return (int)hipErrorInvalidValue;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (fp8) mfma_loop<true><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(iters, sink, clk);
    else mfma_loop<false><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(iters, sink, clk);
    return status();
}

extern "C" int sqp_read_stream(const void *x, size_t bytes, int blocks, uint32_t *sink,
                               uint64_t *clk, void *stream) {
    if (!x || !sink || bytes < 16 || bytes % 16 || blocks < 1) return (int)hipErrorInvalidValue;
    read_stream<<<dim3((unsigned)blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream)>>>(
        reinterpret_cast<const u4v *>(x), (int64_t)(bytes / 16), sink, clk);
    return status();
}

extern "C" int sqp_rw_stream(const void *x, size_t bytes, void *y, int blocks, int nt_store,
                             uint64_t *clk, void *stream) {
    if (!x || !y || bytes < 16 || bytes % 16 || blocks < 1) return (int)hipErrorInvalidValue;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const auto *xv = reinterpret_cast<const u4v *>(x);
    auto *yv = reinterpret_cast<u2v *>(y);
    const int64_t n = (int64_t)(bytes / 16);
    if (nt_store) rw_stream<true><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(xv, yv, n, clk);
    else rw_stream<false><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(xv, yv, n, clk);
    return status();
}

extern "C" int sqp_clock_rates(int *wall_khz, int *peak_sclk_khz) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess && wall_khz)
        e = hipDeviceGetAttribute(wall_khz, hipDeviceAttributeWallClockRate, dev);
    if (e == hipSuccess && peak_sclk_khz)
        e = hipDeviceGetAttribute(peak_sclk_khz, hipDeviceAttributeClockRate, dev);
    return (int)e;
}
