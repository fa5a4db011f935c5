// Folding the smoothing into the preceding norm, and the fused norm -> int8
// quantizer (the SmoothQuant tutorial page, section 融入 LayerNorm: the norm
// y_j = (x_j - mu) / sigma * gamma_j + beta_j with gamma'_j = gamma_j / s_j,
// beta'_j = beta_j / s_j emits the smoothed activation y_j / s_j, so the
// activation quantizer needs no multiply by 1/s and the residual row is read
// once).
//
// Row statistics are exact.  An fp16 value times 2^24 is an integer below
// 2^40 (subnormals included), so S1 = sum x 2^24 fits int64 and
// S2 = sum (x 2^24)^2 fits 128 bits, and both are independent of the order
// in which the block adds them up (K <= 16384).  From them, in double:
//   layer norm: mu = S1 / (K 2^24), sigma^2 = (K S2 - S1^2) / (K^2 2^48)
//   RMS norm:   mu = 0,             sigma^2 = S2 / (K 2^48)
//   rstd = 1 / sqrt(sigma^2 + eps)
// (double division and square root are correctly rounded), then mu and rstd
// are rounded to fp32.  The 128-bit integers become doubles as
// fl(hi 2^64 + fl(lo)).
#include <type_traits>

#include "sq_device.h"
#include "sq_launch.h"

namespace sq {

typedef unsigned __int128 u128;

__global__ void fold_norm_kernel(const float *__restrict__ gamma, const float *__restrict__ beta,
                                 const float *__restrict__ s, int64_t K,
                                 float *__restrict__ gamma_out, float *__restrict__ beta_out) {
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= K) return;
    const float sj = s[j];
    const float g = gamma[j];
    const float b = beta ? beta[j] : 0.0f;
    gamma_out[j] = g / sj;
    if (beta) beta_out[j] = b / sj;
}

// fp16 bits -> |x| 2^24 (exact integer) and its sign.
__device__ __forceinline__ uint64_t f16_fixed_mag(uint32_t h) {
    const uint32_t e = (h >> 10) & 31u, m = h & 1023u;
    return e ? (uint64_t)(1024u | m) << (e - 1) : (uint64_t)m;
}

__device__ __forceinline__ double u128_to_double(u128 v) {
    const uint64_t hi = (uint64_t)(v >> 64), lo = (uint64_t)v;
    return (double)hi * 18446744073709551616.0 + (double)lo;
}

// mu and rstd (fp32) from the exact row sums (see the file comment).
template <int NORM>
__device__ __forceinline__ void norm_stats(int64_t S1, u128 S2, int64_t K, float eps, float &mu,
                                           float &rstd) {
    const double kd = (double)K;
    double var;
    mu = 0.0f;
    if constexpr (NORM == 0) {
        mu = (float)((double)S1 / (kd * 16777216.0));
        const uint64_t a1 = (uint64_t)(S1 < 0 ? -S1 : S1);
        const u128 v = (u128)(uint64_t)K * S2 - (u128)a1 * a1;  // >= 0 (Cauchy-Schwarz)
        var = u128_to_double(v) / (kd * kd * 281474976710656.0);
    } else {
        var = u128_to_double(S2) / (kd * 281474976710656.0);
    }
    rstd = (float)(1.0 / sqrt(var + (double)eps));
}

// A 256-thread block per row, walking rows_per_block consecutive rows; ITS
// 16-byte vectors (8 fp16) per thread.  Every load is unconditional, with
// out-of-range vector indices clamped to the row's last vector (loaded, not
// used): a load under a lane-divergent branch would wait for all earlier
// memory operations.  The row's sums and maximum are combined across the 4
// waves through LDS slots that alternate between consecutive rows, so one
// barrier per reduction suffices.  The ALU work of the exact sums (a 128-bit
// multiply-add per element), not HBM, bounds the kernel on long streams.
template <int ITS, int NORM, bool HAS_BETA, bool DYN>
__global__ __launch_bounds__(256) void norm_quant_kernel(const uint4 *__restrict__ x,
                                                         int64_t rows, int64_t K,
                                                         const float *__restrict__ gamma,
                                                         const float *__restrict__ beta,
                                                         float eps,
                                                         const float *__restrict__ static_scale,
                                                         int8_t *__restrict__ q,
                                                         float *__restrict__ scale,
                                                         int rows_per_block) {
    __shared__ int64_t sh_s1[2][4];
    __shared__ uint64_t sh_lo[2][4], sh_hi[2][4];
    __shared__ float sh_max[2][4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (!DYN && blockIdx.x == 0 && tid == 0) scale[0] = static_scale[0];
    const int64_t nvec = K / 8;

    // gamma / beta of this thread's vectors: loaded once for all the
    // block's rows.
    float4 g[ITS][2], b[HAS_BETA ? ITS : 1][2];
#pragma unroll
    for (int it = 0; it < ITS; ++it) {
        const int64_t vi = tid + (int64_t)it * 256;
        const int64_t vc = vi < nvec ? vi : nvec - 1;
        const float4 *gp = reinterpret_cast<const float4 *>(gamma + vc * 8);
        g[it][0] = gp[0];
        g[it][1] = gp[1];
        if constexpr (HAS_BETA) {
            const float4 *bp = reinterpret_cast<const float4 *>(beta + vc * 8);
            b[it][0] = bp[0];
            b[it][1] = bp[1];
        }
    }
    auto load_row = [&](int64_t r, uint4 (&raw)[ITS]) {
        const uint4 *xr = x + r * nvec;
#pragma unroll
        for (int it = 0; it < ITS; ++it) {
            const int64_t vi = tid + (int64_t)it * 256;
            raw[it] = ld_nt(xr + (vi < nvec ? vi : nvec - 1));
        }
    };
    // Rows are handled in pairs from two register buffers: the next row's
    // loads are issued before this row is processed (and before its
    // stores), and each buffer's wait covers only its own loads.  The LDS
    // slots alternate with the buffer, so one barrier per reduction
    // suffices: a wave can overwrite a slot only two rows later, after a
    // barrier every wave reaches once it has read the slot.
    auto process = [&](int64_t r, const uint4 (&raw)[ITS], auto par_c) {
        constexpr int PAR = decltype(par_c)::value;
        // Exact row sums.  sum x in double: every term is a multiple of 2^-24
        // and |sum| < 16384 * 65504 < 2^30, so no partial sum ever rounds.
        // sum (x 2^24)^2 = sum M^2 2^(2s) (x 2^24 = M 2^s, M the 11-bit
        // significand, a term < 2^80) is kept as two carry-free 64-bit sums of
        // the term's bits above and below bit 32: hi parts < 2^48 and lo parts
        // < 2^32 add up over a whole row (16384 terms) without overflow, and the
        // sum is hi 2^32 + lo.
        double s1d = 0.0;
        uint64_t hi = 0, lo = 0;
    #pragma unroll
        for (int it = 0; it < ITS; ++it) {
            if (tid + (int64_t)it * 256 < nvec) {
                const uint32_t w[4] = {raw[it].x, raw[it].y, raw[it].z, raw[it].w};
                float v[8];
                widen16<F16>(raw[it], v);
    #pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t h = (w[e >> 1] >> (16 * (e & 1))) & 0xffffu;
                    s1d += (double)v[e];
                    const uint32_t ex = (h >> 10) & 31u;
                    const uint32_t m = (h & 1023u) | (ex ? 1024u : 0u);
                    const uint32_t sh = ex ? 2u * (ex - 1u) : 0u;      // 0 .. 58
                    const uint32_t sl = sh < 32u ? sh : 32u;
                    const uint64_t full = (uint64_t)(m * m) << sl;      // m^2 < 2^22
                    lo += (uint32_t)full;                               // bits 0 .. 31
                    hi += (full >> 32) << (sh - sl);                    // bits 32 .. 79, / 2^32
                }
            }
        }
    #pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            s1d += __shfl_xor(s1d, off, kWave);
            hi += __shfl_xor(hi, off, kWave);
            lo += __shfl_xor(lo, off, kWave);
        }
        const int64_t s1 = (int64_t)(s1d * 16777216.0);  // exact: an integer below 2^54
        if (lane == 0) {
            sh_s1[PAR][wave] = s1;
            sh_lo[PAR][wave] = lo;
            sh_hi[PAR][wave] = hi;
        }
        __syncthreads();
        int64_t S1 = 0;
        uint64_t H = 0, Lo = 0;
    #pragma unroll
        for (int w = 0; w < 4; ++w) {
            S1 += sh_s1[PAR][w];
            H += sh_hi[PAR][w];
            Lo += sh_lo[PAR][w];
        }
        const u128 S2 = ((u128)H << 32) + Lo;

        float mu, rstd;
        norm_stats<NORM>(S1, S2, K, eps, mu, rstd);

        // The normalized, scaled row (kept in registers for the store pass).
        float y[ITS][8];
        float amax = 0.0f;
    #pragma unroll
        for (int it = 0; it < ITS; ++it) {
            float v[8];
            widen16<F16>(raw[it], v);
            const float gv[8] = {g[it][0].x, g[it][0].y, g[it][0].z, g[it][0].w,
                                 g[it][1].x, g[it][1].y, g[it][1].z, g[it][1].w};
            const bool live = tid + (int64_t)it * 256 < nvec;
    #pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float n = NORM == 0 ? (v[e] - mu) * rstd : v[e] * rstd;
                float t = n * gv[e];
                if constexpr (HAS_BETA) {
                    const float bv[8] = {b[it][0].x, b[it][0].y, b[it][0].z, b[it][0].w,
                                         b[it][1].x, b[it][1].y, b[it][1].z, b[it][1].w};
                    t = t + bv[e];
                }
                y[it][e] = t;
                if (live) amax = fmaxf(amax, fabsf(t));
            }
        }

        float inv;
        if constexpr (DYN) {
            amax = wave_max(amax);
            if (lane == 0) sh_max[PAR][wave] = amax;
            __syncthreads();
            float a = fmaxf(fmaxf(sh_max[PAR][0], sh_max[PAR][1]), fmaxf(sh_max[PAR][2], sh_max[PAR][3]));
            if (!(a > 1e-8f)) a = 1e-8f;
            inv = 127.0f / a;
            if (tid == 0) scale[r] = a / 127.0f;
        } else {
            inv = static_scale[1];
        }
        int8_t *qr = q + r * K;
    #pragma unroll
        for (int it = 0; it < ITS; ++it) {
            const int64_t vi = tid + (int64_t)it * 256;
            if (vi < nvec) {
                uint2 o;
                o.x = pack4(quant_i8(y[it][0], inv), quant_i8(y[it][1], inv), quant_i8(y[it][2], inv),
                            quant_i8(y[it][3], inv));
                o.y = pack4(quant_i8(y[it][4], inv), quant_i8(y[it][5], inv), quant_i8(y[it][6], inv),
                            quant_i8(y[it][7], inv));
                *reinterpret_cast<uint2 *>(qr + vi * 8) = o;
            }
        }
    };
    const int64_t r_begin = (int64_t)blockIdx.x * rows_per_block;
    const int64_t r_end = r_begin + rows_per_block < rows ? r_begin + rows_per_block : rows;
    uint4 b0[ITS], b1[ITS];
    load_row(r_begin, b0);
    // The prefetch is conditional: no load is issued past the block's last
    // row.  (An unconditional prefetch that re-read an already fetched row
    // gave wrong sums on this GPU: that load hits in cache, and the exact
    // wait counts the compiler derives for the other buffer assume every
    // load retires in issue order.)
    for (int64_t r = r_begin;; r += 2) {
        if (r + 1 < r_end) load_row(r + 1, b1);
        process(r, b0, std::integral_constant<int, 0>{});
        if (r + 1 >= r_end) break;
        if (r + 2 < r_end) load_row(r + 2, b0);
        process(r + 1, b1, std::integral_constant<int, 1>{});
        if (r + 2 >= r_end) break;
    }
}

void launch_fold_norm(const float *gamma, const float *beta, const float *s, int64_t K,
                      float *gamma_out, float *beta_out, hipStream_t stream) {
    fold_norm_kernel<<<dim3((unsigned)((K + 255) / 256)), dim3(256), 0, stream>>>(
        gamma, beta, s, K, gamma_out, beta_out);
}

template <int ITS, int NORM>
static void launch_nq(const void *x, int64_t M, int64_t K, const float *gamma,
                      const float *beta, float eps, int dynamic, const float *static_scale,
                      int8_t *q, float *scale, hipStream_t stream) {
    // ~2048 blocks (one round at 8 per CU), several rows each when there are
    // many, so gamma / beta are read once per block.
    int64_t rpb = (M + 2047) / 2048;
    if (rpb < 1) rpb = 1;
    dim3 grid((unsigned)((M + rpb - 1) / rpb)), block(256);
    auto *xv = reinterpret_cast<const uint4 *>(x);
#define SQ_NQ(HB, DY)                                                                          \
    norm_quant_kernel<ITS, NORM, HB, DY><<<grid, block, 0, stream>>>(xv, M, K, gamma, beta,     \
                                                                   eps, static_scale, q, scale, \
                                                                   (int)rpb)
    if (beta) {
        if (dynamic) SQ_NQ(true, true);
        else SQ_NQ(true, false);
    } else {
        if (dynamic) SQ_NQ(false, true);
        else SQ_NQ(false, false);
    }
#undef SQ_NQ
}

void launch_norm_quant(const void *x, int64_t M, int64_t K, int norm, const float *gamma,
                       const float *beta, float eps, int dynamic, const float *static_scale,
                       int8_t *q, float *scale, hipStream_t stream) {
    const int64_t its = (K / 8 + 255) / 256;  // K <= 16384: at most 8
#define SQ_NQI(ITS)                                                                           \
    do {                                                                                      \
        if (norm == 0) launch_nq<ITS, 0>(x, M, K, gamma, beta, eps, dynamic, static_scale, q, \
                                         scale, stream);                                      \
        else launch_nq<ITS, 1>(x, M, K, gamma, beta, eps, dynamic, static_scale, q, scale,    \
                               stream);                                                       \
    } while (0)
    if (its <= 1) SQ_NQI(1);
    else if (its <= 2) SQ_NQI(2);
    else if (its <= 4) SQ_NQI(4);
    else SQ_NQI(8);
#undef SQ_NQI
}

}  // namespace sq
