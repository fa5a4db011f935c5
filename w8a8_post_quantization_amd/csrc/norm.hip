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
// in which the block adds them up (K <= 16384).  The kernel forms them from
// sums in double that never round (see norm_quant_kernel).  From them:
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

// Wave sums and maxima through DPP lane moves (no LDS round trip): four
// steps leave each 16-lane row's total in all its lanes, two row broadcasts
// then carry the wave's total into lane 63.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_i32(int v) {
    if constexpr (ROWS == 0xf) return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, false);
    else return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xf, false);  // other rows: 0
}
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)dpp_i32<CTRL, ROWS>((int)(uint32_t)u);
    const uint32_t hi = (uint32_t)dpp_i32<CTRL, ROWS>((int)(uint32_t)(u >> 32));
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror,
// row_bcast:15 into rows 1 and 3, row_bcast:31 into rows 2 and 3.
__device__ __forceinline__ double wave_sum_to_last(double v) {
    v += dpp_f64<0xb1, 0xf>(v);
    v += dpp_f64<0x4e, 0xf>(v);
    v += dpp_f64<0x141, 0xf>(v);
    v += dpp_f64<0x140, 0xf>(v);
    v += dpp_f64<0x142, 0xa>(v);
    v += dpp_f64<0x143, 0xc>(v);
    return v;
}
// Non-negative inputs: lanes outside a broadcast's rows read 0.
__device__ __forceinline__ float wave_max_to_last(float v) {
    v = fmaxf(v, __int_as_float(dpp_i32<0xb1, 0xf>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_i32<0x4e, 0xf>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_i32<0x141, 0xf>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_i32<0x140, 0xf>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_i32<0x142, 0xa>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_i32<0x143, 0xc>(__float_as_int(v))));
    return v;
}

// The low bytes of eight words, in order, as two words: perm's selector
// 0x0c0c0400 takes [b0 of the second operand, b0 of the first, 0, 0], and
// 0x05040100 joins two such halves.
__device__ __forceinline__ uint2 pack_low_bytes(const uint32_t (&bits)[8]) {
    uint2 o;
    o.x = __builtin_amdgcn_perm(__builtin_amdgcn_perm(bits[3], bits[2], 0x0c0c0400u),
                                __builtin_amdgcn_perm(bits[1], bits[0], 0x0c0c0400u),
                                0x05040100u);
    o.y = __builtin_amdgcn_perm(__builtin_amdgcn_perm(bits[7], bits[6], 0x0c0c0400u),
                                __builtin_amdgcn_perm(bits[5], bits[4], 0x0c0c0400u),
                                0x05040100u);
    return o;
}

// Round four fp32 values of magnitude below 2^22 to integers (half to
// even) and pack their two's complement low bytes into one word: each add
// of 1.5 2^23 rounds its value and writes the low byte of the sum's bits
// straight into byte n of the word (an SDWA destination select), the
// other bytes kept.
__device__ __forceinline__ uint32_t round_pack4(float z0, float z1, float z2, float z3,
                                                float magic) {
    uint32_t w;
    asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:DWORD "
        "src1_sel:DWORD"
        : "=v"(w) : "v"(z0), "v"(magic));
    asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD "
        "src1_sel:DWORD"
        : "+v"(w) : "v"(z1), "v"(magic));
    asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD "
        "src1_sel:DWORD"
        : "+v"(w) : "v"(z2), "v"(magic));
    asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD "
        "src1_sel:DWORD"
        : "+v"(w) : "v"(z3), "v"(magic));
    return w;
}

// Eight codes; NT: a nontemporal store, for outputs larger than the 256 MB
// last-level cache (streamed past the caches, a 940 MB -> 470 MB norm
// measured about 9 % faster; smaller outputs stay cached for the GEMM that
// reads them next).
typedef unsigned int u2v_nt __attribute__((ext_vector_type(2)));
template <bool NT>
__device__ __forceinline__ void store8(int8_t *p, uint32_t a, uint32_t b) {
    if constexpr (NT) __builtin_nontemporal_store(u2v_nt{a, b}, reinterpret_cast<u2v_nt *>(p));
    else *reinterpret_cast<uint2 *>(p) = make_uint2(a, b);
}

// A 256-thread block per row, walking rows_per_block consecutive rows; ITS
// 16-byte vectors (8 fp16) per thread.  Every load is unconditional, with
// out-of-range vector indices clamped to the row's last vector (loaded, not
// used): a load under a lane-divergent branch would wait for all earlier
// memory operations.  The row's sums and maximum are combined across the 4
// waves through LDS slots that alternate between consecutive rows, so one
// barrier per exchange suffices.  (Four waves per row, one per SIMD, keep
// the work between barriers even across the SIMDs; more waves per row
// repeat the per-row reductions more often.)
template <int ITS, int NORM, bool HAS_BETA, bool DYN, bool BETA_LDS>
__global__ __launch_bounds__(256) void norm_quant_kernel(const uint4 *__restrict__ x,
                                                         int64_t rows, int64_t K,
                                                         const float *__restrict__ gamma,
                                                         const float *__restrict__ beta,
                                                         float eps,
                                                         const float *__restrict__ static_scale,
                                                         int8_t *__restrict__ q,
                                                         float *__restrict__ scale,
                                                         int rows_per_block) {
    constexpr int T = 256;
    __shared__ int64_t sh_s1[2][4];
    __shared__ int64_t sh_lo[2][4], sh_hi[2][4];
    __shared__ float sh_max[2][4];
    __shared__ float sh_stat[2][2];  // mu, rstd of the row (written by wave 0)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wave_base = __builtin_amdgcn_readfirstlane(tid & ~63);  // wave-uniform
    if (!DYN && blockIdx.x == 0 && tid == 0) scale[0] = static_scale[0];
    const int64_t nvec = K / 8;

    // gamma (and, for rows of up to 16 K bytes, beta too) of this thread's
    // vectors stay in registers, loaded once for all the block's rows.
    // Otherwise beta is staged in LDS (K floats, dynamic shared memory):
    // that frees 8 ITS registers, enough for a third wave per SIMD.
    constexpr bool BETA_REG = HAS_BETA && !BETA_LDS;
    float4 g[ITS][2], b[BETA_REG ? ITS : 1][2];
#pragma unroll
    for (int it = 0; it < ITS; ++it) {
        const int64_t vi = tid + (int64_t)it * T;
        const int64_t vc = vi < nvec ? vi : nvec - 1;
        const float4 *gp = reinterpret_cast<const float4 *>(gamma + vc * 8);
        g[it][0] = gp[0];
        g[it][1] = gp[1];
        if constexpr (BETA_REG) {
            const float4 *bp = reinterpret_cast<const float4 *>(beta + vc * 8);
            b[it][0] = bp[0];
            b[it][1] = bp[1];
        }
    }
    extern __shared__ float4 sh_beta[];  // [K / 4] when BETA_LDS
    if constexpr (BETA_LDS) {
        const float4 *bp = reinterpret_cast<const float4 *>(beta);
        for (int64_t i = tid; i < K / 4; i += T) sh_beta[i] = bp[i];
        __syncthreads();
    }
    auto load_row = [&](int64_t r, uint4 (&raw)[ITS]) {
        const uint4 *xr = x + r * nvec;
#pragma unroll
        for (int it = 0; it < ITS; ++it) {
            const int64_t vi = tid + (int64_t)it * T;
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
        // Exact row sums in double.  sum x: every term is a multiple of 2^-24
        // and a wave's |sum| < 4096 * 65504 < 2^28, so no partial sum rounds.
        // sum x^2: x^2 is exact in double; fma(x, x, C) with C = 1.5 2^45
        // lands in [2^45, 2^46), where the spacing is 2^-7, so
        // h = fma(x, x, C) - C is x^2 rounded to a multiple of 2^-7 and
        // l = fma(x, x, -h) = x^2 - h is exact (a multiple of 2^-48, |l| <=
        // 2^-8).  A wave adds at most 512 ITS <= 4096 terms: the h sum stays
        // below 2^44 (2^51 steps of 2^-7) and the l sum below 2^4 (2^52 steps
        // of 2^-48), so neither ever rounds, in any order.  Each wave's three sums are
        // then exact integers in units of 2^-24, 2^-7 and 2^-48.
        constexpr double kSplit = 52776558133248.0;  // 1.5 * 2^45
        double s1d = 0.0, shi = 0.0, slo = 0.0;
    #pragma unroll
        for (int it = 0; it < ITS; ++it) {
            if (tid + (int64_t)it * T < nvec) {
                float v[8];
                widen16<F16>(raw[it], v);
    #pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const double d = (double)v[e];
                    if constexpr (NORM == 0) s1d += d;
                    const double h = __builtin_fma(d, d, kSplit) - kSplit;
                    shi += h;
                    slo += __builtin_fma(d, d, -h);
                }
            }
        }
        if constexpr (NORM == 0) s1d = wave_sum_to_last(s1d);
        shi = wave_sum_to_last(shi);
        slo = wave_sum_to_last(slo);
        if (lane == 63) {
            sh_s1[PAR][wave] = (int64_t)(s1d * 16777216.0);        // x 2^24
            sh_hi[PAR][wave] = (int64_t)(shi * 128.0);             // x^2 2^7
            sh_lo[PAR][wave] = (int64_t)(slo * 281474976710656.0); // x^2 2^48
        }
        __syncthreads();
        // Row totals: |S1| < 2^54, H < 2^53, |L| < 2^54; the row's
        // sum (x 2^24)^2 = H 2^41 + L.  Wave 0 alone turns them into mu and
        // rstd (about a tenth of a row's VALU work per wave, in fp64
        // divisions and a square root) and passes them on through LDS.
        if (wave_base == 0) {
            int64_t S1 = 0, H = 0, L = 0;
    #pragma unroll
            for (int w = 0; w < 4; ++w) {
                if constexpr (NORM == 0) S1 += sh_s1[PAR][w];
                H += sh_hi[PAR][w];
                L += sh_lo[PAR][w];
            }
            const u128 S2 = (u128)(((__int128)H << 41) + L);
            float mu0, rstd0;
            norm_stats<NORM>(S1, S2, K, eps, mu0, rstd0);
            if (lane == 0) {
                sh_stat[PAR][0] = mu0;
                sh_stat[PAR][1] = rstd0;
            }
        }
        __syncthreads();
        const float mu = sh_stat[PAR][0], rstd = sh_stat[PAR][1];

        // The normalized, scaled row (kept in registers for the store pass).
        // Slots past the row's end hold copies of its last vector (clamped
        // loads of x, gamma and beta), so they may enter the maximum; slots
        // no lane of this wave owns are skipped on a scalar branch.
        float y[ITS][8];
        float amax = 0.0f;
    #pragma unroll
        for (int it = 0; it < ITS; ++it) {
            if (wave_base + it * T >= nvec) continue;
            float v[8];
            widen16<F16>(raw[it], v);
            const float gv[8] = {g[it][0].x, g[it][0].y, g[it][0].z, g[it][0].w,
                                 g[it][1].x, g[it][1].y, g[it][1].z, g[it][1].w};
            float4 bl[2];
            if constexpr (BETA_LDS) {
                const int64_t vi = tid + (int64_t)it * T;
                const int64_t vc = vi < nvec ? vi : nvec - 1;
                bl[0] = sh_beta[vc * 2];
                bl[1] = sh_beta[vc * 2 + 1];
            } else if constexpr (BETA_REG) {
                bl[0] = b[it][0];
                bl[1] = b[it][1];
            }
    #pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float n = NORM == 0 ? (v[e] - mu) * rstd : v[e] * rstd;
                float t = n * gv[e];
                if constexpr (HAS_BETA) {
                    const float bv[8] = {bl[0].x, bl[0].y, bl[0].z, bl[0].w,
                                         bl[1].x, bl[1].y, bl[1].z, bl[1].w};
                    t = t + bv[e];
                }
                y[it][e] = t;
                amax = fmaxf(amax, fabsf(t));
            }
        }

        float inv;
        if constexpr (DYN) {
            amax = wave_max_to_last(amax);
            if (lane == 63) sh_max[PAR][wave] = amax;
            __syncthreads();
            float a = fmaxf(fmaxf(sh_max[PAR][0], sh_max[PAR][1]), fmaxf(sh_max[PAR][2], sh_max[PAR][3]));
            if (!(a > 1e-8f)) a = 1e-8f;
            inv = 127.0f / a;
            if (tid == 0) scale[r] = a / 127.0f;
        } else {
            inv = static_scale[1];
        }
        // q = clamp(rint(fl(y inv)), -127, 127).  Adding 1.5 2^23 to a value
        // of magnitude below 2^22 rounds it to an integer, half to even, and
        // leaves that integer's two's complement low byte in the low byte of
        // the sum's bits.  With the per-token step |y| <= a, so
        // |fl(y inv)| <= 127 (1 + 2^-24) and the clamp never acts; with a
        // fixed step the product is clamped first (rint and the clamp commute
        // at integer bounds).
        int8_t *qr = q + r * K;
    #pragma unroll
        for (int it = 0; it < ITS; ++it) {
            if (wave_base + it * T >= nvec) continue;
            uint32_t bits[8];
    #pragma unroll
            for (int e = 0; e < 8; ++e) {
                float z = y[it][e] * inv;
                if constexpr (!DYN) z = __builtin_amdgcn_fmed3f(z, -127.0f, 127.0f);
                bits[e] = __float_as_uint(z + 12582912.0f);
            }
            const int64_t vi = tid + (int64_t)it * T;
            if (vi < nvec) *reinterpret_cast<uint2 *>(qr + vi * 8) = pack_low_bytes(bits);
        }
    };
    const int64_t r_begin = (int64_t)blockIdx.x * rows_per_block;
    const int64_t r_end = r_begin + rows_per_block < rows ? r_begin + rows_per_block : rows;
    uint4 b0[ITS], b1[ITS];
    load_row(r_begin, b0);
    // The prefetch is conditional: no load is issued past the block's last
    // row.  (A variant whose prefetch re-read the block's last row
    // unconditionally gave wrong sums now and then; it was not kept and its
    // cause was not found.  It was not the order in which loads return: a
    // wave's vector-memory loads return in issue order, which the partial
    // waits of every kernel here, and the compiler's own, rely on.)
    for (int64_t r = r_begin;; r += 2) {
        if (r + 1 < r_end) load_row(r + 1, b1);
        process(r, b0, std::integral_constant<int, 0>{});
        if (r + 1 >= r_end) break;
        if (r + 2 < r_end) load_row(r + 2, b0);
        process(r + 1, b1, std::integral_constant<int, 1>{});
        if (r + 2 >= r_end) break;
    }
}

// The wave's value of a double in lane 63, in every lane (two scalar reads).
__device__ __forceinline__ double from_lane63(double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 63);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// One wave per row, for rows of at most 8192 elements when there are many
// rows: a row's statistics then take one wave's reductions, with no
// exchange through LDS and no barrier, instead of four waves' (which on
// 7168-element rows cost about a third of the block-per-row kernel's
// instructions).  Lane l owns the row's vectors l, l + 64, ..., l + 64
// (ITS - 1); the waves of the chip walk the rows round-robin.  gamma and
// beta are staged once per block in LDS, each split into two planes of
// float4 (elements 0-3 and 4-7 of every vector) so that consecutive lanes
// read consecutive 16 bytes.  The first pass widens the row to fp32 in
// registers, where it stays for the second; the next row's loads are
// issued right after it, into the fp16 registers it has freed.
//
// Exact row sums.  sum x as in the block-per-row kernel (|sum| < 8192 *
// 65504 < 2^29 in steps of 2^-24: no partial sum rounds).  sum x^2 by a
// running accumulator held in [2^45, 2^46), where doubles are spaced 2^-7:
// a = fma(x, x, acc) is acc plus x^2 rounded to a multiple of 2^-7, so
// h = a - acc is exact (both in one binade) and l = fma(x, x, -h) = x^2 - h
// is exact (|l| <= 2^-8, a multiple of 2^-48).  The accumulator starts at
// 1.5 2^45 and a lane adds at most 128 squares below 2^32, so it stays
// below 2^46; its final value minus the start is the lane's sum of h,
// exactly.  The wave's h sum stays below 8192 * 2^32 = 2^45 (2^52 steps of
// 2^-7) and its l sum within 2^5 (2^53 steps of 2^-48), in any order.
template <int ITS, int NORM, bool HAS_BETA, bool DYN, bool NT, int WPB>
__global__ __launch_bounds__(WPB * 64) void norm_quant_wave_kernel(
    const uint4 *__restrict__ x, int64_t rows, const float *__restrict__ gamma,
    const float *__restrict__ beta, float eps, const float *__restrict__ static_scale,
    int8_t *__restrict__ q, float *__restrict__ scale) {
    constexpr int NV = ITS * 64;  // vectors per row: K = 512 ITS
    constexpr int64_t K = NV * 8;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (!DYN && blockIdx.x == 0 && tid == 0) scale[0] = static_scale[0];

    extern __shared__ float4 sh_gb[];  // gamma planes [2][NV], then beta planes [2][NV]
    {
        const float4 *gp = reinterpret_cast<const float4 *>(gamma);
        const float4 *bp = reinterpret_cast<const float4 *>(beta);
        for (int i = tid; i < NV; i += WPB * 64) {
            sh_gb[i] = gp[2 * i];
            sh_gb[NV + i] = gp[2 * i + 1];
            if constexpr (HAS_BETA) {
                sh_gb[2 * NV + i] = bp[2 * i];
                sh_gb[3 * NV + i] = bp[2 * i + 1];
            }
        }
    }
    __syncthreads();
    const float4 *const g_lo = sh_gb + lane, *const g_hi = sh_gb + NV + lane;
    const float4 *const b_lo = sh_gb + 2 * NV + lane, *const b_hi = sh_gb + 3 * NV + lane;
    const float inv_static = DYN ? 0.0f : static_scale[1];
    // q = clamp(rint(fl(y inv)), -127, 127), as in the block-per-row kernel
    // (the clamp acts only with a fixed step).
    const float magic = 12582912.0f;  // 1.5 2^23

    const int64_t stride = (int64_t)gridDim.x * WPB;
    uint4 raw[ITS];
    // A row's loads, in the order the first pass uses them (the barriers
    // keep the scheduler from reordering them), so that each use waits for
    // its own load only.
    auto load_row = [&](int64_t row) {
        const uint4 *xr = x + row * NV + lane;
    #pragma unroll
        for (int it = 0; it < ITS; ++it) {
            raw[it] = ld_nt(xr + it * 64);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // One row; with PF the next row's loads are issued into raw[] once the
    // first pass has widened this row to fp32 (straight-line code, so the
    // compiler's waits count exactly the loads each use needs).
    auto row = [&](int64_t r, auto pf_c) {
        constexpr bool PF = decltype(pf_c)::value;
        // Four independent sets of the three sums (element e of a vector
        // feeds set e mod 4), so that the dependent fp64 steps of one
        // element overlap those of the next three; each set's sums are
        // exact (a quarter of the lane's terms), and so are their totals.
        constexpr double kAcc = 52776558133248.0;  // 1.5 * 2^45
        constexpr int NS = 4;
        double s1s[NS], accs[NS], slos[NS];
    #pragma unroll
        for (int j = 0; j < NS; ++j) {  // -0 + x = x for every x: the first adds fold away
            s1s[j] = -0.0;
            accs[j] = kAcc;
            slos[j] = -0.0;
        }
        float v[ITS][8];  // the row in fp32, then the normalized row in place
    #pragma unroll
        for (int it = 0; it < ITS; ++it) {
            widen16<F16>(raw[it], v[it]);
            // widened once, kept for the second pass
            asm volatile("" : "+v"(v[it][0]), "+v"(v[it][1]), "+v"(v[it][2]), "+v"(v[it][3]),
                         "+v"(v[it][4]), "+v"(v[it][5]), "+v"(v[it][6]), "+v"(v[it][7]));
            // Written step by step over the vector (each step on the eight
            // elements before the next), the order the scheduler keeps.
            double d[8], a[8], h[8], l[8];
    #pragma unroll
            for (int e = 0; e < 8; ++e) d[e] = (double)v[it][e];
    #pragma unroll
            for (int e = 0; e < 8; ++e) a[e] = __builtin_fma(d[e], d[e], e < NS ? accs[e] : a[e - NS]);
    #pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = a[e] - (e < NS ? accs[e] : a[e - NS]);
    #pragma unroll
            for (int e = 0; e < 8; ++e) l[e] = __builtin_fma(d[e], d[e], -h[e]);
    #pragma unroll
            for (int j = 0; j < NS; ++j) {
                accs[j] = a[j + NS];
                slos[j] = (slos[j] + l[j]) + l[j + NS];
                if constexpr (NORM == 0) s1s[j] = (s1s[j] + d[j]) + d[j + NS];
            }
        }
        double s1d = (s1s[0] + s1s[1]) + (s1s[2] + s1s[3]);
        double shi = ((accs[0] - kAcc) + (accs[1] - kAcc)) + ((accs[2] - kAcc) + (accs[3] - kAcc));
        double slo = (slos[0] + slos[1]) + (slos[2] + slos[3]);
        if constexpr (PF) {
            __builtin_amdgcn_sched_barrier(0);
            load_row(r + stride);
        }
        if constexpr (NORM == 0) s1d = from_lane63(wave_sum_to_last(s1d));
        shi = from_lane63(wave_sum_to_last(shi));
        slo = from_lane63(wave_sum_to_last(slo));
        // The row's sums as integers: S1 = sum x 2^24, H = sum h 2^7,
        // L = sum l 2^48, and sum (x 2^24)^2 = H 2^41 + L.
        const int64_t S1 = NORM == 0 ? (int64_t)(s1d * 16777216.0) : 0;
        const int64_t H = (int64_t)(shi * 128.0);
        const int64_t L = (int64_t)(slo * 281474976710656.0);
        float mu, rstd;
        norm_stats<NORM>(S1, (u128)(((__int128)H << 41) + L), K, eps, mu, rstd);

        // The normalized, scaled row: kept in registers when its maximum
        // sets the step, else quantized at once.
        int8_t *const qr = q + r * K + lane * 8;
        float amax = 0.0f;
    #pragma unroll
        for (int it = 0; it < ITS; ++it) {
            const float4 ga = g_lo[it * 64], gb = g_hi[it * 64];
            const float gv[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
            float bv[8] = {};
            if constexpr (HAS_BETA) {
                const float4 ba = b_lo[it * 64], bb = b_hi[it * 64];
                bv[0] = ba.x; bv[1] = ba.y; bv[2] = ba.z; bv[3] = ba.w;
                bv[4] = bb.x; bv[5] = bb.y; bv[6] = bb.z; bv[7] = bb.w;
            }
            float t[8];
    #pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float n = NORM == 0 ? (v[it][e] - mu) * rstd : v[it][e] * rstd;
                t[e] = n * gv[e];
                if constexpr (HAS_BETA) t[e] = t[e] + bv[e];
            }
            if constexpr (DYN) {
    #pragma unroll
                for (int e = 0; e < 8; ++e) {
                    v[it][e] = t[e];
                    amax = fmaxf(amax, fabsf(t[e]));
                }
            } else {
                float z[8];
    #pragma unroll
                for (int e = 0; e < 8; ++e)
                    z[e] = __builtin_amdgcn_fmed3f(t[e] * inv_static, -127.0f, 127.0f);
                store8<NT>(qr + it * 512, round_pack4(z[0], z[1], z[2], z[3], magic),
                           round_pack4(z[4], z[5], z[6], z[7], magic));
            }
        }
        if constexpr (DYN) {
            float a = __int_as_float(
                __builtin_amdgcn_readlane(__float_as_int(wave_max_to_last(amax)), 63));
            if (!(a > 1e-8f)) a = 1e-8f;
            const float inv = 127.0f / a;
            if (lane == 0) scale[r] = a / 127.0f;
    #pragma unroll
            for (int it = 0; it < ITS; ++it) {
                float z[8];
    #pragma unroll
                for (int e = 0; e < 8; ++e) z[e] = v[it][e] * inv;
                store8<NT>(qr + it * 512, round_pack4(z[0], z[1], z[2], z[3], magic),
                           round_pack4(z[4], z[5], z[6], z[7], magic));
            }
        }
    };
    // The first row is peeled, so the loop is only ever entered after a
    // row like its own: stores of that row after loads of this one, and
    // the compiler's waits for the loads need not wait for the stores.
    int64_t r = (int64_t)blockIdx.x * WPB + wave;
    if (r >= rows) return;
    load_row(r);
    if (r + stride < rows) {
        row(r, std::true_type{});
        for (r += stride; r + stride < rows; r += stride) row(r, std::true_type{});
    }
    row(r, std::false_type{});
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
    // Beta goes to LDS when the block walks several rows (the staging
    // costs more than it saves for one row) and the row fits (ITS <= 4).
    const bool beta_lds = beta && ITS <= 4 && rpb > 1;
    const size_t lds = beta_lds ? (size_t)K * sizeof(float) : 0;
#define SQ_NQ(HB, DY, BL)                                                                      \
    norm_quant_kernel<ITS, NORM, HB, DY, BL><<<grid, block, lds, stream>>>(                     \
        xv, M, K, gamma, beta, eps, static_scale, q, scale, (int)rpb)
    if (beta_lds) {
        if constexpr (ITS <= 4) {
            if (dynamic) SQ_NQ(true, true, true);
            else SQ_NQ(true, false, true);
        }
    } else if (beta) {
        if (dynamic) SQ_NQ(true, true, false);
        else SQ_NQ(true, false, false);
    } else {
        if (dynamic) SQ_NQ(false, true, false);
        else SQ_NQ(false, false, false);
    }
#undef SQ_NQ
}

// Compute units of the current device (cached per device).
static int cu_count() {
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] <= 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

template <int ITS, int NORM>
static void launch_nq_wave(const void *x, int64_t M, const float *gamma, const float *beta,
                           float eps, int dynamic, const float *static_scale, int8_t *q,
                           float *scale, hipStream_t stream) {
    // One block of 8 waves per compute unit (fewer for few rows); the waves
    // walk the rows round-robin.
    constexpr int WPB = 8;
    const int64_t want = (M + WPB - 1) / WPB;
    const int64_t cus = cu_count();
    dim3 grid((unsigned)(want < cus ? want : cus)), block(WPB * 64);
    const size_t lds = (size_t)ITS * 512 * (beta ? 2 : 1) * sizeof(float);
    auto *xv = reinterpret_cast<const uint4 *>(x);
    const bool nt = M * ITS * 512 > ((int64_t)256 << 20);  // codes beyond the last-level cache
#define SQ_NQW(HB, DY, NT)                                                                     \
    norm_quant_wave_kernel<ITS, NORM, HB, DY, NT, WPB><<<grid, block, lds, stream>>>(           \
        xv, M, gamma, beta, eps, static_scale, q, scale)
#define SQ_NQW2(HB, DY)                                                                        \
    do {                                                                                       \
        if (nt) SQ_NQW(HB, DY, true);                                                          \
        else SQ_NQW(HB, DY, false);                                                            \
    } while (0)
    if (beta) {
        if (dynamic) SQ_NQW2(true, true);
        else SQ_NQW2(true, false);
    } else {
        if (dynamic) SQ_NQW2(false, true);
        else SQ_NQW2(false, false);
    }
#undef SQ_NQW2
#undef SQ_NQW
}

void launch_norm_quant(const void *x, int64_t M, int64_t K, int norm, const float *gamma,
                       const float *beta, float eps, int dynamic, const float *static_scale,
                       int8_t *q, float *scale, hipStream_t stream, int force_kernel) {
    // The wave-per-row kernel (built for K = 512 ITS, ITS in {4, 6, ...,
    // 16}) from 1024 rows up; with fewer rows, one wave per row leaves most
    // of the chip idle and the block-per-row kernel, four waves per row,
    // finishes sooner (7168-element rows: 4.6 against 8.7 us at 256 rows,
    // even at 1024, 11 against 19 us at 2048).
    const bool wave_k = K % 1024 == 0 && K >= 2048 && K <= 8192;
    if (wave_k && (force_kernel == 1 || (force_kernel != 0 && M >= 1024))) {
#define SQ_NQWI(ITS)                                                                          \
    case ITS:                                                                                 \
        if (norm == 0) launch_nq_wave<ITS, 0>(x, M, gamma, beta, eps, dynamic, static_scale, q, \
                                              scale, stream);                                 \
        else launch_nq_wave<ITS, 1>(x, M, gamma, beta, eps, dynamic, static_scale, q, scale,   \
                                    stream);                                                  \
        return;
        switch (K / 512) {
            SQ_NQWI(4) SQ_NQWI(6) SQ_NQWI(8) SQ_NQWI(10) SQ_NQWI(12) SQ_NQWI(14) SQ_NQWI(16)
            default: break;
        }
#undef SQ_NQWI
    }
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
