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
// With FP8 = true the codes are OCP e4m3fn instead (448 in place of 127:
// step = fl(a/448), q = e4m3(clamp(fl(v * fl(448/a)), -448, 448)) by the
// hardware conversion, which rounds to nearest even and is exact on every
// in-range value; the SmoothQuant encyclopedia page, 技術原理與特性: INT8 or
// FP8 units).
// Weights may also carry a per-row factor applied first,
// v = fl(fl(x[r, k] * row_mul[r]) * mul[k]): the next layer's 1/s folded
// into this layer's output channels (the SmoothQuant tutorial page, section
// 融入前序线性层的权重: up_proj for down_proj, v_proj for o_proj).
//
// One 64-lane wave per row (or, for few rows, one 256-thread block per
// row).  Each lane keeps its 16-byte vectors of the row in registers (up to
// 16 per lane: 8192 16-bit or 4096 fp32 elements), so HBM is read once and
// written once; longer rows re-read from L2.
#include "sq_device.h"
#include "sq_launch.h"

namespace sq {


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

extern __shared__ float4 smul4[];

// LLM.int8() mask mode (ol.on): the column multiplier is 1 for a kept
// column and 0 for an outlier column, derived where it is read from the
// column abs-max (mul then points to it): a column is an outlier dimension
// when its largest |x| reaches the threshold (the xdnf.cn LLM.int8()
// explainer, §2.2 and §4.1).
__device__ __forceinline__ float keep(float colmax, float thr) {
    return colmax >= thr ? 0.0f : 1.0f;
}
__device__ __forceinline__ float4 keep4(float4 c, float thr) {
    return make_float4(keep(c.x, thr), keep(c.y, thr), keep(c.z, thr), keep(c.w, thr));
}

// The extra blocks of a masked quantizer (the last ol.blocks blocks of the
// grid, after the row blocks: the row blocks keep the even spread over the
// compute units they have without them, measured 3 us faster for the
// 2048 x 4096 activations than with the extra blocks first).  Each
// rebuilds the ascending outlier list from the column maxima: a pass covers
// 256 * C columns, thread t the C consecutive columns from t * C, loaded as
// four 16-byte vectors with no condition (K % 16 == 0, so a thread's columns
// are all in range or all past the end, and those past it re-read the last
// 16; a load under a lane-dependent condition would make the compiler wait
// for each one before the next); a wave prefix sum of the per-thread hit counts plus the earlier
// waves' totals gives each thread its first list slot.  Block 0 writes the
// mask, the list and |O|; every block keeps the first cap entries in LDS and,
// when |O| <= cap, gathers its share of the side operands (element e of the
// cnt (M + N) values, e = b * 256 + tid, b * 256 + tid + 256 * blocks, ...;
// consecutive threads take consecutive rows of one column, so the stores are
// coalesced).  Called by every thread of the block.
__device__ void outlier_side_block(const float *__restrict__ colmax,
                                   const uint16_t *__restrict__ x16, int64_t K,
                                   const OutlierList &ol, int b) {
    const int64_t M = ol.M;
    constexpr int C = 16;
    __shared__ int wave_tot[4];
    __shared__ int s_idx[kSideColsMax];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool lead = b == 0;
    int base = 0;  // list entries of earlier passes (the same in every thread)
    for (int64_t j0 = 0; j0 < K; j0 += 256 * C) {
        const int64_t jb = j0 + (int64_t)tid * C;
        const float4 *src = reinterpret_cast<const float4 *>(colmax + (jb < K ? jb : K - C));
        float v[C];
#pragma unroll
        for (int i = 0; i < C / 4; ++i) {
            const float4 f = src[i];
            v[4 * i] = f.x;
            v[4 * i + 1] = f.y;
            v[4 * i + 2] = f.z;
            v[4 * i + 3] = f.w;
        }
        uint32_t hits = 0;
#pragma unroll
        for (int i = 0; i < C; ++i)
            if (jb + i < K && v[i] >= ol.thr) hits |= 1u << i;
        const int n = __popc(hits);
        int incl = n;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int o = __shfl_up(incl, d, 64);
            if (lane >= d) incl += o;
        }
        if (lane == 63) wave_tot[wave] = incl;
        __syncthreads();
        int slot = base + incl - n;
        for (int w = 0; w < wave; ++w) slot += wave_tot[w];
        base += wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
#pragma unroll
        for (int i = 0; i < C; ++i) {
            if (jb + i >= K) break;
            const bool hit = (hits >> i) & 1u;
            if (lead) {
                ol.mask[jb + i] = hit ? 0.0f : 1.0f;
                if (hit) ol.idx[slot] = (int32_t)(jb + i);
            }
            if (hit && slot < ol.cap) s_idx[slot] = (int32_t)(jb + i);
            slot += hit;
        }
        __syncthreads();  // wave_tot is rewritten by the next pass; s_idx complete
    }
    if (lead && tid == 0) {
        *ol.count = base;
        if (ol.count_out) *ol.count_out = base;
    }
    const int64_t cnt = base;
    if (cnt == 0 || cnt > ol.cap) return;  // nothing, or the GEMM reads x and w directly
    // Four elements per thread per round, their loads issued together
    // (indices past the end clamped to the last element, whose value is
    // then not stored).
    const int64_t nx = cnt * M, total = nx + cnt * ol.N;
    const int64_t stride = (int64_t)ol.blocks * 256;
    constexpr int U = 4;
    for (int64_t e0 = (int64_t)b * 256 + tid; e0 < total; e0 += U * stride) {
        float val[U];
        int64_t at[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int64_t e = e0 + u * stride;
            e = e < total ? e : total - 1;
            const bool isx = e < nx;
            const int64_t f = isx ? e : e - nx, rows = isx ? M : ol.N;
            const int64_t t = f / rows, r = f - t * rows;
            const uint16_t *src = isx ? x16 : ol.w16;
            val[u] = (float)__builtin_bit_cast(_Float16, src[r * K + s_idx[t]]);
            at[u] = e;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (e0 + u * stride >= total) break;
            const int64_t e = at[u];
            if (e < nx) ol.xo[e] = val[u];
            else ol.wo[e - nx] = val[u];
        }
    }
}

// One 16-byte vector of a row widened to fp32, times the row multiplier rm
// (HAS_ROW) and the column multipliers (HAS_MUL: from LDS when staged, else
// from global memory; in the LLM.int8() mask mode those are the column
// maxima, turned into 1 / 0 here).
template <int DT, bool HAS_MUL, bool MUL_LDS, bool HAS_ROW = false>
__device__ __forceinline__ void scaled(const uint4 &raw, const float *__restrict__ mul,
                                       int64_t e0, float *v, float rm = 1.0f,
                                       const OutlierList *ol = nullptr) {
    constexpr int V = Vec<DT>::n;
    widen16<DT>(raw, v);
    if constexpr (HAS_ROW) {
#pragma unroll
        for (int i = 0; i < V; ++i) v[i] = v[i] * rm;
    }
    if constexpr (HAS_MUL) {
        float m[V];
        if constexpr (MUL_LDS) {
#pragma unroll
            for (int i = 0; i < V / 4; ++i) {
                const float4 t = smul4[e0 / 4 + i];
                m[4 * i] = t.x;
                m[4 * i + 1] = t.y;
                m[4 * i + 2] = t.z;
                m[4 * i + 3] = t.w;
            }
        } else {
            load_mul<DT>(mul, e0, m);
            if (ol && ol->on) {
#pragma unroll
                for (int i = 0; i < V; ++i) m[i] = keep(m[i], ol->thr);
            }
        }
#pragma unroll
        for (int i = 0; i < V; ++i) v[i] = v[i] * m[i];
    }
}

// Four values -> four e4m3 bytes (clamped to the finite range first: the
// conversion does not saturate).
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d, float inv) {
    const float za = __builtin_amdgcn_fmed3f(a * inv, -448.0f, 448.0f);
    const float zb = __builtin_amdgcn_fmed3f(b * inv, -448.0f, 448.0f);
    const float zc = __builtin_amdgcn_fmed3f(c * inv, -448.0f, 448.0f);
    const float zd = __builtin_amdgcn_fmed3f(d * inv, -448.0f, 448.0f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(za, zb, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(zc, zd, w, true);
    return (uint32_t)w;
}

// Four values -> four int8 codes: clamp(round_half_even(fl(v * inv)), +-127).
// Adding 1.5 2^23 to a value below 2^22 in magnitude rounds it to an integer,
// half to even, and leaves that integer's two's complement low byte in the
// low byte of the sum's bits; v_perm gathers the four low bytes.  With a
// per-row step (CLAMP = false) |fl(v * fl(127 / a))| <= 127 (1 + 2^-24)^2
// because |v| <= a, so the clamp cannot act; with a fixed step it clamps
// first (rounding and clamping commute at integer bounds).
template <bool CLAMP>
__device__ __forceinline__ uint32_t pack_i8x4(float a, float b, float c, float d, float inv) {
    float z[4] = {a * inv, b * inv, c * inv, d * inv};
    uint32_t u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (CLAMP) z[i] = __builtin_amdgcn_fmed3f(z[i], -127.0f, 127.0f);
        u[i] = __float_as_uint(z[i] + 12582912.0f);
    }
    return __builtin_amdgcn_perm(__builtin_amdgcn_perm(u[3], u[2], 0x0c0c0400u),
                                 __builtin_amdgcn_perm(u[1], u[0], 0x0c0c0400u), 0x05040100u);
}

template <bool FP8> struct QMax;
template <> struct QMax<false> { static constexpr float v = 127.0f; };
template <> struct QMax<true> { static constexpr float v = 448.0f; };

// NT: nontemporal stores, for outputs larger than the last-level cache
// (they are not read back before being evicted anyway, and streaming them
// past the caches measured 6.1 TB/s against 5.4 for plain stores on a
// 940 MB -> 470 MB stream; below the cache size plain stores are faster and
// leave the codes cached for the GEMM that reads them next).
typedef unsigned int u2v __attribute__((ext_vector_type(2)));
template <bool NT>
__device__ __forceinline__ void st_codes(int8_t *p, uint32_t a, uint32_t b) {
    if constexpr (NT) __builtin_nontemporal_store(u2v{a, b}, reinterpret_cast<u2v *>(p));
    else *reinterpret_cast<uint2 *>(p) = make_uint2(a, b);
}
template <bool NT>
__device__ __forceinline__ void st_codes(int8_t *p, uint32_t a) {
    if constexpr (NT) __builtin_nontemporal_store(a, reinterpret_cast<uint32_t *>(p));
    else *reinterpret_cast<uint32_t *>(p) = a;
}

template <int DT, bool FP8, bool CLAMP, bool NT = false>
__device__ __forceinline__ void store_q(int8_t *__restrict__ q, int64_t e0, const float *v,
                                        float inv) {
    if constexpr (FP8) {
        if constexpr (Vec<DT>::n == 8)
            st_codes<NT>(q + e0, pack_fp8x4(v[0], v[1], v[2], v[3], inv),
                         pack_fp8x4(v[4], v[5], v[6], v[7], inv));
        else
            st_codes<NT>(q + e0, pack_fp8x4(v[0], v[1], v[2], v[3], inv));
    } else if constexpr (Vec<DT>::n == 8) {
        st_codes<NT>(q + e0, pack_i8x4<CLAMP>(v[0], v[1], v[2], v[3], inv),
                     pack_i8x4<CLAMP>(v[4], v[5], v[6], v[7], inv));
    } else {
        st_codes<NT>(q + e0, pack_i8x4<CLAMP>(v[0], v[1], v[2], v[3], inv));
    }
}

// mul comes from LDS when it fits (K <= kMulLds floats): it is read once per
// block instead of once per row, and - more important - reading it from
// global memory inside the store loop would make each iteration wait for
// the earlier stores as well (vmcnt counts loads and stores alike).
constexpr int kMulLds = 16384;

// ITS > 0: the row is held in registers, ITS 16-byte vectors per lane, with
// out-of-range indices clamped to the row's last vector (loaded but not
// used) so every load is unconditional: a load inside a lane-divergent
// branch makes the compiler wait for all earlier memory operations first,
// which would serialize the row's loads.  ITS = 0: rows longer than
// 16 x 64 vectors, streamed twice (the second pass hits L2).
template <int DT, bool HAS_MUL, bool DYN, int ITS, bool MUL_LDS, bool HAS_ROW, bool FP8,
          bool NTS, bool NTL>
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint4 *__restrict__ x,
                                                         int64_t rows, int64_t K,
                                                         const float *__restrict__ mul_g,
                                                         const float *__restrict__ row_mul,
                                                         const float *__restrict__ static_scale,
                                                         int8_t *__restrict__ q,
                                                         float *__restrict__ scale,
                                                         int rows_per_wave, OutlierList ol) {
    constexpr int V = Vec<DT>::n;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (ol.on) {
        const int first = (int)gridDim.x - ol.blocks;
        if ((int)blockIdx.x >= first) {
            outlier_side_block(mul_g, reinterpret_cast<const uint16_t *>(x), K, ol,
                               (int)blockIdx.x - first);
            return;
        }
    }
    const int64_t bid = blockIdx.x;  // row block
    if (!DYN && bid == 0 && threadIdx.x == 0) scale[0] = static_scale[0];
    // The multiplier's address space is fixed at compile time (an LDS or a
    // global pointer), so its reads are ds_read / global_load, never flat.
    const float *mul = mul_g;
    if constexpr (HAS_MUL && MUL_LDS) {
        // Four 16-byte loads per thread in flight at once (indices past the
        // end clamped to the last vector, not stored): one memory latency
        // per 4096 multipliers instead of one per 1024.
        const float4 *src = reinterpret_cast<const float4 *>(mul_g);
        const int64_t n4 = K / 4;
        for (int64_t i0 = threadIdx.x; i0 < n4; i0 += 4 * 256) {
            float4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t i = i0 + u * 256;
                v[u] = src[i < n4 ? i : n4 - 1];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t i = i0 + u * 256;
                if (i < n4) smul4[i] = ol.on ? keep4(v[u], ol.thr) : v[u];
            }
        }
        __syncthreads();
    }
    const int64_t nvec = K / V;
    const float inv_static = DYN ? 0.0f : static_scale[1];

    // Rows of this wave: ((block * rows_per_wave + i) * 4 + wave).  The wave
    // index is made explicitly uniform so row bounds become scalar branches.
    const int64_t wv = __builtin_amdgcn_readfirstlane(wave);
    auto row_of = [&](int i) { return (bid * rows_per_wave + i) * 4 + wv; };

    if constexpr (DYN && ITS > 0) {
        // Two rows in flight per wave: row i + 1's loads are issued before
        // row i's stores, so waiting for them never waits for those stores
        // (vector memory operations complete in issue order).
        auto load_row = [&](int64_t r, uint4 (&b)[ITS]) {
            const uint4 *xr = x + r * nvec;
#pragma unroll
            for (int it = 0; it < ITS; ++it) {
                const int64_t vi = lane + (int64_t)it * kWave;
                b[it] = ld16<NTL>(xr + (vi < nvec ? vi : nvec - 1));
            }
        };
        auto finish_row = [&](int64_t r, const uint4 (&b)[ITS]) {
            const float rm = HAS_ROW ? row_mul[r] : 1.0f;
            float a = 0.0f;
#pragma unroll
            for (int it = 0; it < ITS; ++it) {
                const int64_t vi = lane + (int64_t)it * kWave;
                const int64_t vc = vi < nvec ? vi : nvec - 1;
                float v[V];
                scaled<DT, HAS_MUL, MUL_LDS, HAS_ROW>(b[it], mul, vc * V, v, rm, &ol);
#pragma unroll
                for (int i = 0; i < V; ++i) a = fmaxf(a, fabsf(v[i]));
            }
            a = wave_max(a);
            if (!(a > 1e-8f)) a = 1e-8f;
            const float inv = QMax<FP8>::v / a;
            if (lane == 0) scale[r] = a / QMax<FP8>::v;
            int8_t *qr = q + r * K;
#pragma unroll
            for (int it = 0; it < ITS; ++it) {
                // Recompute the scaled values from the raw row rather than
                // keep ITS*V floats alive across the reduction (which would
                // not fit next to a second row in flight).
                uint4 raw = b[it];
                asm volatile("" : "+v"(raw.x), "+v"(raw.y), "+v"(raw.z), "+v"(raw.w));
                const int64_t vi = lane + (int64_t)it * kWave;
                if (vi < nvec) {
                    float v[V];
                    scaled<DT, HAS_MUL, MUL_LDS, HAS_ROW>(raw, mul, vi * V, v, rm, &ol);
                    store_q<DT, FP8, false, NTS>(qr, vi * V, v, inv);
                }
            }
        };
        uint4 b0[ITS], b1[ITS];
        int64_t r0 = row_of(0);
        if (r0 >= rows) return;
        load_row(r0, b0);
        for (int i = 0;; i += 2) {
            const int64_t r1 = row_of(i + 1);
            const bool h1 = i + 1 < rows_per_wave && r1 < rows;
            if (h1) load_row(r1, b1);
            finish_row(r0, b0);
            if (!h1) break;
            const int64_t r2 = row_of(i + 2);
            const bool h2 = i + 2 < rows_per_wave && r2 < rows;
            if (h2) load_row(r2, b0);
            finish_row(r1, b1);
            if (!h2) break;
            r0 = r2;
        }
        return;
    }

    for (int rw = 0; rw < rows_per_wave; ++rw) {
        const int64_t r = row_of(rw);
        if (r >= rows) break;
        const uint4 *xr = x + r * nvec;
        int8_t *qr = q + r * K;
        if constexpr (DYN) {
            const float rm = HAS_ROW ? row_mul[r] : 1.0f;
            float a = 0.0f;
            for (int64_t vi = lane; vi < nvec; vi += kWave) {
                float v[V];
                scaled<DT, HAS_MUL, MUL_LDS, HAS_ROW>(xr[vi], mul, vi * V, v, rm, &ol);
#pragma unroll
                for (int i = 0; i < V; ++i) a = fmaxf(a, fabsf(v[i]));
            }
            a = wave_max(a);
            if (!(a > 1e-8f)) a = 1e-8f;
            const float inv = QMax<FP8>::v / a;
            if (lane == 0) scale[r] = a / QMax<FP8>::v;
            for (int64_t vi = lane; vi < nvec; vi += kWave) {
                float v[V];
                scaled<DT, HAS_MUL, MUL_LDS, HAS_ROW>(xr[vi], mul, vi * V, v, rm, &ol);
                store_q<DT, FP8, false, NTS>(qr, vi * V, v, inv);
            }
        } else {
            for (int64_t vi = lane; vi < nvec; vi += kWave) {
                float v[V];
                scaled<DT, HAS_MUL, MUL_LDS>(xr[vi], mul, vi * V, v);
                store_q<DT, FP8, true, NTS>(qr, vi * V, v, inv_static);
            }
        }
    }
}

// Few rows (fewer than the chip's wave slots): one 256-thread block per row,
// ITS 16-byte vectors per thread, all loads (row and multiplier) issued
// before the reduction; the row maximum is combined across the 4 waves
// through LDS.  Out-of-range vector indices are clamped to the row's last
// vector (loaded, not used) so every load is unconditional.
template <int DT, bool HAS_MUL, bool DYN, int ITS, bool HAS_ROW, bool FP8>
__global__ __launch_bounds__(256) void quant_row_block_kernel(const uint4 *__restrict__ x,
                                                              int64_t K,
                                                              const float *__restrict__ mul,
                                                              const float *__restrict__ row_mul,
                                                              const float *__restrict__ static_scale,
                                                              int8_t *__restrict__ q,
                                                              float *__restrict__ scale,
                                                              OutlierList ol) {
    constexpr int V = Vec<DT>::n;
    __shared__ float wmax[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (ol.on) {
        const int first = (int)gridDim.x - ol.blocks;
        if ((int)blockIdx.x >= first) {
            outlier_side_block(mul, reinterpret_cast<const uint16_t *>(x), K, ol,
                               (int)blockIdx.x - first);
            return;
        }
    }
    const int64_t r = blockIdx.x;
    if (!DYN && r == 0 && tid == 0) scale[0] = static_scale[0];
    const int64_t nvec = K / V;
    const uint4 *xr = x + r * nvec;
    uint4 raw[ITS];
    float m[HAS_MUL ? ITS : 1][HAS_MUL ? V : 1];
#pragma unroll
    for (int it = 0; it < ITS; ++it) {
        const int64_t vi = tid + (int64_t)it * 256;
        const int64_t vc = vi < nvec ? vi : nvec - 1;
        raw[it] = ld16<false>(xr + vc);  // at most 2048 rows: an input that may be read again
        if constexpr (HAS_MUL) load_mul<DT>(mul, vc * V, m[it]);
    }
    if constexpr (HAS_MUL) {
        if (ol.on) {
#pragma unroll
            for (int it = 0; it < ITS; ++it)
#pragma unroll
                for (int i = 0; i < V; ++i) m[it][i] = keep(m[it][i], ol.thr);
        }
    }
    const float rm = HAS_ROW ? row_mul[r] : 1.0f;
    float inv;
    if constexpr (DYN) {
        float a = 0.0f;
#pragma unroll
        for (int it = 0; it < ITS; ++it) {
            const int64_t vi = tid + (int64_t)it * 256;
            float v[V];
            widen16<DT>(raw[it], v);
#pragma unroll
            for (int i = 0; i < V; ++i) {
                if constexpr (HAS_ROW) v[i] = v[i] * rm;
                if constexpr (HAS_MUL) v[i] = v[i] * m[it][i];
                if (vi < nvec) a = fmaxf(a, fabsf(v[i]));
            }
        }
        a = wave_max(a);
        if (lane == 0) wmax[wave] = a;
        __syncthreads();
        a = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
        if (!(a > 1e-8f)) a = 1e-8f;
        inv = QMax<FP8>::v / a;
        if (tid == 0) scale[r] = a / QMax<FP8>::v;
    } else {
        inv = static_scale[1];
    }
    int8_t *qr = q + r * K;
#pragma unroll
    for (int it = 0; it < ITS; ++it) {
        const int64_t vi = tid + (int64_t)it * 256;
        if (vi < nvec) {
            float v[V];
            widen16<DT>(raw[it], v);
            if constexpr (HAS_ROW) {
#pragma unroll
                for (int i = 0; i < V; ++i) v[i] = v[i] * rm;
            }
            if constexpr (HAS_MUL) {
#pragma unroll
                for (int i = 0; i < V; ++i) v[i] = v[i] * m[it][i];
            }
            store_q<DT, FP8, !DYN>(qr, vi * V, v, inv);
        }
    }
}

template <int DT, bool HAS_MUL, bool DYN, bool HAS_ROW = false, bool FP8 = false>
static void launch_q(const void *x, int64_t rows, int64_t K, const float *mul,
                     const float *static_scale, int8_t *q, float *scale, hipStream_t stream,
                     const float *row_mul = nullptr, const OutlierList *olp = nullptr) {
    OutlierList ol = olp ? *olp : OutlierList{};
    // LLM.int8(): extra blocks for the outlier list and the side operands,
    // about one per 128 rows of x and w (a few gathered values per thread
    // for a few outlier columns).
    int64_t extra = 0;
    if (ol.on) {
        extra = (ol.M + ol.N) / 128;
        extra = extra < 1 ? 1 : extra > 64 ? 64 : extra;
        ol.blocks = (int)extra;
    }
    auto *xv = reinterpret_cast<const uint4 *>(x);
    const int64_t nvec = K / Vec<DT>::n;
    // Fewer rows than ~2 waves per SIMD of the chip, and long enough rows:
    // a block per row.
    if (rows < 2048 && nvec >= 256 && nvec <= 8 * 256) {
        const int64_t its = (nvec + 255) / 256;
        dim3 grid((unsigned)(rows + extra)), block(256);
#define SQ_B(ITS) \
    quant_row_block_kernel<DT, HAS_MUL, DYN, ITS, HAS_ROW, FP8><<<grid, block, 0, stream>>>(   \
        xv, K, mul, row_mul, static_scale, q, scale, ol)
        if (its <= 1) SQ_B(1);
        else if (its <= 2) SQ_B(2);
        else if (its <= 4) SQ_B(4);
        else SQ_B(8);
#undef SQ_B
        return;
    }
    // Codes larger than the 256 MB last-level cache are stored nontemporally.
    const bool nts = rows * K > (int64_t)256 << 20;
    // Rows per wave: enough blocks to fill the chip (>= ~1024), more rows
    // per block when there are plenty, so the multiplier is staged rarely:
    // up to 8 with plain stores (a3's 28672 rows: 7, 106 us against 112 with
    // 2), up to MAX_RPW_NT with nontemporal ones (the 65536-row stream:
    // 2 rows, 240 us against 265 with 8).
    constexpr int64_t MAX_RPW_NT = 2;
    int64_t rpw = rows / (4 * 1024);
    if (rpw < 1) rpw = 1;
    if (rpw > (nts ? MAX_RPW_NT : 8)) rpw = nts ? MAX_RPW_NT : 8;
    const int64_t blocks = (rows + 4 * rpw - 1) / (4 * rpw);
    const bool mul_lds = HAS_MUL && K <= kMulLds;
    const size_t shmem = mul_lds ? (size_t)K * sizeof(float) : 0;
    dim3 grid((unsigned)(blocks + extra)), block(256);
    const int64_t nit = (nvec + kWave - 1) / kWave;  // vectors per lane
    const int its = !DYN ? 0 : nit <= 2 ? 2 : nit <= 4 ? 4 : nit <= 8 ? 8 : nit <= 16 ? 16 : 0;
    // Inputs larger than the caches are loaded nontemporally (codes
    // beyond the cache imply such an input).
    const bool ntl = nts || rows * K * dt_bytes(DT) > kNtLoadBytes;
#define SQ_Q(ITS, LDS, NT, NL)                                                                  \
    quant_rows_kernel<DT, HAS_MUL, DYN, ITS, LDS, HAS_ROW, FP8, NT, NL><<<grid, block, shmem,      \
                                                                          stream>>>(            \
        xv, rows, K, mul, row_mul, static_scale, q, scale, (int)rpw, ol)
#define SQ_QL(ITS)                                           \
    do {                                                     \
        if (mul_lds && nts) SQ_Q(ITS, true, true, true);     \
        else if (mul_lds && ntl) SQ_Q(ITS, true, false, true); \
        else if (mul_lds) SQ_Q(ITS, true, false, false);     \
        else if (nts) SQ_Q(ITS, false, true, true);          \
        else if (ntl) SQ_Q(ITS, false, false, true);         \
        else SQ_Q(ITS, false, false, false);                 \
    } while (0)
    switch (its) {
        case 2: SQ_QL(2); break;
        case 4: SQ_QL(4); break;
        case 8: SQ_QL(8); break;
        case 16: SQ_QL(16); break;
        default: SQ_QL(0); break;
    }
#undef SQ_QL
#undef SQ_Q
}

template <int DT>
static void launch_dt_fp8(const void *x, int64_t rows, int64_t K, const float *mul, int dynamic,
                          const float *static_scale, int8_t *q, float *scale,
                          hipStream_t stream) {
    if (mul) {
        if (dynamic) launch_q<DT, true, true, false, true>(x, rows, K, mul, static_scale, q, scale, stream);
        else launch_q<DT, true, false, false, true>(x, rows, K, mul, static_scale, q, scale, stream);
    } else {
        if (dynamic) launch_q<DT, false, true, false, true>(x, rows, K, mul, static_scale, q, scale, stream);
        else launch_q<DT, false, false, false, true>(x, rows, K, mul, static_scale, q, scale, stream);
    }
}

template <int DT>
static void launch_dt(const void *x, int64_t rows, int64_t K, const float *mul, int dynamic,
                      const float *static_scale, int8_t *q, float *scale, hipStream_t stream,
                      const float *row_mul, const OutlierList *ol) {
    if (ol) {  // LLM.int8(): per-row steps over the kept columns
        launch_q<DT, true, true>(x, rows, K, mul, static_scale, q, scale, stream, nullptr, ol);
        return;
    }
    if (row_mul) {  // weights only: per-row steps
        if (mul) launch_q<DT, true, true, true>(x, rows, K, mul, static_scale, q, scale, stream, row_mul);
        else launch_q<DT, false, true, true>(x, rows, K, mul, static_scale, q, scale, stream, row_mul);
        return;
    }
    if (mul) {
        if (dynamic) launch_q<DT, true, true>(x, rows, K, mul, static_scale, q, scale, stream);
        else launch_q<DT, true, false>(x, rows, K, mul, static_scale, q, scale, stream);
    } else {
        if (dynamic) launch_q<DT, false, true>(x, rows, K, mul, static_scale, q, scale, stream);
        else launch_q<DT, false, false>(x, rows, K, mul, static_scale, q, scale, stream);
    }
}

void launch_quant_rows_fp8(const void *x, int dt, int64_t rows, int64_t K, const float *mul,
                           int dynamic, const float *static_scale, uint8_t *q, float *scale,
                           hipStream_t stream) {
    if (rows == 0) {
        if (!dynamic) launch_copy_f32(static_scale, scale, stream);
        return;
    }
    if (K <= 0) return;  // rejected by the C ABI: the kernels clamp to the last vector
    int8_t *qq = reinterpret_cast<int8_t *>(q);
    if (dt == F32) launch_dt_fp8<F32>(x, rows, K, mul, dynamic, static_scale, qq, scale, stream);
    else if (dt == F16) launch_dt_fp8<F16>(x, rows, K, mul, dynamic, static_scale, qq, scale, stream);
    else launch_dt_fp8<BF16>(x, rows, K, mul, dynamic, static_scale, qq, scale, stream);
}

void launch_quant_rows(const void *x, int dt, int64_t rows, int64_t K, const float *mul,
                       int dynamic, const float *static_scale, int8_t *q, float *scale,
                       hipStream_t stream, const float *row_mul, const OutlierList *ol) {
    if (rows == 0) {
        if (!dynamic)  // the per-tensor step is still reported
            launch_copy_f32(static_scale, scale, stream);
        return;
    }
    if (K <= 0) return;  // rejected by the C ABI: the kernels clamp to the last vector
    if (dt == F32) launch_dt<F32>(x, rows, K, mul, dynamic, static_scale, q, scale, stream, row_mul, ol);
    else if (dt == F16) launch_dt<F16>(x, rows, K, mul, dynamic, static_scale, q, scale, stream, row_mul, ol);
    else launch_dt<BF16>(x, rows, K, mul, dynamic, static_scale, q, scale, stream, row_mul, ol);
}

}  // namespace sq
