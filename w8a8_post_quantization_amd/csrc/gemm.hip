// int8 x int8 -> int32 GEMM with the outer-product dequant epilogue
//   acc[m, n] = sum_k xq[m, k] * wq[n, k]                (exact int32)
//   y[m, n]   = fl(fl((float)acc) * fl(dx_m * dw_n))     (+ LLM.int8() side)
// (the SmoothQuant tutorial page: Y = diag(dX) X_int8 W_int8 diag(dW); the
// xdnf.cn LLM.int8() explainer §2.1: int32 accumulation and the c_x (x) c_w
// outer product; §2.2 for the fp16 side product over outlier columns).
//
// Two kernels, same bits:
//  * gemm_tile: M > 32.  256 threads = 4 waves, block tile BM x BN, K staged
//    through LDS 128 bytes at a time, double-buffered (global -> registers
//    -> LDS while the MFMAs consume the other buffer).  Each wave owns a
//    (BM/WM) x (BN/WN) sub-tile of v_mfma_i32_32x32x32_i8 fragments.  Both
//    operands are K-contiguous, so a lane's 16-byte MFMA operand is one
//    ds_read_b128.  LDS rows are 128 bytes; chunk c of row r lives at slot
//    c ^ swz(r), which keeps ds_write_b128 and ds_read_b128 free of bank
//    conflicts whether 8 or 16 lanes are served per cycle.
//  * gemm_skinny: M <= 32 (decode).  HBM-bound on the weight stream: a block
//    owns 32 weight rows, its 4 waves split K, v_mfma_i32_16x16x64_i8 with
//    weight rows as the MFMA rows and tokens (padded to 16 / 32) as columns;
//    int32 partials are summed exactly through LDS.
//
// An integer dot product does not depend on the order of its terms, so the
// assignment of K bytes to MFMA lanes only has to be the same for both
// operands; the float epilogue is per element and order-free.
#include <stdlib.h>

#include "sq_device.h"
#include "sq_launch.h"

namespace sq {

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int YDT>
__device__ __forceinline__ void store_y(void *y, int64_t i, float v) {
    reinterpret_cast<typename OutT<YDT>::T *>(y)[i] = narrow<YDT>(v);
}

__device__ __forceinline__ float h2f(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

struct GemmArgs {
    const int8_t *xq;
    const int8_t *wq;
    int M, N, K;
    const float *xs;
    int xs_per_row;
    const float *ws;
    void *y;
    int32_t *acc_out;
    const uint16_t *x16;   // side term (LLM.int8()), or null
    const uint16_t *w16;
    const int32_t *idx;
    const int32_t *count;
    int tiles_n;
};

// Each thread fetches (at most) one row step and one column step at kernel
// start; they are written to LDS only after the main loop, when the loads
// have long completed.
template <int BM, int BN>
struct TileScales {
    float x, w;
    __device__ __forceinline__ void load(const GemmArgs &p, int m0, int n0) {
        const int t = threadIdx.x;
        x = 0.0f;
        w = 0.0f;
        if (t < BM) {
            const int m = m0 + t < p.M ? m0 + t : p.M - 1;
            x = p.xs[p.xs_per_row ? m : 0];
        }
        if (t < BN) {
            const int n = n0 + t < p.N ? n0 + t : p.N - 1;
            w = p.ws[n];
        }
    }
    __device__ __forceinline__ void publish(float *sx, float *sw) const {
        const int t = threadIdx.x;
        if (t < BM) sx[t] = x;
        if (t < BN) sw[t] = w;
    }
};

// Dequant epilogue shared by the tiled kernels.  32x32 accumulator layout:
// lane l, register v holds row 8*(v/4) + 4*(l/32) + (v%4), column l%32 of
// the fragment.  With SIDE, the LLM.int8() fp16 side product over the
// outlier columns is accumulated in ascending column order, staged through
// LDS 32 columns at a time (rows padded to 33 floats), and added to the
// dequantized value before narrowing.
//
// The row and column steps come from LDS (sx[BM], sw[BN]): reading them from
// global memory inside the store loop would make every iteration wait for
// all earlier stores too (vmcnt counts loads and stores alike).
template <int BM, int BN, int WM, int WN, int YDT, bool SIDE>
__device__ __forceinline__ void epilogue(const GemmArgs &p,
                                         int16v (&acc)[BM / WM / 32][BN / WN / 32],
                                         int8_t *smem, const float *sx, const float *sw, int m0,
                                         int n0) {
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int fr = lane & 31, fh = lane >> 5;
    const int M = p.M, N = p.N, K = p.K;
    float dw[FN];
    int ncol[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        ncol[j] = n0 + wn * WTN + j * 32 + fr;
        dw[j] = sw[wn * WTN + j * 32 + fr];
    }
    float side[SIDE ? FM : 1][SIDE ? FN : 1][16];
    if constexpr (SIDE) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) side[i][j][v] = 0.0f;
        float *xo = reinterpret_cast<float *>(smem);
        float *wo = xo + BM * 33;
        const int cnt = *p.count;
        for (int t0 = 0; t0 < cnt; t0 += 32) {
            const int tn = cnt - t0 < 32 ? cnt - t0 : 32;
            __syncthreads();
            for (int e = tid; e < BM * 32; e += 256) {
                const int r = e >> 5, t = e & 31;
                const int gr = m0 + r < M ? m0 + r : M - 1;
                xo[r * 33 + t] = t < tn ? h2f(p.x16[(int64_t)gr * K + p.idx[t0 + t]]) : 0.0f;
            }
            for (int e = tid; e < BN * 32; e += 256) {
                const int r = e >> 5, t = e & 31;
                const int gr = n0 + r < N ? n0 + r : N - 1;
                wo[r * 33 + t] = t < tn ? h2f(p.w16[(int64_t)gr * K + p.idx[t0 + t]]) : 0.0f;
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int rl = wm * WTM + i * 32 + 8 * (v >> 2) + 4 * fh + (v & 3);
                        const int cl = wn * WTN + j * 32 + fr;
                        float s = side[i][j][v];
                        for (int t = 0; t < tn; ++t) {
                            const float prod = xo[rl * 33 + t] * wo[cl * 33 + t];
                            s = s + prod;
                        }
                        side[i][j][v] = s;
                    }
        }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int ml = wm * WTM + i * 32 + 8 * (v >> 2) + 4 * fh + (v & 3);
            const int m = m0 + ml;
            if (m >= M) continue;
            const float dx = sx[ml];
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                if (ncol[j] >= N) continue;
                const int64_t o = (int64_t)m * N + ncol[j];
                const float c = dx * dw[j];
                const float deq = (float)acc[i][j][v] * c;
                if constexpr (SIDE) store_y<YDT>(p.y, o, deq + side[i][j][v]);
                else store_y<YDT>(p.y, o, deq);
                if (p.acc_out) p.acc_out[o] = acc[i][j][v];
            }
        }
}

template <int BM, int BN, int WM, int WN, int YDT, bool SIDE>
__global__ __launch_bounds__(256, 1) void gemm_tile(GemmArgs p) {
    constexpr int BK = 128;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int A_PER_T = BM * 8 / 256, B_PER_T = BN * 8 / 256;
    static_assert(WM * WN == 4, "4 waves");
    static_assert(FM >= 1 && FN >= 1 && A_PER_T >= 1 && B_PER_T >= 1, "tile");

    __shared__ __attribute__((aligned(16))) int8_t smem[2 * (BM + BN) * BK];
    __shared__ float sx[BM], sw[BN];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int tile_m = blockIdx.x / p.tiles_n, tile_n = blockIdx.x % p.tiles_n;
    const int m0 = tile_m * BM, n0 = tile_n * BN;
    const int M = p.M, N = p.N, K = p.K;
    TileScales<BM, BN> scl;
    scl.load(p, m0, n0);

    // Global source rows of this thread's chunks (clamped: rows past the
    // edge load a valid duplicate row whose outputs are never stored).
    const int8_t *a_src[A_PER_T];
    int a_lds[A_PER_T], a_kc[A_PER_T];
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
        const int c = tid + 256 * i, r = c >> 3, kc = c & 7;
        const int gr = m0 + r < M ? m0 + r : M - 1;
        a_src[i] = p.xq + (int64_t)gr * K + kc * 16;
        a_kc[i] = kc * 16;
        a_lds[i] = r * BK + ((kc ^ swz(r)) << 4);
    }
    const int8_t *b_src[B_PER_T];
    int b_lds[B_PER_T], b_kc[B_PER_T];
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
        const int c = tid + 256 * i, r = c >> 3, kc = c & 7;
        const int gr = n0 + r < N ? n0 + r : N - 1;
        b_src[i] = p.wq + (int64_t)gr * K + kc * 16;
        b_kc[i] = kc * 16;
        b_lds[i] = BM * BK + r * BK + ((kc ^ swz(r)) << 4);
    }

    uint4 ra[A_PER_T], rb[B_PER_T];
    // Loads past the K tail read chunk 0 of the row instead and are zeroed
    // afterwards: unconditional loads keep the compiler from serializing them.
    auto load_global = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i) {
            const bool ok = k0 + a_kc[i] < K;
            const uint4 v = *reinterpret_cast<const uint4 *>(a_src[i] + (ok ? k0 : -a_kc[i]));
            ra[i] = ok ? v : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < B_PER_T; ++i) {
            const bool ok = k0 + b_kc[i] < K;
            const uint4 v = *reinterpret_cast<const uint4 *>(b_src[i] + (ok ? k0 : -b_kc[i]));
            rb[i] = ok ? v : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_lds = [&](int buf) {
        int8_t *base = smem + buf * (BM + BN) * BK;
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i) *reinterpret_cast<uint4 *>(base + a_lds[i]) = ra[i];
#pragma unroll
        for (int i = 0; i < B_PER_T; ++i) *reinterpret_cast<uint4 *>(base + b_lds[i]) = rb[i];
    };

    // Fragment read offsets: lane -> (row within 32, 16-byte K half).
    const int fr = lane & 31, fh = lane >> 5;
    int a_row[FM], b_row[FN];
#pragma unroll
    for (int f = 0; f < FM; ++f) a_row[f] = wm * WTM + f * 32 + fr;
#pragma unroll
    for (int f = 0; f < FN; ++f) b_row[f] = BM + wn * WTN + f * 32 + fr;

    int16v acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;

    const int nk = (K + BK - 1) / BK;
    if (nk > 0) {
        load_global(0);
        store_lds(0);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) load_global((kt + 1) * BK);
        const int8_t *base = smem + cur * (BM + BN) * BK;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int ch = 2 * ks + fh;
            int4v af[FM], bf[FN];
#pragma unroll
            for (int f = 0; f < FM; ++f)
                af[f] = *reinterpret_cast<const int4v *>(
                    base + a_row[f] * BK + ((ch ^ swz(a_row[f])) << 4));
#pragma unroll
            for (int f = 0; f < FN; ++f)
                bf[f] = *reinterpret_cast<const int4v *>(
                    base + b_row[f] * BK + ((ch ^ swz(b_row[f] - BM)) << 4));
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j],
                                                                       0, 0, 0);
        }
        if (kt + 1 < nk) store_lds(cur ^ 1);
        __syncthreads();
    }

    scl.publish(sx, sw);
    __syncthreads();
    epilogue<BM, BN, WM, WN, YDT, SIDE>(p, acc, smem, sx, sw, m0, n0);
}

// ---------------------------------------------------------------- pipelined

typedef __attribute__((address_space(3))) void lds_void_t;

// One direct-to-LDS load: 16 bytes per lane from `g` into LDS at
// lds_base + 16 * lane (lds_base wave-uniform, in M0).  Written as inline
// asm on purpose: the compiler treats every later LDS read as possibly
// aliasing an LDS write that is still in flight from the builtin form and
// waits for all of them (vmcnt(0)) before the read, which drains the whole
// prefetch ring each stage.  Here the kernel's own vmcnt waits and
// barriers order the ring.  The instruction has no register results; its
// address operands are read when it issues.  s_nop covers the M0-write ->
// LDS-DMA hazard.
__device__ __forceinline__ void lds_dma16(const void *g, uint32_t lds_base) {
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off"
        :
        : "v"(g), "s"(lds_base)
        : "memory", "m0");
}

// s_waitcnt vmcnt(N) leaving lgkmcnt / expcnt alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for the LDS ring only.  __syncthreads() carries a
// release fence that waits for every outstanding global load (vmcnt(0)),
// which would drain the in-flight stages; here each wave has already waited
// for its own stage loads with vmcnt(N), and only LDS traffic must be
// complete before the barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Vector store of 4 consecutive outputs (8 bytes for 16-bit types, 16 for
// fp32), narrowed with round-to-nearest-even.
template <int YDT>
__device__ __forceinline__ void store_y4(void *y, int64_t i, const float *v) {
    if constexpr (YDT == F32) {
        *reinterpret_cast<float4 *>(reinterpret_cast<float *>(y) + i) =
            make_float4(v[0], v[1], v[2], v[3]);
    } else {
        using T = typename OutT<YDT>::T;
        T h[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) h[q] = narrow<YDT>(v[q]);
        *reinterpret_cast<uint2 *>(reinterpret_cast<T *>(y) + i) = __builtin_bit_cast(uint2, h);
    }
}

// Epilogue of the K % 64 == 0 kernel.  The MFMAs there take weight rows as
// the A operand and tokens as B, so lane l, register v of fragment (i, j)
// holds output column n = 8*(v/4) + 4*(l/32) + (v%4) of n-fragment i and
// row m = l%32 of m-fragment j: four consecutive columns of one row per
// group of four registers, stored as one 8- or 16-byte vector.
template <int BM, int BN, int WM, int WN, int YDT, bool SIDE>
__device__ __forceinline__ void epilogue_nt(const GemmArgs &p,
                                            int16v (&acc)[BN / WN / 32][BM / WM / 32],
                                            int8_t *smem, const float *sx, const float *sw,
                                            int m0, int n0) {
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int fr = lane & 31, fh = lane >> 5;
    const int M = p.M, N = p.N, K = p.K;
    const bool vec_y = (N & 3) == 0 && ((uintptr_t)p.y & 15) == 0;
    const bool vec_a = (N & 3) == 0 && ((uintptr_t)p.acc_out & 15) == 0;
    float side[SIDE ? FN : 1][SIDE ? FM : 1][16];
    if constexpr (SIDE) {
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) side[i][j][v] = 0.0f;
        float *xo = reinterpret_cast<float *>(smem);
        float *wo = xo + BM * 33;
        const int cnt = *p.count;
        for (int t0 = 0; t0 < cnt; t0 += 32) {
            const int tn = cnt - t0 < 32 ? cnt - t0 : 32;
            __syncthreads();
            for (int e = tid; e < BM * 32; e += 256) {
                const int r = e >> 5, t = e & 31;
                const int gr = m0 + r < M ? m0 + r : M - 1;
                xo[r * 33 + t] = t < tn ? h2f(p.x16[(int64_t)gr * K + p.idx[t0 + t]]) : 0.0f;
            }
            for (int e = tid; e < BN * 32; e += 256) {
                const int r = e >> 5, t = e & 31;
                const int gr = n0 + r < N ? n0 + r : N - 1;
                wo[r * 33 + t] = t < tn ? h2f(p.w16[(int64_t)gr * K + p.idx[t0 + t]]) : 0.0f;
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int nl = wn * WTN + i * 32 + 8 * (v >> 2) + 4 * fh + (v & 3);
                        const int ml = wm * WTM + j * 32 + fr;
                        float sum = side[i][j][v];
                        for (int t = 0; t < tn; ++t) {
                            const float prod = xo[ml * 33 + t] * wo[nl * 33 + t];
                            sum = sum + prod;
                        }
                        side[i][j][v] = sum;
                    }
        }
    }
#pragma unroll
    for (int j = 0; j < FM; ++j) {
        const int ml = wm * WTM + j * 32 + fr;
        const int m = m0 + ml;
        const float dx = sx[ml];
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int nl = wn * WTN + i * 32 + 8 * g + 4 * fh;
                const int n = n0 + nl;
                const float4 dw4 = *reinterpret_cast<const float4 *>(sw + nl);
                const float dwq[4] = {dw4.x, dw4.y, dw4.z, dw4.w};
                float yv[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float c = dx * dwq[q];
                    const float deq = (float)acc[i][j][4 * g + q] * c;
                    if constexpr (SIDE) yv[q] = deq + side[i][j][4 * g + q];
                    else yv[q] = deq;
                }
                if (m < M) {
                    const int64_t o = (int64_t)m * N + n;
                    if (vec_y && n + 3 < N) {
                        store_y4<YDT>(p.y, o, yv);
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            if (n + q < N) store_y<YDT>(p.y, o + q, yv[q]);
                    }
                    if (p.acc_out) {
                        if (vec_a && n + 3 < N) {
                            *reinterpret_cast<int4 *>(p.acc_out + o) =
                                make_int4(acc[i][j][4 * g], acc[i][j][4 * g + 1],
                                          acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
                        } else {
#pragma unroll
                            for (int q = 0; q < 4; ++q)
                                if (n + q < N) p.acc_out[o + q] = acc[i][j][4 * g + q];
                        }
                    }
                }
            }
    }
}

// Scheduling pattern after the stage barrier: each MFMA is followed by one
// DS read (while any remain) and its share of the stage's direct loads.
template <int MQ, int RQ, int L, int R>
__device__ __forceinline__ void sched_tail() {
    if constexpr (R < MQ) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // MFMA
        if constexpr (R < RQ) __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);  // DS read
        constexpr int per = (L + MQ - 1) / MQ;
        constexpr int left = L - R * per;
        if constexpr (left > 0)
            __builtin_amdgcn_sched_group_barrier(0x020, left < per ? left : per, 1);  // VMEM read
        sched_tail<MQ, RQ, L, R + 1>();
    }
}

// K % 128 == 0.  K is staged 128 bytes at a time through an ST-deep LDS ring
// filled by direct-to-LDS loads (global_load_lds_dwordx4): each wave
// instruction moves 8 rows x 128 bytes, so every request to L2 is a whole
// 128-byte line (with 64-byte stages each line was fetched as two 64-byte
// requests, and the number of requests the vector L1 keeps in flight - not
// bytes or L2 bandwidth - capped the per-CU feed rate).  Lane l writes LDS
// bytes [16 l, 16 l + 16) of its 1 KiB block; the swizzle (see swz) is
// applied by choosing which global chunk each lane fetches.  All ST stages are
// in flight.
//
// Each stage is consumed as four 32-byte quarters with ping-pong fragment
// registers: a quarter's LDS reads overlap the previous quarter's MFMAs, and
// after the stage barrier the next stage's first reads overlap the last
// quarter's MFMAs, so the MFMA pipe does not wait for a full LDS round trip.
// Weight rows are the MFMA A operand (see epilogue_nt).
template <int BM, int BN, int WM, int WN, int ST, int YDT, bool SIDE>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 2))) void gemm_pp(
    GemmArgs p) {
    constexpr int BK = 128;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int LA = BM / 32, LB = BN / 32;  // load instructions per wave per stage
    constexpr int L = LA + LB;
    constexpr int STAGE = (BM + BN) * BK;
    static_assert(WM * WN == 4 && FM >= 1 && FN >= 1, "tile");
    static_assert(ST >= 2 && (ST - 1) * L < 64, "pipeline depth");

    __shared__ __attribute__((aligned(1024))) int8_t smem[ST * STAGE];
    __shared__ __attribute__((aligned(16))) float sx[BM], sw[BN];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int tile_m = blockIdx.x / p.tiles_n, tile_n = blockIdx.x % p.tiles_n;
    const int m0 = tile_m * BM, n0 = tile_n * BN;
    const int M = p.M, N = p.N, K = p.K;
    TileScales<BM, BN> scl;
    scl.load(p, m0, n0);

    const int8_t *a_src[LA];
    const int8_t *b_src[LB];
#pragma unroll
    for (int j = 0; j < LA; ++j) {
        const int row = (wave * LA + j) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ swz(row);
        const int gr = m0 + row < M ? m0 + row : M - 1;
        a_src[j] = p.xq + (int64_t)gr * K + c * 16;
    }
#pragma unroll
    for (int j = 0; j < LB; ++j) {
        const int row = (wave * LB + j) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ swz(row);
        const int gr = n0 + row < N ? n0 + row : N - 1;
        b_src[j] = p.wq + (int64_t)gr * K + c * 16;
    }
    // Stage s of K into ring slot `slot`: this wave's A blocks are the 1 KiB
    // blocks wave*LA + j of the slot, its B blocks follow the A tile at
    // wave*LB + j (the same blocks the global rows above were chosen for).
    const uint32_t waveu = (uint32_t)__builtin_amdgcn_readfirstlane(wave);
    const uint32_t lds_a = (uint32_t)(uintptr_t)(lds_void_t *)smem + waveu * (LA * 1024u);
    const uint32_t lds_b =
        (uint32_t)(uintptr_t)(lds_void_t *)smem + (uint32_t)(BM * BK) + waveu * (LB * 1024u);
    auto issue = [&](int s, int slot) {
        const uint32_t so = (uint32_t)(slot * STAGE);
        const int k0 = s * BK;
#pragma unroll
        for (int j = 0; j < LA; ++j) lds_dma16(a_src[j] + k0, lds_a + so + (uint32_t)(j * 1024));
#pragma unroll
        for (int j = 0; j < LB; ++j) lds_dma16(b_src[j] + k0, lds_b + so + (uint32_t)(j * 1024));
    };

    const int fr = lane & 31, fh = lane >> 5;
    const int fsw = swz(fr);  // fragment bases are multiples of 32 rows
    int off[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) off[q] = ((2 * q + fh) ^ fsw) << 4;
    auto read_frags = [&](int s, int q, int4v (&xf)[FM], int4v (&wf)[FN]) {
        const int8_t *base = smem + (s % ST) * STAGE + off[q];
#pragma unroll
        for (int f = 0; f < FM; ++f)
            xf[f] = *reinterpret_cast<const int4v *>(base + (wm * WTM + f * 32 + fr) * BK);
#pragma unroll
        for (int f = 0; f < FN; ++f)
            wf[f] = *reinterpret_cast<const int4v *>(base + BM * BK + (wn * WTN + f * 32 + fr) * BK);
    };

    int16v acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;
    auto mma = [&](const int4v (&xf)[FM], const int4v (&wf)[FN]) {
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wf[i], xf[j], acc[i][j], 0, 0, 0);
    };

    // Main loop.  Its two halves are branch-free so the scheduler can
    // interleave: a wave issues in order, so a ds_read (or direct load)
    // queued behind an MFMA that waits for the matrix core cannot issue; the
    // sched_group_barrier sequences place one memory instruction after each
    // MFMA, letting LDS traffic and the next stage's loads run under the
    // MFMAs.  Past the last stage, the free ring slot is refilled with the
    // last stage (never read), which keeps every iteration's load count -
    // and so the vmcnt arithmetic - the same; all loads are drained before
    // the epilogue.
    constexpr int RQ = FM + FN;       // ds_read_b128 per quarter
    constexpr int MQ = FM * FN;       // MFMAs per quarter
    static_assert(RQ <= MQ, "one read per MFMA slot");
    const int nk = K / BK;
#pragma unroll
    for (int s = 0; s < ST; ++s) issue(s < nk ? s : nk - 1, s);
    wait_vmcnt<(ST - 1) * L>();
    lds_barrier();
    int4v xa[FM], wa[FN], xb[FM], wb[FN];
    read_frags(0, 0, xa, wa);
    for (int kt = 0; kt < nk; ++kt) {
        read_frags(kt, 1, xb, wb);
        mma(xa, wa);
        read_frags(kt, 2, xa, wa);
        mma(xb, wb);
        read_frags(kt, 3, xb, wb);
        mma(xa, wa);
#pragma unroll
        for (int q = 0; q < 3; ++q) {
#pragma unroll
            for (int r = 0; r < RQ; ++r) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
            }
            __builtin_amdgcn_sched_group_barrier(0x008, MQ - RQ, 0);
        }
        wait_vmcnt<(ST - 2) * L>();  // stage kt + 1 has landed
        lds_barrier();               // every wave has read stage kt: its slot is free
        read_frags(kt + 1, 0, xa, wa);
        issue(kt + ST < nk ? kt + ST : nk - 1, kt % ST);
        mma(xb, wb);
        sched_tail<MQ, RQ, L, 0>();  // MFMA, DS read, direct loads, ...
    }
    wait_vmcnt<0>();
    scl.publish(sx, sw);
    __syncthreads();  // steps visible; the side term may reuse the ring
    epilogue_nt<BM, BN, WM, WN, YDT, SIDE>(p, acc, smem, sx, sw, m0, n0);
}

// ---------------------------------------------------------------- skinny

template <int FT, int YDT>
__global__ __launch_bounds__(256) void gemm_skinny(GemmArgs p) {
    constexpr int NR = 32;  // weight rows per block: two 16-row fragments
    __shared__ int red[4][2][FT][64 * 4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int M = p.M, N = p.N, K = p.K;
    const int n0 = blockIdx.x * NR;
    const int r16 = lane & 15, kg = (lane >> 4) * 16;

    const int8_t *wrow[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        const int n = n0 + f * 16 + r16;
        wrow[f] = p.wq + (int64_t)(n < N ? n : N - 1) * K + kg;
    }
    const int8_t *xrow[FT];
#pragma unroll
    for (int t = 0; t < FT; ++t) {
        const int m = t * 16 + r16;
        xrow[t] = p.xq + (int64_t)(m < M ? m : M - 1) * K + kg;
    }

    int4v acc[2][FT];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int t = 0; t < FT; ++t) acc[f][t] = int4v{0, 0, 0, 0};

    // Steps of this thread's outputs (n = n0 + tid % 32, m = tid / 32 + 8 q),
    // fetched before the K loop so the epilogue issues stores only.
    constexpr int EPT = NR * 16 * FT / 256;  // outputs per thread
    const int n_own = n0 + (tid & 31);
    const float w_own = p.ws[n_own < N ? n_own : N - 1];
    float x_own[EPT];
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
        const int m = (tid >> 5) + 8 * q;
        x_own[q] = p.xs[p.xs_per_row ? (m < M ? m : M - 1) : 0];
    }

    const int steps = (K + 63) / 64;
    const int per = (steps + 3) / 4;
    const int s0 = wave * per;
    const int s1 = s0 + per < steps ? s0 + per : steps;
    constexpr int U = 4;
    int s = s0;
    for (; s + U <= s1; s += U) {
        int4v a[U][2], b[U][FT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = (s + u) * 64;
            const bool ok = k + kg < K;
            const int kk = ok ? k : -kg;  // past the tail: load chunk 0, zero it
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                const int4v v = *reinterpret_cast<const int4v *>(wrow[f] + kk);
                a[u][f] = ok ? v : int4v{0, 0, 0, 0};
            }
#pragma unroll
            for (int t = 0; t < FT; ++t) {
                const int4v v = *reinterpret_cast<const int4v *>(xrow[t] + kk);
                b[u][t] = ok ? v : int4v{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
                for (int t = 0; t < FT; ++t)
                    acc[f][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u][f], b[u][t],
                                                                       acc[f][t], 0, 0, 0);
    }
    for (; s < s1; ++s) {
        const int k = s * 64;
        const bool ok = k + kg < K;
        const int kk = ok ? k : -kg;
        int4v a[2], b[FT];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            const int4v v = *reinterpret_cast<const int4v *>(wrow[f] + kk);
            a[f] = ok ? v : int4v{0, 0, 0, 0};
        }
#pragma unroll
        for (int t = 0; t < FT; ++t) {
            const int4v v = *reinterpret_cast<const int4v *>(xrow[t] + kk);
            b[t] = ok ? v : int4v{0, 0, 0, 0};
        }
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int t = 0; t < FT; ++t)
                acc[f][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[f], b[t], acc[f][t], 0, 0, 0);
    }

#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int t = 0; t < FT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) red[wave][f][t][v * 64 + lane] = acc[f][t][v];
    __syncthreads();

    // 16x16 accumulator layout: lane l, register v holds MFMA row
    // 4*(l/16) + v (a weight row) and column l%16 (a token).  Threads take
    // outputs with n fastest so stores of a token row are contiguous.
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
        const int e = tid + 256 * q;
        const int nl = e % NR, ml = e / NR;
        const int m = ml, n = n0 + nl;
        if (m >= M || n >= N) continue;
        const int f = nl >> 4, i = nl & 15, t = ml >> 4, j = ml & 15;
        const int l = (i >> 2) * 16 + j, v = i & 3;
        const int a = red[0][f][t][v * 64 + l] + red[1][f][t][v * 64 + l] +
                      red[2][f][t][v * 64 + l] + red[3][f][t][v * 64 + l];
        const float c = x_own[q] * w_own;
        const int64_t o = (int64_t)m * N + n;
        store_y<YDT>(p.y, o, (float)a * c);
        if (p.acc_out) p.acc_out[o] = a;
    }
}

// ---------------------------------------------------------------- launch

template <int BM, int BN, int WM, int WN, bool SIDE>
static void launch_tile_t(GemmArgs &a, int y_dt, hipStream_t stream) {
    const int tm = (a.M + BM - 1) / BM, tn = (a.N + BN - 1) / BN;
    a.tiles_n = tn;
    dim3 grid((unsigned)(tm * tn)), block(256);
    if (y_dt == F32) gemm_tile<BM, BN, WM, WN, F32, SIDE><<<grid, block, 0, stream>>>(a);
    else if (y_dt == F16) gemm_tile<BM, BN, WM, WN, F16, SIDE><<<grid, block, 0, stream>>>(a);
    else gemm_tile<BM, BN, WM, WN, BF16, SIDE><<<grid, block, 0, stream>>>(a);
}

template <int BM, int BN, int WM, int WN, int ST, bool SIDE>
static void launch_pipe_t(GemmArgs &a, int y_dt, hipStream_t stream) {
    const int tm = (a.M + BM - 1) / BM, tn = (a.N + BN - 1) / BN;
    a.tiles_n = tn;
    dim3 grid((unsigned)(tm * tn)), block(256);
    if (y_dt == F32) gemm_pp<BM, BN, WM, WN, ST, F32, SIDE><<<grid, block, 0, stream>>>(a);
    else if (y_dt == F16) gemm_pp<BM, BN, WM, WN, ST, F16, SIDE><<<grid, block, 0, stream>>>(a);
    else gemm_pp<BM, BN, WM, WN, ST, BF16, SIDE><<<grid, block, 0, stream>>>(a);
}

template <int FT>
static void launch_skinny_t(GemmArgs &a, int y_dt, hipStream_t stream) {
    dim3 grid((unsigned)((a.N + 31) / 32)), block(256);
    if (y_dt == F32) gemm_skinny<FT, F32><<<grid, block, 0, stream>>>(a);
    else if (y_dt == F16) gemm_skinny<FT, F16><<<grid, block, 0, stream>>>(a);
    else gemm_skinny<FT, BF16><<<grid, block, 0, stream>>>(a);
}

// Tile shape: the candidate whose tiles fill the 256 CUs best, weighted by
// how much MFMA work each tile does per byte staged through LDS.
static int pick_tile(int64_t M, int64_t N) {
    struct C { int bm, bn; double eff; int per_cu; };
    const C cands[3] = {{256, 256, 1.0, 1}, {256, 128, 0.85, 1}, {128, 128, 0.7, 2}};
    int best = 0;
    double best_score = -1;
    for (int i = 0; i < 3; ++i) {
        const int64_t tiles = ((M + cands[i].bm - 1) / cands[i].bm) * ((N + cands[i].bn - 1) / cands[i].bn);
        const int64_t slots = 256 * cands[i].per_cu;
        const int64_t rounds = (tiles + slots - 1) / slots;
        const double score = (double)tiles / (double)(rounds * slots) * cands[i].eff;
        if (score > best_score + 1e-9) { best_score = score; best = i; }
    }
    return best;
}

void launch_gemm(const int8_t *xq, const int8_t *wq, int64_t M, int64_t N, int64_t K,
                 const float *x_scale, int per_row, const float *w_scale, void *y, int y_dt,
                 int32_t *acc_out, const SideTerm *side, hipStream_t stream) {
    if (M == 0 || N == 0) return;
    GemmArgs a{};
    a.xq = xq; a.wq = wq; a.M = (int)M; a.N = (int)N; a.K = (int)K;
    a.xs = x_scale; a.xs_per_row = per_row; a.ws = w_scale; a.y = y; a.acc_out = acc_out;
    const bool pipe = K % 128 == 0;
    if (side) {
        a.x16 = side->x16; a.w16 = side->w16; a.idx = side->idx; a.count = side->count;
        if (pipe) launch_pipe_t<128, 128, 2, 2, 2, true>(a, y_dt, stream);
        else launch_tile_t<128, 128, 2, 2, true>(a, y_dt, stream);
        return;
    }
    if (M <= 16) { launch_skinny_t<1>(a, y_dt, stream); return; }
    if (M <= 32) { launch_skinny_t<2>(a, y_dt, stream); return; }
    // SQ_GEMM_TILE=0|1|2 forces a tile shape (for coverage of every shape).
    int tile = pick_tile(M, N);
    if (const char *e = getenv("SQ_GEMM_TILE")) {
        if (e[0] >= '0' && e[0] <= '2' && e[1] == 0) tile = e[0] - '0';
    }
    if (pipe) {
        switch (tile) {
            case 0: launch_pipe_t<256, 256, 2, 2, 2, false>(a, y_dt, stream); break;
            case 1: launch_pipe_t<256, 128, 2, 2, 3, false>(a, y_dt, stream); break;
            default: launch_pipe_t<128, 128, 2, 2, 2, false>(a, y_dt, stream); break;
        }
        return;
    }
    switch (tile) {
        case 0: launch_tile_t<256, 256, 2, 2, false>(a, y_dt, stream); break;
        case 1: launch_tile_t<256, 128, 2, 2, false>(a, y_dt, stream); break;
        default: launch_tile_t<128, 128, 2, 2, false>(a, y_dt, stream); break;
    }
}

}  // namespace sq
