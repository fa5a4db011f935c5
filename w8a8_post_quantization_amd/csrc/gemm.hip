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

template <int BM, int BN, int WM, int WN, int YDT, bool SIDE>
__global__ __launch_bounds__(256, 1) void gemm_tile(GemmArgs p) {
    constexpr int BK = 128;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int A_PER_T = BM * 8 / 256, B_PER_T = BN * 8 / 256;
    static_assert(WM * WN == 4, "4 waves");
    static_assert(FM >= 1 && FN >= 1 && A_PER_T >= 1 && B_PER_T >= 1, "tile");

    __shared__ __attribute__((aligned(16))) int8_t smem[2 * (BM + BN) * BK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int tile_m = blockIdx.x / p.tiles_n, tile_n = blockIdx.x % p.tiles_n;
    const int m0 = tile_m * BM, n0 = tile_n * BN;
    const int M = p.M, N = p.N, K = p.K;

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
    auto load_global = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i)
            ra[i] = k0 + a_kc[i] < K ? *reinterpret_cast<const uint4 *>(a_src[i] + k0)
                                     : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < B_PER_T; ++i)
            rb[i] = k0 + b_kc[i] < K ? *reinterpret_cast<const uint4 *>(b_src[i] + k0)
                                     : make_uint4(0, 0, 0, 0);
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

    // Epilogue.  32x32 accumulator layout: lane l, register v holds
    // row 8*(v/4) + 4*(l/32) + (v%4), column l%32 of the fragment.
    float dw[FN];
    int ncol[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        ncol[j] = n0 + wn * WTN + j * 32 + fr;
        dw[j] = ncol[j] < N ? p.ws[ncol[j]] : 0.0f;
    }

    if constexpr (SIDE) {
        // fp16 side product over the outlier columns, ascending, staged
        // through LDS 32 columns at a time (rows padded to 33 floats).
        float side[FM][FN][16];
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
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = m0 + wm * WTM + i * 32 + 8 * (v >> 2) + 4 * fh + (v & 3);
                if (m >= M) continue;
                const float dx = p.xs[p.xs_per_row ? m : 0];
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    if (ncol[j] >= N) continue;
                    const int64_t o = (int64_t)m * N + ncol[j];
                    const float c = dx * dw[j];
                    const float deq = (float)acc[i][j][v] * c;
                    store_y<YDT>(p.y, o, deq + side[i][j][v]);
                    if (p.acc_out) p.acc_out[o] = acc[i][j][v];
                }
            }
    } else {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = m0 + wm * WTM + i * 32 + 8 * (v >> 2) + 4 * fh + (v & 3);
                if (m >= M) continue;
                const float dx = p.xs[p.xs_per_row ? m : 0];
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    if (ncol[j] >= N) continue;
                    const int64_t o = (int64_t)m * N + ncol[j];
                    const float c = dx * dw[j];
                    store_y<YDT>(p.y, o, (float)acc[i][j][v] * c);
                    if (p.acc_out) p.acc_out[o] = acc[i][j][v];
                }
            }
    }
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
#pragma unroll
            for (int f = 0; f < 2; ++f)
                a[u][f] = ok ? *reinterpret_cast<const int4v *>(wrow[f] + k) : int4v{0, 0, 0, 0};
#pragma unroll
            for (int t = 0; t < FT; ++t)
                b[u][t] = ok ? *reinterpret_cast<const int4v *>(xrow[t] + k) : int4v{0, 0, 0, 0};
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
        int4v a[2], b[FT];
#pragma unroll
        for (int f = 0; f < 2; ++f)
            a[f] = ok ? *reinterpret_cast<const int4v *>(wrow[f] + k) : int4v{0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < FT; ++t)
            b[t] = ok ? *reinterpret_cast<const int4v *>(xrow[t] + k) : int4v{0, 0, 0, 0};
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
    for (int e = tid; e < NR * 16 * FT; e += 256) {
        const int nl = e % NR, ml = e / NR;
        const int m = ml, n = n0 + nl;
        if (m >= M || n >= N) continue;
        const int f = nl >> 4, i = nl & 15, t = ml >> 4, j = ml & 15;
        const int l = (i >> 2) * 16 + j, v = i & 3;
        const int a = red[0][f][t][v * 64 + l] + red[1][f][t][v * 64 + l] +
                      red[2][f][t][v * 64 + l] + red[3][f][t][v * 64 + l];
        const float c = p.xs[p.xs_per_row ? m : 0] * p.ws[n];
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
    if (side) {
        a.x16 = side->x16; a.w16 = side->w16; a.idx = side->idx; a.count = side->count;
        launch_tile_t<128, 128, 2, 2, true>(a, y_dt, stream);
        return;
    }
    if (M <= 16) { launch_skinny_t<1>(a, y_dt, stream); return; }
    if (M <= 32) { launch_skinny_t<2>(a, y_dt, stream); return; }
    // SQ_GEMM_TILE=0|1|2 forces a tile shape (for coverage of every shape).
    int tile = pick_tile(M, N);
    if (const char *e = getenv("SQ_GEMM_TILE")) {
        if (e[0] >= '0' && e[0] <= '2' && e[1] == 0) tile = e[0] - '0';
    }
    switch (tile) {
        case 0: launch_tile_t<256, 256, 2, 2, false>(a, y_dt, stream); break;
        case 1: launch_tile_t<256, 128, 2, 2, false>(a, y_dt, stream); break;
        default: launch_tile_t<128, 128, 2, 2, false>(a, y_dt, stream); break;
    }
}

}  // namespace sq
