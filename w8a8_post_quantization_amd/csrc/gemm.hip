// int8 x int8 -> int32 GEMM with the outer-product dequant epilogue
//   acc[m, n] = sum_k xq[m, k] * wq[n, k]                (exact int32)
//   y[m, n]   = fl(fl((float)acc) * fl(dx_m * dw_n))     (+ LLM.int8() side)
// (the SmoothQuant tutorial page: Y = diag(dX) X_int8 W_int8 diag(dW); the
// xdnf.cn LLM.int8() explainer §2.1: int32 accumulation and the c_x (x) c_w
// outer product; §2.2 for the fp16 side product over outlier columns).
//
// Three kernels, same bits:
//  * gemm_pp: M > 32 and K % 128 == 0 (every prefill shape).  Block tile
//    BM x BN of 4 or 8 waves, each wave a (BM/WM) x (BN/WN) sub-tile of
//    v_mfma_i32_32x32x32_i8 fragments.  K is streamed 128 bytes a stage into
//    a ring of LDS stages with direct-to-LDS loads (no register staging),
//    and the MFMAs of one stage interleave with the LDS reads of the next.
//  * gemm_tile: M > 32 with K % 128 != 0.  Same tiles, K staged through
//    registers into a double-buffered LDS tile, tail loads clamped.
//    In both, LDS rows are 128 bytes and chunk c of row r lives at slot
//    c ^ swz(r), which keeps the 16-byte LDS reads free of bank conflicts.
//  * gemm_dec: M <= 32 (decode), bound by the weight stream: a block owns
//    16..64 weight rows, its 4 waves split K and stream it through private
//    LDS rings with coalesced direct-to-LDS loads; v_mfma_i32_16x16x64_i8
//    with weight rows as the MFMA rows and tokens (padded to 16 / 32) as
//    columns; int32 partials are summed exactly through LDS.
//
// An integer dot product does not depend on the order of its terms, so the
// assignment of K bytes to MFMA lanes only has to be the same for both
// operands; the float epilogue is per element and order-free.
#include <type_traits>

#include "sq_device.h"
#include "sq_launch.h"

namespace sq {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int int8x __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int YDT>
__device__ __forceinline__ void store_y(void *y, int64_t i, float v) {
    reinterpret_cast<typename OutT<YDT>::T *>(y)[i] = narrow<YDT>(v);
}

__device__ __forceinline__ float h2f(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// One step of the LLM.int8() side sum, acc + x w with x and w fp16 values
// (widened exactly): their product has at most 22 significant bits and lies
// between 2^-48 and 2^32 in magnitude (or is 0), so it is exact in fp32 and
// the fused multiply-add's one rounding is the rounding of the addition:
// the same value as fl(acc + fl(x w)), in one instruction instead of two.
__device__ __forceinline__ float side_fma(float x, float w, float acc) {
    return __builtin_fmaf(x, w, acc);
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
    const float *xo;       // compact side operands, used when |O| <= side_cap
    const float *wo;
    int side_cap;
    int tiles_n;
    int tiles_m;
    int xcd_gm, xcd_gn;  // XCD grid of the tile mapping (tile_of), or 0: row-major
};

// The tile of block b.  The hardware deals a kernel's blocks to the 8 XCDs
// round-robin (block b to XCD b % 8), and each XCD has its own L2.  With an
// XCD grid gm x gn (gm | tiles_m, gn | tiles_n, gm gn = 8) XCD x takes the
// tiles of one sub-rectangle (tiles_m / gm) x (tiles_n / gn) of the tile
// grid, row-major, so it fetches only those activation rows and weight rows
// instead of most of both.  Any mapping gives the same results (a
// bijection of tiles); only the cache traffic changes.
__device__ __forceinline__ void tile_of(const GemmArgs &p, int b, int &tm, int &tn) {
    if (p.xcd_gm == 0) {
        tm = b / p.tiles_n;
        tn = b % p.tiles_n;
        return;
    }
    const int x = b & 7, j = b >> 3;
    const int rm = p.tiles_m / p.xcd_gm, rn = p.tiles_n / p.xcd_gn;
    tm = (x / p.xcd_gn) * rm + j / rn;
    tn = (x % p.xcd_gn) * rn + j % rn;
}

// LDS layout of a staged chunk of outlier columns, column-major so that one
// 16-byte read gives four consecutive rows of one column: activation values
// at xo[t * XS + r], weight values at wo[t * WS + r], wo = xo + 32 * XS.
template <int BM, int BN>
struct SideLds {
    static constexpr int XS = BM + 4, WS = BN + 4;
    static constexpr int BYTES = 32 * (XS + WS) * 4;
};

// Stage outlier columns t0 .. t0 + tn - 1 (tn <= 32) of the tile's
// activation rows and weight rows into LDS as floats (SideLds layout; only
// columns t < tn are written).  Thread tid serves activation row tid % BM
// for columns tid / BM, tid / BM + NT / BM, ... and weight row tid % BN for
// columns tid / BN, tid / BN + NT / BN, ...: the column is the same across a
// wave (BM, BN multiples of 64), dead columns cost no load, and the loads of
// a group of four columns are all issued before the first is written.  With
// `compact` the values come from the gathered side operands (p.xo, p.wo:
// one column's rows are contiguous, so a wave's load is coalesced); else
// each is a 2-byte gather from the fp16 rows at the column's index (a
// scalar load).
template <int BM, int BN, int NT>
__device__ __forceinline__ void stage_side(const GemmArgs &p, float *xo, float *wo, int m0,
                                           int n0, int t0, int tn, bool compact) {
    static_assert(BM % 64 == 0 && BN % 64 == 0 && NT % BM == 0 && NT % BN == 0,
                  "side staging");
    constexpr int PX = NT / BM, PW = NT / BN, G = 4;
    constexpr int XS = SideLds<BM, BN>::XS, WS = SideLds<BM, BN>::WS;
    const int tid = threadIdx.x;
    const int rx = tid % BM, rw = tid % BN;
    const int cx = __builtin_amdgcn_readfirstlane(tid / BM);
    const int cw = __builtin_amdgcn_readfirstlane(tid / BN);
    const int mr = m0 + rx < p.M ? m0 + rx : p.M - 1;
    const int nr = n0 + rw < p.N ? n0 + rw : p.N - 1;
    const uint16_t *xr = p.x16 + (int64_t)mr * p.K;
    const uint16_t *wr = p.w16 + (int64_t)nr * p.K;
    const float *xc = p.xo + (int64_t)t0 * p.M + mr;
    const float *wc = p.wo + (int64_t)t0 * p.N + nr;
    const int32_t *idx = p.idx + t0;
    for (int q = 0; q * G * PX < tn || q * G * PW < tn; ++q) {
        float vx[G], vw[G];
        if (compact) {
#pragma unroll
            for (int k = 0; k < G; ++k) {
                const int t = cx + PX * (q * G + k);
                vx[k] = t < tn ? xc[(int64_t)t * p.M] : 0.0f;
            }
#pragma unroll
            for (int k = 0; k < G; ++k) {
                const int t = cw + PW * (q * G + k);
                vw[k] = t < tn ? wc[(int64_t)t * p.N] : 0.0f;
            }
        } else {
#pragma unroll
            for (int k = 0; k < G; ++k) {
                const int t = cx + PX * (q * G + k);
                vx[k] = t < tn ? h2f(xr[idx[t]]) : 0.0f;
            }
#pragma unroll
            for (int k = 0; k < G; ++k) {
                const int t = cw + PW * (q * G + k);
                vw[k] = t < tn ? h2f(wr[idx[t]]) : 0.0f;
            }
        }
#pragma unroll
        for (int k = 0; k < G; ++k) {
            const int t = cx + PX * (q * G + k);
            if (t < tn) xo[t * XS + rx] = vx[k];
        }
#pragma unroll
        for (int k = 0; k < G; ++k) {
            const int t = cw + PW * (q * G + k);
            if (t < tn) wo[t * WS + rw] = vw[k];
        }
    }
}

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
// LDS 32 columns at a time (SideLds), and added to the dequantized value
// before narrowing.
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
    const int M = p.M, N = p.N;
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
        using L = SideLds<BM, BN>;
        static_assert(L::BYTES <= 2 * (BM + BN) * 128, "side chunk fits the ring");
        float *xo = reinterpret_cast<float *>(smem);
        float *wo = xo + 32 * L::XS;
        const int cnt = *p.count;
        const bool compact = cnt <= p.side_cap;
        for (int t0 = 0; t0 < cnt; t0 += 32) {
            const int tn = cnt - t0 < 32 ? cnt - t0 : 32;
            __syncthreads();
            stage_side<BM, BN, 256>(p, xo, wo, m0, n0, t0, tn, compact);
            __syncthreads();
            // column by column, so each output still sums in ascending order
            for (int t = 0; t < tn; ++t) {
                float wv[FN];
#pragma unroll
                for (int j = 0; j < FN; ++j) wv[j] = wo[t * L::WS + wn * WTN + j * 32 + fr];
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const float4 x4 = *reinterpret_cast<const float4 *>(
                            xo + t * L::XS + wm * WTM + i * 32 + 8 * g + 4 * fh);
                        const float xq[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
                        for (int j = 0; j < FN; ++j)
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                side[i][j][4 * g + q] = side_fma(xq[q], wv[j], side[i][j][4 * g + q]);
                            }
                    }
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
    int tile_m, tile_n;
    tile_of(p, blockIdx.x, tile_m, tile_n);
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

// The same with the nontemporal hint, for data read once (a weight stream
// that should not displace reused lines in the caches).
__device__ __forceinline__ void lds_dma16_nt(const void *g, uint32_t lds_base) {
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off nt"
        :
        : "v"(g), "s"(lds_base)
        : "memory", "m0");
}

// NL (1..4) direct-to-LDS loads under one M0 write: load j moves 16 bytes
// per lane from g[j] into LDS at lds_base + 1024 j + 16 lane.  The
// instruction offset (1024 j) is added to both the global and the LDS
// address, so g[j] is passed biased by -1024 j.  Rewriting M0 before every
// load makes each wave wait for its previous load to be accepted: measured
// on this GPU from an L2-resident source, 4 waves per CU moved 23 B/clk with
// one M0 write per load and 51.5 B/clk (the vector L1's rate for coalesced
// register loads) with one per four loads.  (The GEMMs here issue few
// enough loads per stage that their times did not change.)  NT adds the
// nontemporal hint.
template <int NL, bool NT>
__device__ __forceinline__ void lds_dma_group(const int8_t *const *g, uint32_t lds_base) {
    static_assert(NL >= 1 && NL <= 4, "one M0 covers 4 KB of instruction offsets");
    const int8_t *b0 = g[0];
    const int8_t *b1 = NL > 1 ? g[1] - 1024 : nullptr;
    const int8_t *b2 = NL > 2 ? g[2] - 2048 : nullptr;
    const int8_t *b3 = NL > 3 ? g[3] - 3072 : nullptr;
#define SQ_DMA_ASM(HINT)                                                                   \
    if constexpr (NL == 1) {                                                               \
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\t"                                    \
                     "global_load_lds_dwordx4 %0, off" HINT                                \
                     : : "v"(b0), "s"(lds_base) : "memory", "m0");                         \
    } else if constexpr (NL == 2) {                                                        \
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\t"                                    \
                     "global_load_lds_dwordx4 %0, off" HINT "\n\t"                        \
                     "global_load_lds_dwordx4 %1, off offset:1024" HINT                    \
                     : : "v"(b0), "v"(b1), "s"(lds_base) : "memory", "m0");                \
    } else if constexpr (NL == 3) {                                                        \
        asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\t"                                    \
                     "global_load_lds_dwordx4 %0, off" HINT "\n\t"                        \
                     "global_load_lds_dwordx4 %1, off offset:1024" HINT "\n\t"            \
                     "global_load_lds_dwordx4 %2, off offset:2048" HINT                    \
                     : : "v"(b0), "v"(b1), "v"(b2), "s"(lds_base) : "memory", "m0");       \
    } else {                                                                               \
        asm volatile("s_mov_b32 m0, %4\n\ts_nop 0\n\t"                                    \
                     "global_load_lds_dwordx4 %0, off" HINT "\n\t"                        \
                     "global_load_lds_dwordx4 %1, off offset:1024" HINT "\n\t"            \
                     "global_load_lds_dwordx4 %2, off offset:2048" HINT "\n\t"            \
                     "global_load_lds_dwordx4 %3, off offset:3072" HINT                    \
                     : : "v"(b0), "v"(b1), "v"(b2), "v"(b3), "s"(lds_base)                  \
                     : "memory", "m0");                                                    \
    }
    if constexpr (NT) {
        SQ_DMA_ASM(" nt")
    } else {
        SQ_DMA_ASM("")
    }
#undef SQ_DMA_ASM
}

// Loads j = 0 .. N-1 of a stage into consecutive 1 KB LDS blocks, M0 set
// once per four.
template <int N, bool NT>
__device__ __forceinline__ void lds_dma_run(const int8_t *const *g, uint32_t lds_base) {
#pragma unroll
    for (int j0 = 0; j0 < N; j0 += 4) {
        if (N - j0 >= 4) lds_dma_group<4, NT>(g + j0, lds_base + (uint32_t)(j0 * 1024));
        else if (N - j0 == 3) lds_dma_group<3, NT>(g + j0, lds_base + (uint32_t)(j0 * 1024));
        else if (N - j0 == 2) lds_dma_group<2, NT>(g + j0, lds_base + (uint32_t)(j0 * 1024));
        else lds_dma_group<1, NT>(g + j0, lds_base + (uint32_t)(j0 * 1024));
    }
}

// s_waitcnt vmcnt(N) leaving lgkmcnt / expcnt alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most `later` stages of P loads each are in flight
// (later <= L, or negative for none; vmcnt takes an immediate, hence the
// unrolled choice).
template <int L, int P>
__device__ __forceinline__ void wait_stages(int later) {
    if constexpr (L == 0) {
        wait_vmcnt<0>();
    } else {
        if (later >= L) wait_vmcnt<L * P>();
        else wait_stages<L - 1, P>(later);
    }
}

// Workgroup barrier for the LDS ring only.  __syncthreads() carries a
// release fence that waits for every outstanding global load (vmcnt(0)),
// which would drain the in-flight stages; here each wave has already waited
// for its own stage loads with vmcnt(N), and only LDS traffic must be
// complete before the barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}


// Epilogue of the pipelined kernel.  The MFMAs there take weight rows as
// the A operand and tokens as B, so lane l, register v of fragment (i, j)
// holds output column n = 8*(v/4) + 4*(l/32) + (v%4) of n-fragment i and
// row m = l%32 of m-fragment j: four consecutive columns of one row per
// group of four registers.
// Side sums over staged columns t_begin .. tn - 1 (column t of the activation
// rows at xo[t * XS + r], of the weight rows at wo[t * WS + r]), column by
// column, so that each output still sums in ascending column order; each
// thread's outputs are its accumulator fragments' (32x32 layout).
template <int BM, int BN, int WM, int WN, int XS, int WS>
__device__ __forceinline__ void side_columns(const float *xo, const float *wo, int t_begin,
                                             int tn,
                                             float (&side)[BN / WN / 32][BM / WM / 32][16]) {
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int fr = lane & 31, fh = lane >> 5;
    for (int t = t_begin; t < tn; ++t) {
        float xv[FM];
#pragma unroll
        for (int j = 0; j < FM; ++j) xv[j] = xo[t * XS + wm * WTM + j * 32 + fr];
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 w4 = *reinterpret_cast<const float4 *>(wo + t * WS + wn * WTN +
                                                                    i * 32 + 8 * g + 4 * fh);
                const float wq[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
                for (int j = 0; j < FM; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        side[i][j][4 * g + q] = side_fma(xv[j], wq[q], side[i][j][4 * g + q]);
            }
    }
}

// The first side columns (at most kSideEarly, and at most one per main-loop
// stage) are summed inside the main loop, one column per iteration, where
// the vector ALUs are otherwise idle.  Their compact operands go straight
// to an LDS area beside the ring with direct-to-LDS dword loads issued at
// kernel start, before the ring's: loads complete in issue order, so the
// ring's first wait covers them, and they hold no registers.  The area is
// column-major like SideLds (activations ex[t XS + r], XS = BM + 4, then
// weights ew[t WS + r], WS = BN + 4); a wave fills 64 consecutive rows of one
// column per load.  The compact arrays hold side_cap >= kSideEarly columns
// (else nothing is loaded here), so the loads are in bounds whatever |O| turns out to be; columns past |O| are
// never read.  Returns false (nothing issued) without compact operands.
constexpr int kSideEarly = 8;
template <int BM, int BN, int NT>
__device__ __forceinline__ bool side_early_load(const GemmArgs &p, int m0, int n0,
                                                uint32_t area) {
    constexpr int PX = NT / BM, PW = NT / BN, XS = BM + 4, WS = BN + 4;
    static_assert(BM % 64 == 0 && BN % 64 == 0 && kSideEarly % PX == 0 &&
                  kSideEarly % PW == 0, "early side columns");
    if (!p.xo || p.side_cap < kSideEarly) return false;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // activations: this wave's rows rb .. rb + 63 of column cx + PX k
    const int rbx = (wave * 64) % BM, cx = (wave * 64) / BM;
    const int mr = m0 + rbx + lane < p.M ? m0 + rbx + lane : p.M - 1;
#pragma unroll
    for (int k = 0; k < kSideEarly / PX; ++k) {
        const int t = cx + PX * k;
        const float *src = p.xo + (int64_t)t * p.M + mr;
        const uint32_t dst = area + (uint32_t)((t * XS + rbx) * 4);
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                     : : "v"(src), "s"(dst) : "memory", "m0");
    }
    const int rbw = (wave * 64) % BN, cw = (wave * 64) / BN;
    const int nr = n0 + rbw + lane < p.N ? n0 + rbw + lane : p.N - 1;
#pragma unroll
    for (int k = 0; k < kSideEarly / PW; ++k) {
        const int t = cw + PW * k;
        const float *src = p.wo + (int64_t)t * p.N + nr;
        const uint32_t dst = area + (uint32_t)((kSideEarly * XS + t * WS + rbw) * 4);
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                     : : "v"(src), "s"(dst) : "memory", "m0");
    }
    return true;
}

template <int BM, int BN, int WM, int WN, int YDT, bool SIDE, typename AccV>
__device__ __forceinline__ void epilogue_nt(const GemmArgs &p,
                                            AccV (&acc)[BN / WN / 32][BM / WM / 32],
                                            int8_t *smem, const float *sx, const float *sw,
                                            int m0, int n0, int cnt_in,
                                            float (&side)[SIDE ? BN / WN / 32 : 1]
                                                         [SIDE ? BM / WM / 32 : 1][16],
                                            int t_from) {
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int NT = 64 * WM * WN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int fr = lane & 31, fh = lane >> 5;
    const int M = p.M, N = p.N;
    if constexpr (SIDE) {
        // side holds the sums over the columns before t_from (added while
        // the main loop's first stages loaded); the rest follow in order.
        using L = SideLds<BM, BN>;
        static_assert(L::BYTES <= 2 * (BM + BN) * 128, "side chunk fits the ring");
        float *xo = reinterpret_cast<float *>(smem);
        float *wo = xo + 32 * L::XS;
        const int cnt = cnt_in;
        const bool compact = cnt <= p.side_cap;
        for (int t0 = t_from; t0 < cnt; t0 += 32) {
            const int tn = cnt - t0 < 32 ? cnt - t0 : 32;
            __syncthreads();
            stage_side<BM, BN, NT>(p, xo, wo, m0, n0, t0, tn, compact);
            __syncthreads();
            side_columns<BM, BN, WM, WN, L::XS, L::WS>(xo, wo, 0, tn, side);
        }
    }
    // Exact int32 sums, when asked for (direct stores, not on the fast path).
    if constexpr (std::is_same_v<AccV, int16v>) if (p.acc_out) {
        const bool vec_a = (N & 3) == 0 && ((uintptr_t)p.acc_out & 15) == 0;
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            const int m = m0 + wm * WTM + j * 32 + fr;
            if (m >= M) continue;
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int n = n0 + wn * WTN + i * 32 + 8 * g + 4 * fh;
                    const int64_t o = (int64_t)m * N + n;
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

    if constexpr (SIDE) {
        // Final values y = fl(fl(acc) * c) + side, folded into the side
        // array now so the accumulators are dead before the slab stores.
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            const float dx = sx[wm * WTM + j * 32 + fr];
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const float4 dw4 =
                        *reinterpret_cast<const float4 *>(sw + wn * WTN + i * 32 + 8 * g + 4 * fh);
                    const float dwq[4] = {dw4.x, dw4.y, dw4.z, dw4.w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float c = dx * dwq[q];
                        const float deq = (float)acc[i][j][4 * g + q] * c;
                        side[i][j][4 * g + q] = deq + side[i][j][4 * g + q];
                    }
                }
        }
        __syncthreads();  // the ring held the side operands
    }

    // Outputs go through a wave-private slab of the (now free) ring: 32 rows
    // x WTN columns of the output type per m-fragment, written from the
    // accumulator layout and read back 16 bytes per lane along rows, so a
    // quarter-wave stores 128-256 contiguous bytes instead of touching 16
    // rows.  16-byte chunk c of slab row r sits at position c ^ f(r).
    using T = typename OutT<YDT>::T;
    constexpr int RB = WTN * (int)sizeof(T);       // slab row bytes
    constexpr int CPR = RB / 16;                   // 16-byte chunks per row
    constexpr int RPW = RB >= 256 ? 1 : 256 / RB;  // rows per 256-byte bank window
    constexpr int EPC = 16 / (int)sizeof(T);       // outputs per chunk
    static_assert(RB % 16 == 0 && WM * WN * 32 * RB <= (BM + BN) * 128 * 2, "slab");
    int8_t *slab = smem + wave * (32 * RB);
    const bool vec_y = ((N * (int)sizeof(T)) & 15) == 0 && ((uintptr_t)p.y & 15) == 0;
    // The weight steps of this lane's columns, read once for every
    // m-fragment (the slab's LDS traffic is what the epilogue waits on).
    float4 dwv[SIDE ? 1 : FN][4];
    if constexpr (!SIDE) {
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                dwv[i][g] = *reinterpret_cast<const float4 *>(sw + wn * WTN + i * 32 + 8 * g + 4 * fh);
    }
#pragma unroll
    for (int j = 0; j < FM; ++j) {
        const int ml = wm * WTM + j * 32 + fr;
        const float dx = sx[ml];
        const int fw = (fr / RPW) & (CPR - 1);
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int cl = i * 32 + 8 * g + 4 * fh;  // first of 4 columns in the wave tile
                const float4 dw4 = dwv[SIDE ? 0 : i][g];
                const float dwq[4] = {dw4.x, dw4.y, dw4.z, dw4.w};
                T h[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if constexpr (SIDE) {
                        h[q] = narrow<YDT>(side[i][j][4 * g + q]);
                    } else {
                        const float c = dx * dwq[q];
                        h[q] = narrow<YDT>((float)acc[i][j][4 * g + q] * c);
                    }
                }
                const int cb = cl * (int)sizeof(T);  // byte offset in the slab row
                int8_t *dst = slab + fr * RB + (((cb >> 4) ^ fw) << 4) + (cb & 15);
                if constexpr (sizeof(T) == 4) *reinterpret_cast<uint4 *>(dst) = __builtin_bit_cast(uint4, h);
                else *reinterpret_cast<uint2 *>(dst) = __builtin_bit_cast(uint2, h);
            }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // slab written (one wave)
        static_assert((32 * CPR) % 64 == 0, "slab chunks per lane");
#pragma unroll
        for (int k = 0; k < 32 * CPR / 64; ++k) {
            const int c = lane + 64 * k;
            const int r = c / CPR, ch = c % CPR;
            const uint4 v = *reinterpret_cast<const uint4 *>(
                slab + r * RB + ((ch ^ ((r / RPW) & (CPR - 1))) << 4));
            const int m = m0 + wm * WTM + j * 32 + r;
            const int n = n0 + wn * WTN + ch * EPC;
            if (m >= M || n >= N) continue;
            T *yp = reinterpret_cast<T *>(p.y) + (int64_t)m * N + n;
            if (vec_y && n + EPC <= N) {
                *reinterpret_cast<uint4 *>(yp) = v;
            } else {
                T e[EPC];
                __builtin_memcpy(e, &v, 16);
#pragma unroll
                for (int q = 0; q < EPC; ++q)
                    if (n + q < N) yp[q] = e[q];
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // slab read before reuse
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

// K % 128 == 0.  K is staged 128 bytes at a time through two LDS rings
// filled by direct-to-LDS loads (global_load_lds_dwordx4): an activation
// ring of STA slots and a weight ring of STB slots.  Each wave instruction
// moves 8 rows x 128 bytes, so every request to L2 is a whole 128-byte line
// (64-byte stages fetched each line as two requests, and the number of
// requests the vector L1 keeps in flight capped the feed rate).  Lane l
// writes LDS bytes [16 l, 16 l + 16) of its 1 KiB block; the swizzle (see
// swz) is applied by choosing which global chunk each lane fetches.
//
// Both rings have the same depth (STA == STB).  A deeper weight ring buys
// no latency when the same waves fetch both operands: loads complete in
// issue order, so waiting for activation stage kt + 1 also waits for every
// weight stage issued before it (a variant with the ring loads split
// between waves by operand, and 2 + 4 or 2 + 5 stages, measured no faster).
// Per iteration the kernel issues the activation stage kt + STA, then the
// weight stage kt + STB, which fixes the vmcnt values below.
//
// Each stage is consumed as four 32-byte quarters with ping-pong fragment
// registers: a quarter's LDS reads overlap the previous quarter's MFMAs, and
// after the stage barrier the next stage's first reads overlap the last
// quarter's MFMAs.  Weight rows are the MFMA A operand (see epilogue_nt).
// The four-wave 128x128 side-term variant asks for two blocks per CU: its
// tiles are small, and one wave per SIMD halves how many tiles a CU has in
// flight.  The eight-wave 256x128 side-term tile runs one block per CU.
template <int BM, int BN, int WM, int WN, int STA, int STB, int YDT, bool SIDE, bool F8 = false>
__global__ __launch_bounds__(64 * WM * WN, (SIDE && WM * WN == 4) ? 2 : 1) __attribute__((amdgpu_waves_per_eu(SIDE ? 2 : 1, 4))) void
gemm_pp(GemmArgs p) {
    constexpr int BK = 128;
    constexpr int NW = WM * WN;  // waves
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int LA = BM / (8 * NW), LB = BN / (8 * NW);  // load instructions per wave per stage
    constexpr int L = LA + LB;
    constexpr int SA = BM * BK, SB = BN * BK;  // bytes of one stage of each operand
    static_assert((NW == 4 || NW == 8) && FM >= 1 && FN >= 1 && LA >= 1 && LB >= 1, "tile");
    static_assert(STA >= 2 && STB == STA, "ring depths");
    static_assert(STA * L < 64, "vmcnt range");

    __shared__ __attribute__((aligned(1024))) int8_t smem[STA * SA + STB * SB];
    __shared__ __attribute__((aligned(16))) float sx[BM], sw[BN];
    // the early side columns' operands (side_early), beside the ring
    __shared__ __attribute__((aligned(16))) float sside[SIDE ? kSideEarly * (BM + BN + 8) : 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    int tile_m, tile_n;
    tile_of(p, blockIdx.x, tile_m, tile_n);
    const int m0 = tile_m * BM, n0 = tile_n * BN;
    const int M = p.M, N = p.N, K = p.K;
    TileScales<BM, BN> scl;
    scl.load(p, m0, n0);
    // LLM.int8(): |O| read now, so nothing waits for it later; the side
    // sums (side_early_load, side_columns) start from zero.
    int scnt = 0;
    float side[SIDE ? FN : 1][SIDE ? FM : 1][16];
    int t_from = 0;  // side columns summed before the epilogue
    if constexpr (SIDE) {
        scnt = *p.count;
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) side[i][j][v] = 0.0f;
    }

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
    // This wave's blocks: activation blocks wave*LA + j of an A slot, weight
    // blocks wave*LB + j of a B slot (the blocks the rows above were chosen
    // for).  LDS byte addresses, wave-uniform for M0.
    const uint32_t waveu = (uint32_t)__builtin_amdgcn_readfirstlane(wave);
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void_t *)smem;
    const uint32_t lds_a = lds0 + waveu * (LA * 1024u);
    const uint32_t lds_b = lds0 + (uint32_t)(STA * SA) + waveu * (LB * 1024u);
    const int nk = K / BK;
    auto issue_a = [&](int s) {  // activation stage s < nk
        const int8_t *g[LA];
#pragma unroll
        for (int j = 0; j < LA; ++j) g[j] = a_src[j] + s * BK;
        lds_dma_run<LA, false>(g, lds_a + (uint32_t)((s % STA) * SA));
    };
    auto issue_b = [&](int s) {  // weight stage s < nk
        const int8_t *g[LB];
#pragma unroll
        for (int j = 0; j < LB; ++j) g[j] = b_src[j] + s * BK;
        lds_dma_run<LB, false>(g, lds_b + (uint32_t)((s % STB) * SB));
    };

    const int fr = lane & 31, fh = lane >> 5;
    const int fsw = swz(fr);  // fragment bases are multiples of 32 rows
    int off[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) off[q] = ((2 * q + fh) ^ fsw) << 4;
    auto read_frags = [&](int s, int q, int4v (&xf)[FM], int4v (&wf)[FN]) {
        const int8_t *ab = smem + (s % STA) * SA + off[q];
        const int8_t *bb = smem + STA * SA + (s % STB) * SB + off[q];
#pragma unroll
        for (int f = 0; f < FM; ++f)
            xf[f] = *reinterpret_cast<const int4v *>(ab + (wm * WTM + f * 32 + fr) * BK);
#pragma unroll
        for (int f = 0; f < FN; ++f)
            wf[f] = *reinterpret_cast<const int4v *>(bb + (wn * WTN + f * 32 + fr) * BK);
    };

    using AccV = std::conditional_t<F8, f32x16, int16v>;
    AccV acc[FN][FM];
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

    if constexpr (F8) {
        // e4m3 operands: one v_mfma_f32_32x32x64_f8f6f4 takes two K quarters
        // (each lane's 16-byte chunk of quarter q and of quarter q + 1 as one
        // 32-byte operand).  A and B are built the same way, so the MFMA
        // sees one consistent permutation of the 64 K values: the sum is the
        // same set of products.  Quarters 2 and 3 are read while quarters 0
        // and 1 multiply, and the next stage's 0 and 1 (after the barrier,
        // with the stage's direct loads) while 2 and 3 multiply.
        auto mma8 = [&](const int4v (&xa)[FM], const int4v (&wa)[FN], const int4v (&xb)[FM],
                        const int4v (&wb)[FN]) {
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j) {
                    const int8x a = __builtin_shufflevector(wa[i], wb[i], 0, 1, 2, 3, 4, 5, 6, 7);
                    const int8x b = __builtin_shufflevector(xa[j], xb[j], 0, 1, 2, 3, 4, 5, 6, 7);
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        a, b, acc[i][j], 0, 0, 0, 0, 0, 0);
                }
        };
#pragma unroll
        for (int s = 0; s < STA; ++s) {
            if (s < nk) {
                issue_a(s);
                issue_b(s);
            }
        }
        wait_stages<STA - 1, L>((nk < STA ? nk : STA) - 1);  // stage 0 landed
        lds_barrier();
        int4v x0[FM], w0[FN], x1[FM], w1[FN], x2[FM], w2[FN], x3[FM], w3[FN];
        read_frags(0, 0, x0, w0);
        read_frags(0, 1, x1, w1);
        int kt = 0;
        for (; kt + STA < nk; ++kt) {
            read_frags(kt, 2, x2, w2);
            read_frags(kt, 3, x3, w3);
            mma8(x0, w0, x1, w1);
            wait_vmcnt<(STA - 2) * L>();  // stage kt + 1 of both operands landed
            lds_barrier();  // every wave has read stage kt: its slots are free
            read_frags(kt + 1, 0, x0, w0);
            read_frags(kt + 1, 1, x1, w1);
            issue_a(kt + STA);
            issue_b(kt + STB);
            mma8(x2, w2, x3, w3);
        }
        for (; kt < nk; ++kt) {  // nothing left to issue
            read_frags(kt, 2, x2, w2);
            read_frags(kt, 3, x3, w3);
            mma8(x0, w0, x1, w1);
            wait_stages<STA - 2, L>(nk - kt - 2);  // stage kt + 1 landed (if any)
            lds_barrier();
            read_frags(kt + 1, 0, x0, w0);  // past the last stage: never multiplied
            read_frags(kt + 1, 1, x1, w1);
            mma8(x2, w2, x3, w3);
        }
        wait_vmcnt<0>();
        scl.publish(sx, sw);
        __syncthreads();
        epilogue_nt<BM, BN, WM, WN, YDT, SIDE>(p, acc, smem, sx, sw, m0, n0, scnt, side,
                                              t_from);
        return;
    } else {
    // Main loop.  Its two halves are branch-free so the scheduler can
    // interleave: a wave issues in order, so a ds_read (or direct load)
    // queued behind an MFMA that waits for the matrix core cannot issue; the
    // sched_group_barrier sequences place one memory instruction after each
    // MFMA.  The last STA iterations (step_tail) issue no loads - there is no
    // stage left - and wait for as many stages as are still in flight.
    constexpr int RQ = FM + FN;  // ds_read_b128 per quarter
    constexpr int MQ = FM * FN;  // MFMAs per quarter
    static_assert(RQ <= MQ, "one read per MFMA slot");
    bool searly = false;  // the early side operands were loaded
    if constexpr (SIDE)
        searly = side_early_load<BM, BN, 64 * NW>(p, m0, n0,
                                                  (uint32_t)(uintptr_t)(lds_void_t *)sside);
#pragma unroll
    for (int s = 0; s < STA; ++s) {
        if (s < nk) {
            issue_a(s);
            issue_b(s);
        }
    }
    // side columns summed in the main loop (kSideEarly at most, one per
    // stage; compact operands only)
    int te = 0;
    if constexpr (SIDE) {
        if (searly && scnt > 0 && scnt <= p.side_cap) {
            te = scnt < kSideEarly ? scnt : kSideEarly;
            te = te < nk - STA ? te : nk - STA;  // stages that still issue loads
            te = te > 0 ? te : 0;
        }
        t_from = te;
    }
    wait_stages<STA - 1, L>((nk < STA ? nk : STA) - 1);  // stage 0 landed
    lds_barrier();
    int4v xa[FM], wa[FN], xb[FM], wb[FN];
    read_frags(0, 0, xa, wa);
    // A stage: quarters 1-3 read while 0-2 multiply, then the barrier, then
    // the next stage's quarter 0 read (and, in step, the next loads issued)
    // while quarter 3 multiplies.
    auto step_tail = [&](int kt) {  // kt + STA >= nk: nothing left to issue
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
        wait_stages<STA - 2, L>(nk - kt - 2);  // stage kt + 1 landed (if any)
        lds_barrier();
        read_frags(kt + 1, 0, xa, wa);  // past the last stage: never multiplied
        mma(xb, wb);
    };
    auto step = [&](int kt) {
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
        wait_vmcnt<(STA - 2) * L>();  // stage kt + 1 of both operands landed
        lds_barrier();  // every wave has read stage kt: its slots are free
        read_frags(kt + 1, 0, xa, wa);
        issue_a(kt + STA);
        issue_b(kt + STB);
        mma(xb, wb);
        sched_tail<MQ, RQ, L, 0>();  // MFMA, DS read, direct loads, ...
    };
    int kt = 0;
    if constexpr (SIDE) {
        // the first te stages each add one early side column (a loop of its
        // own, so the main loop below is the plain one)
        for (; kt < te; ++kt) {
            step(kt);
            side_columns<BM, BN, WM, WN, BM + 4, BN + 4>(sside, sside + kSideEarly * (BM + 4), kt,
                                                         kt + 1, side);
        }
    }
    for (; kt + STA < nk; ++kt) step(kt);
    for (; kt < nk; ++kt) step_tail(kt);
    wait_vmcnt<0>();
    scl.publish(sx, sw);
    __syncthreads();  // steps visible; the side term may reuse the ring
    epilogue_nt<BM, BN, WM, WN, YDT, SIDE>(p, acc, smem, sx, sw, m0, n0, scnt, side,
                                              t_from);
    }
}

// gemm_pp's tiles with eight waves in four pairs whose two waves split
// every stage's K (int8, no side term).  A pair covers one (BM/2) x (BN/2)
// region of the tile: wave w multiplies K quarters 2g and 2g + 1
// (g = (w >> 1) & 1) of activation rows (BM/2) (w >> 2) .. and weight rows
// (BN/2) (w & 1) .. of each stage.  After the last stage the partners swap
// halves through the free ring: wave w keeps the int32 sums of activation
// rows (BM/4) (w >> 1) .. + BM/4 - 1 (the half g of its region) and adds its
// partner's (w ^ 2) sums of the same outputs - an exact integer addition, so
// the results are gemm_pp's bits - which is the (BM/4) x (BN/2) layout of a
// 4 x 2 wave grid, handed to the same epilogue.  At 128 x 128 this runs
// eight waves (two per SIMD) on a tile that gemm_pp covers with four.
template <int BM, int BN, int STA, int YDT>
__global__ __launch_bounds__(512, 1) __attribute__((amdgpu_waves_per_eu(1, 4))) void
gemm_pk(GemmArgs p) {
    constexpr int BK = 128, NW = 8;
    constexpr int FM = BM / 64, FN = BN / 64;         // fragments of a wave's region
    constexpr int FH = FM / 2;                        // m-fragments of a half
    constexpr int LA = BM / (8 * NW), LB = BN / (8 * NW), L = LA + LB;
    constexpr int SA = BM * BK, SB = BN * BK;
    static_assert(FM >= 2 && FM % 2 == 0 && FN >= 1 && LA >= 1 && LB >= 1, "tile");
    static_assert(STA >= 2 && STA * L < 64, "ring");
    static_assert(NW * FN * FH * 4096 <= STA * (SA + SB), "exchange fits the ring");

    __shared__ __attribute__((aligned(1024))) int8_t smem[STA * (SA + SB)];
    __shared__ __attribute__((aligned(16))) float sx[BM], sw[BN];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = (wave >> 1) & 1;                    // K half of each stage
    const int mb = (wave >> 2) * (BM / 2), nb = (wave & 1) * (BN / 2);
    int tile_m, tile_n;
    tile_of(p, blockIdx.x, tile_m, tile_n);
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
    const uint32_t waveu = (uint32_t)__builtin_amdgcn_readfirstlane(wave);
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void_t *)smem;
    const uint32_t lds_a = lds0 + waveu * (LA * 1024u);
    const uint32_t lds_b = lds0 + (uint32_t)(STA * SA) + waveu * (LB * 1024u);
    const int nk = K / BK;
    auto issue = [&](int s) {  // both operands of stage s < nk
        const int8_t *ga[LA];
        const int8_t *gb[LB];
#pragma unroll
        for (int j = 0; j < LA; ++j) ga[j] = a_src[j] + s * BK;
#pragma unroll
        for (int j = 0; j < LB; ++j) gb[j] = b_src[j] + s * BK;
        lds_dma_run<LA, false>(ga, lds_a + (uint32_t)((s % STA) * SA));
        lds_dma_run<LB, false>(gb, lds_b + (uint32_t)((s % STA) * SB));
    };

    const int fr = lane & 31, fh = lane >> 5;
    const int fsw = swz(fr);
    const int off0 = ((4 * g + fh) ^ fsw) << 4;       // quarter 2g
    const int off1 = ((4 * g + 2 + fh) ^ fsw) << 4;   // quarter 2g + 1
    auto read_frags = [&](int s, int off, int4v (&xf)[FM], int4v (&wf)[FN]) {
        const int8_t *ab = smem + (s % STA) * SA + off;
        const int8_t *bb = smem + STA * SA + (s % STA) * SB + off;
#pragma unroll
        for (int f = 0; f < FM; ++f)
            xf[f] = *reinterpret_cast<const int4v *>(ab + (mb + f * 32 + fr) * BK);
#pragma unroll
        for (int f = 0; f < FN; ++f)
            wf[f] = *reinterpret_cast<const int4v *>(bb + (nb + f * 32 + fr) * BK);
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

    // Main loop: the quarter-2g fragments multiply while the quarter-2g+1
    // ones load; after the stage barrier the next stage's quarter-2g loads
    // and the stage's direct loads interleave with the quarter-2g+1 MFMAs.
    // The last STA iterations issue no loads and wait for as many stages as
    // are still in flight.
    constexpr int RQ = FM + FN, MQ = FM * FN;
    static_assert(RQ <= MQ, "one read per MFMA slot");
#pragma unroll
    for (int s = 0; s < STA; ++s)
        if (s < nk) issue(s);
    wait_stages<STA - 1, L>((nk < STA ? nk : STA) - 1);  // stage 0 landed
    lds_barrier();
    int4v xa[FM], wa[FN], xb[FM], wb[FN];
    read_frags(0, off0, xa, wa);
    auto half = [&](int kt) {  // the quarter-2g MFMAs, quarter 2g + 1 read
        read_frags(kt, off1, xb, wb);
        mma(xa, wa);
#pragma unroll
        for (int r = 0; r < RQ; ++r) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        }
        if constexpr (MQ > RQ) __builtin_amdgcn_sched_group_barrier(0x008, MQ - RQ, 0);
    };
    int kt = 0;
    for (; kt + STA < nk; ++kt) {
        half(kt);
        wait_vmcnt<(STA - 2) * L>();  // stage kt + 1 of both operands landed
        lds_barrier();                // every wave has read stage kt: its slots are free
        read_frags(kt + 1, off0, xa, wa);
        issue(kt + STA);
        mma(xb, wb);
        sched_tail<MQ, RQ, L, 0>();
    }
    for (; kt < nk; ++kt) {
        half(kt);
        wait_stages<STA - 2, L>(nk - kt - 2);  // stage kt + 1 landed (if any)
        lds_barrier();
        read_frags(kt + 1, off0, xa, wa);  // past the last stage: never multiplied
        mma(xb, wb);
    }
    wait_vmcnt<0>();
    scl.publish(sx, sw);
    __syncthreads();  // ring free: every wave has read the last stage

    // Swap halves with the partner through the ring: fragment (i, jj) of the
    // half sent (m-fragment FH (1 - g) + jj) is written as 4 lane-major
    // 16-byte rows at wave w's slot; the partner reads the same lane's
    // values, so both sides keep the accumulator layout.  g is
    // wave-uniform: one branch, static register indices.
    constexpr int SLOT = FN * FH * 4 * 64;  // int4v per wave
    int4v *const xs = reinterpret_cast<int4v *>(smem);
    int4v *const mine = xs + wave * SLOT;
    const int4v *const theirs = xs + (wave ^ 2) * SLOT;
    int16v fin[FN][FH];
    auto swap_halves = [&](auto g_c) {
        constexpr int G = decltype(g_c)::value;
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int jj = 0; jj < FH; ++jj)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int16v &a = acc[i][FH * (1 - G) + jj];
                    mine[((i * FH + jj) * 4 + c) * 64 + lane] =
                        int4v{a[4 * c], a[4 * c + 1], a[4 * c + 2], a[4 * c + 3]};
                }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int jj = 0; jj < FH; ++jj)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int4v t = theirs[((i * FH + jj) * 4 + c) * 64 + lane];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        fin[i][jj][4 * c + e] = acc[i][FH * G + jj][4 * c + e] + t[e];
                }
    };
    if (__builtin_amdgcn_readfirstlane(g)) swap_halves(std::integral_constant<int, 1>{});
    else swap_halves(std::integral_constant<int, 0>{});
    __syncthreads();  // exchange read: the epilogue reuses the ring
    float side_unused[1][1][16];
    epilogue_nt<BM, BN, 4, 2, YDT, false>(p, fin, smem, sx, sw, m0, n0, 0, side_unused, 0);
}

// ---------------------------------------------------------------- decode

// Decode GEMM (M <= 32), bound by the weight stream.  A block owns 16*NF
// weight rows; its 4 waves split K and each streams its K range through a
// private ring of S LDS stages with direct-to-LDS loads.  A stage holds
// U 64-byte K steps of the 16*NF weight rows and the 16*FT token rows.
//
// Why LDS: in MFMA operand layout the 16 lanes of a quarter-wave hold 16
// different rows, so a 16-byte-per-lane register load touches 16 cache
// lines per quarter-wave (64 tag lookups per 1 KB instruction) and the
// texture data path, not HBM, sets the rate.  Here each 1 KB load has a
// quarter-wave read one contiguous row span (16 / U rows of 64*U bytes per
// load), and the fragments are read back from LDS in operand layout.  Chunk
// c of row r sits at position c ^ f(r) of its row so that the 16 rows a
// quarter-wave reads fall in distinct banks.
//
// K order inside the MFMA is free for integer sums: both operands use
// "lane group g of step s holds bytes 64 s + 16 g .. + 15 of the stage".
// The e4m3 form (F8, U = 2) feeds one v_mfma_f32_16x16x128_f8f6f4 per stage
// with each lane's chunks of both steps as one 32-byte operand, built the
// same way for weights and tokens, and sums the waves' fp32 partials in a
// fixed order.
template <int U>
__device__ __forceinline__ int dec_swz(int r) {
    return (r / (4 / U)) & (4 * U - 1);
}

template <int NF, int FT, int U, int S, int YDT, bool NT, bool F8 = false>
__global__ __launch_bounds__(256) void gemm_dec(GemmArgs p) {
    static_assert(U == 1 || U == 2 || U == 4, "stage width");
    static_assert(!F8 || U == 2, "e4m3: two 64-byte steps per MFMA");
    static_assert((16 * NF * 16 * FT) % 256 == 0, "whole outputs per thread");
    static_assert(S >= 2 && S <= 6, "ring depth");
    constexpr int NR = 16 * NF;
    constexpr int NFR = NF + FT;                 // fragments per stage
    constexpr int P = NFR * U;                   // 1 KB loads per stage
    constexpr int SLOT = P * 1024;               // one stage of one wave
    constexpr int RING = S * SLOT;
    constexpr int RED = 4 * NF * FT * 1024;      // int32 partial sums of 4 waves
    constexpr int LDSB = 4 * RING > RED ? 4 * RING : RED;
    constexpr int RPI = 16 / U;                  // rows per 1 KB load
    constexpr int CPR = 4 * U;                   // 16-byte chunks per row per stage
    __shared__ __align__(16) char smem[LDSB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int M = p.M, N = p.N, K = p.K;
    const int n0 = blockIdx.x * NR;

    // Loader side: in load u of fragment j, lane l fetches row u*RPI + l/CPR
    // of the fragment, chunk (l % CPR) ^ f(row) of the stage.
    const int lr = lane / CPR, lp = lane % CPR;
    const int8_t *src[NFR][U];
    int coff[U];  // byte offset of the lane's chunk inside a stage
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int r = u * RPI + lr;
        const int c = lp ^ dec_swz<U>(r);
        coff[u] = 16 * c;
#pragma unroll
        for (int j = 0; j < NFR; ++j) {
            const int8_t *row;
            if (j < NF) {
                const int n = n0 + j * 16 + r;
                row = p.wq + (int64_t)(n < N ? n : N - 1) * K;
            } else {
                const int m = (j - NF) * 16 + r;
                row = p.xq + (int64_t)(m < M ? m : M - 1) * K;
            }
            src[j][u] = row;
        }
    }

    // Steps of this thread's outputs e = tid + 256 q (n fastest), fetched
    // before the loop so the epilogue issues stores only (and so they are
    // older than every ring load).  When NR divides 256 every output of a
    // thread has the same weight row.
    constexpr int EPT = NR * 16 * FT / 256;
    constexpr bool ONE_W = 256 % NR == 0;
    float w_own[ONE_W ? 1 : EPT], x_own[EPT];
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
        const int e = tid + 256 * q;
        const int nn = n0 + e % NR, m = e / NR;
        if (!ONE_W || q == 0) w_own[ONE_W ? 0 : q] = p.ws[nn < N ? nn : N - 1];
        x_own[q] = p.xs[p.xs_per_row ? (m < M ? m : M - 1) : 0];
    }

    // This wave's stages [s0, s0 + n), wave-uniform.
    const int nst = (K + 64 * U - 1) / (64 * U);
    const int per = (nst + 3) / 4;
    const int waveu = __builtin_amdgcn_readfirstlane(wave);
    const int s0 = waveu * per;
    const int n = (s0 + per < nst ? s0 + per : nst) - s0;
    const uint32_t ring = (uint32_t)(uintptr_t)(lds_void_t *)smem + (uint32_t)(waveu * RING);

    auto issue = [&](int t) {  // stage s0 + t into slot t % S
        const int off = (s0 + t) * 64 * U;
        const uint32_t slot = ring + (uint32_t)((t % S) * SLOT);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // A chunk at or past K is not loaded: the lane re-reads the
            // row's first 16 bytes and the reader masks that chunk to zero.
            const int o = off + coff[u] < K ? off + coff[u] : 0;
#pragma unroll
            for (int j = 0; j < NFR; ++j) {
                if (NT && j < NF) lds_dma16_nt(src[j][u] + o, slot + (uint32_t)((j * U + u) * 1024));
                else lds_dma16(src[j][u] + o, slot + (uint32_t)((j * U + u) * 1024));
            }
        }
    };

    using DAcc = std::conditional_t<F8, f32x4, int4v>;
    DAcc acc[NF][FT];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int t = 0; t < FT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[f][t][v] = 0;

    // Reader side: lane (g = lane / 16, i = lane % 16) takes row i, chunk
    // 4 s + g of step s.
    const int ri = lane & 15, rg = lane >> 4;
    const int fi = dec_swz<U>(ri);
    const char *smem_w = smem + waveu * RING + ri * (64 * U);

#pragma unroll
    for (int t = 0; t < S - 1; ++t)
        if (t < n) issue(t);
    for (int t = 0; t < n; ++t) {
        // Stage t has landed once at most min(S - 2, n - 1 - t) later stages
        // are still in flight (loads complete in order).
        wait_stages<S - 2, P>(n - 1 - t);
        if (t + S - 1 < n) {
            // Slot (t - 1) % S is refilled: its LDS reads must be done.
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            issue(t + S - 1);
        }
        const char *sb = smem_w + (t % S) * SLOT;
        const int off = (s0 + t) * 64 * U;
        if constexpr (F8) {
            int4v a[2][NF], b[2][FT];
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const int c = 4 * st + rg;
                const bool ok = off + 16 * c < K;
                const int pos = 16 * (c ^ fi);
#pragma unroll
                for (int f = 0; f < NF; ++f) {
                    const int4v v = *reinterpret_cast<const int4v *>(sb + f * U * 1024 + pos);
                    a[st][f] = ok ? v : int4v{0, 0, 0, 0};
                }
#pragma unroll
                for (int x = 0; x < FT; ++x)
                    b[st][x] = *reinterpret_cast<const int4v *>(sb + (NF + x) * U * 1024 + pos);
            }
#pragma unroll
            for (int f = 0; f < NF; ++f)
#pragma unroll
                for (int x = 0; x < FT; ++x) {
                    const int8x av = __builtin_shufflevector(a[0][f], a[1][f], 0, 1, 2, 3, 4, 5, 6, 7);
                    const int8x bv = __builtin_shufflevector(b[0][x], b[1][x], 0, 1, 2, 3, 4, 5, 6, 7);
                    acc[f][x] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        av, bv, acc[f][x], 0, 0, 0, 0, 0, 0);
                }
            continue;
        }
#pragma unroll
        for (int st = 0; st < U; ++st) {
            const int c = 4 * st + rg;
            const bool ok = off + 16 * c < K;
            const int pos = 16 * (c ^ fi);
            int4v a[NF], b[FT];
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                const int4v v = *reinterpret_cast<const int4v *>(sb + f * U * 1024 + pos);
                a[f] = ok ? v : int4v{0, 0, 0, 0};
            }
#pragma unroll
            for (int x = 0; x < FT; ++x)
                b[x] = *reinterpret_cast<const int4v *>(sb + (NF + x) * U * 1024 + pos);
#pragma unroll
            for (int f = 0; f < NF; ++f)
#pragma unroll
                for (int x = 0; x < FT; ++x)
                    acc[f][x] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[f], b[x], acc[f][x], 0, 0, 0);
        }
    }
    wait_vmcnt<0>();
    __syncthreads();  // every wave is done with its ring: reuse it for the sums

    using RedT = std::conditional_t<F8, float, int>;
    RedT *red = reinterpret_cast<RedT *>(smem);  // [wave][f][t][v * 64 + lane]
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int t = 0; t < FT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                red[((wave * NF + f) * FT + t) * 256 + v * 64 + lane] = acc[f][t][v];
    __syncthreads();

    // 16x16 accumulator layout: lane l, register v holds weight row
    // 4*(l/16) + v and token l%16.  Threads take outputs with n fastest so
    // the stores of a token row are contiguous.
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
        const int e = tid + 256 * q;
        const int nl = e % NR, ml = e / NR;
        const int m = ml, nn = n0 + nl;
        if (m >= M || nn >= N) continue;
        const int f = nl >> 4, i = nl & 15, t = ml >> 4, j = ml & 15;
        const int l = (i >> 2) * 16 + j, v = i & 3;
        RedT a = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) a += red[((w * NF + f) * FT + t) * 256 + v * 64 + l];
        const float cs = x_own[q] * w_own[ONE_W ? 0 : q];
        const int64_t o = (int64_t)m * N + nn;
        store_y<YDT>(p.y, o, (float)a * cs);
        if constexpr (!F8) if (p.acc_out) p.acc_out[o] = a;
    }
}

// ---------------------------------------------------------------- launch

// XCD grid for tile_of: the factorization gm x gn = 8 (gm | tm, gn | tn)
// that fetches the fewest operand bytes per XCD, rm BM + rn BN rows of K
// bytes; none (row-major order) when the tiles do not split 8 ways.
static void set_xcd_grid(GemmArgs &a, int tm, int tn, int bm, int bn) {
    a.tiles_m = tm;
    a.tiles_n = tn;
    a.xcd_gm = a.xcd_gn = 0;
    long best = -1;
    for (int gm = 1; gm <= 8; gm *= 2) {
        const int gn = 8 / gm;
        if (tm % gm || tn % gn) continue;
        const long cost = (long)(tm / gm) * bm + (long)(tn / gn) * bn;
        if (best < 0 || cost < best) {
            best = cost;
            a.xcd_gm = gm;
            a.xcd_gn = gn;
        }
    }
}

template <int BM, int BN, int WM, int WN, bool SIDE>
static void launch_tile_t(GemmArgs &a, int y_dt, hipStream_t stream) {
    const int tm = (a.M + BM - 1) / BM, tn = (a.N + BN - 1) / BN;
    set_xcd_grid(a, tm, tn, BM, BN);
    dim3 grid((unsigned)(tm * tn)), block(256);
    if (y_dt == F32) gemm_tile<BM, BN, WM, WN, F32, SIDE><<<grid, block, 0, stream>>>(a);
    else if (y_dt == F16) gemm_tile<BM, BN, WM, WN, F16, SIDE><<<grid, block, 0, stream>>>(a);
    else gemm_tile<BM, BN, WM, WN, BF16, SIDE><<<grid, block, 0, stream>>>(a);
}

template <int BM, int BN, int WM, int WN, int STA, int STB, bool SIDE, bool F8 = false>
static void launch_pipe_t(GemmArgs &a, int y_dt, hipStream_t stream) {
    const int tm = (a.M + BM - 1) / BM, tn = (a.N + BN - 1) / BN;
    set_xcd_grid(a, tm, tn, BM, BN);
    dim3 grid((unsigned)(tm * tn)), block(64 * WM * WN);
    if (y_dt == F32) gemm_pp<BM, BN, WM, WN, STA, STB, F32, SIDE, F8><<<grid, block, 0, stream>>>(a);
    else if (y_dt == F16) gemm_pp<BM, BN, WM, WN, STA, STB, F16, SIDE, F8><<<grid, block, 0, stream>>>(a);
    else gemm_pp<BM, BN, WM, WN, STA, STB, BF16, SIDE, F8><<<grid, block, 0, stream>>>(a);
}

template <int BM, int BN, int STA>
static void launch_pk_t(GemmArgs &a, int y_dt, hipStream_t stream) {
    const int tm = (a.M + BM - 1) / BM, tn = (a.N + BN - 1) / BN;
    set_xcd_grid(a, tm, tn, BM, BN);
    dim3 grid((unsigned)(tm * tn)), block(512);
    if (y_dt == F32) gemm_pk<BM, BN, STA, F32><<<grid, block, 0, stream>>>(a);
    else if (y_dt == F16) gemm_pk<BM, BN, STA, F16><<<grid, block, 0, stream>>>(a);
    else gemm_pk<BM, BN, STA, BF16><<<grid, block, 0, stream>>>(a);
}

template <int NF, int FT, int U, int S, bool NT, bool F8 = false>
static void launch_dec_t(GemmArgs &a, int y_dt, hipStream_t stream) {
    dim3 grid((unsigned)((a.N + 16 * NF - 1) / (16 * NF))), block(256);
    if (y_dt == F32) gemm_dec<NF, FT, U, S, F32, NT, F8><<<grid, block, 0, stream>>>(a);
    else if (y_dt == F16) gemm_dec<NF, FT, U, S, F16, NT, F8><<<grid, block, 0, stream>>>(a);
    else gemm_dec<NF, FT, U, S, BF16, NT, F8><<<grid, block, 0, stream>>>(a);
}

// Decode above 16 tokens: 112 weight rows per block instead of 128 when
// that fills the 256 CUs clearly better (N = 28672: 256 blocks against 224).
static bool dec_rows_112(int64_t N) {
    auto fill = [](int64_t blocks) {  // busy fraction of the CUs over all rounds
        const int64_t rounds = (blocks + 255) / 256;
        return (double)blocks / (double)(rounds * 256);
    };
    return fill((N + 111) / 112) > fill((N + 127) / 128) + 0.02;
}

// Tile shape: the candidate whose tiles fill the 256 CUs best, weighted by
// how much MFMA work each tile does per byte staged through LDS.
static int pick_tile(int64_t M, int64_t N, int64_t K) {
    struct C { int bm, bn; double eff; int per_cu; };
    // 256 x 128 relative to 256 x 256: 0.85 per unit of work at long K, 0.72
    // at K <= 2048, where each tile's prologue and epilogue weigh more
    // (4096 x 4096 x 1024: one round of 256 x 256 tiles 24.2 us, two of
    // 256 x 128 33.4 us; 4096 x 6144 x 1024: 38.8 us against 45.0).
    const double eff1 = K <= 2048 ? 0.72 : 0.85;
    const C cands[3] = {{256, 256, 1.0, 1}, {256, 128, eff1, 1}, {128, 128, 0.7, 2}};
    int best = 0;
    double best_score = -1;
    for (int i = 0; i < 3; ++i) {
        const int64_t tiles = ((M + cands[i].bm - 1) / cands[i].bm) * ((N + cands[i].bn - 1) / cands[i].bn);
        const int64_t slots = 256 * cands[i].per_cu;
        const int64_t rounds = (tiles + slots - 1) / slots;
        const double score = (double)tiles / (double)(rounds * slots) * cands[i].eff;
        if (score > best_score + 1e-9) { best_score = score; best = i; }
    }
    // 256 x 128 tiles leaving at least half the CUs idle: 128 x 128 tiles
    // give every CU a block; at a short K four waves (measured at
    // 4096 x 1024 x 1024: 11.1 us against 12.3-12.8), at a long K eight in
    // K-split pairs (4096 x 1024 x 3072: 21.1 us against 23.5 with four
    // waves and 25.8 on 256 x 128 tiles; at K = 1024 the pairs gain nothing).
    const int64_t t1 = ((M + 255) / 256) * ((N + 127) / 128);
    const int64_t t2 = ((M + 127) / 128) * ((N + 127) / 128);
    if (best == 1 && t1 <= 128 && t2 >= 256) return K <= 2048 ? 2 : 3;
    return best;
}

void launch_gemm(const int8_t *xq, const int8_t *wq, int64_t M, int64_t N, int64_t K,
                 const float *x_scale, int per_row, const float *w_scale, void *y, int y_dt,
                 int32_t *acc_out, const SideTerm *side, hipStream_t stream, int force_tile) {
    // K >= 16 past the C ABI's checks; every kernel below clamps its tail
    // loads to the last K stage or chunk, which must exist.
    if (M <= 0 || N <= 0 || K <= 0) return;
    GemmArgs a{};
    a.xq = xq; a.wq = wq; a.M = (int)M; a.N = (int)N; a.K = (int)K;
    a.xs = x_scale; a.xs_per_row = per_row; a.ws = w_scale; a.y = y; a.acc_out = acc_out;
    const bool pipe = K % 128 == 0;
    // force_tile 0 | 1 | 2 | 3 (the coverage entry points) overrides the choice.
    const int tile = force_tile >= 0 && force_tile <= 3 ? force_tile : pick_tile(M, N, K);
    if (side) {
        // With the side term 256 x 256 tiles would need the side sums next
        // to 128 accumulator registers: the 256-row choices take 256 x 128.
        a.x16 = side->x16; a.w16 = side->w16; a.idx = side->idx; a.count = side->count;
        a.xo = side->xo; a.wo = side->wo; a.side_cap = side->xo && side->wo ? side->cap : -1;
        // (the K-split pairs have no side-term form: their choice keeps 256 x 128)
        if (pipe && (tile < 2 || tile == 3)) launch_pipe_t<256, 128, 4, 2, 3, 3, true>(a, y_dt, stream);
        else if (pipe) launch_pipe_t<128, 128, 2, 2, 2, 2, true>(a, y_dt, stream);
        else launch_tile_t<128, 128, 2, 2, true>(a, y_dt, stream);
        return;
    }
    if (M <= 32) {
        // Weight rows per block and ring shape by token count: more rows
        // per block as M grows (each block re-reads all M token rows: 128
        // weight rows per block above 16 tokens, measured 43 us against
        // 47 us with 64 at M = 32, or 112 where that fills the CUs better:
        // 40 us at N = 28672), two 64-byte K steps a stage so that a
        // stage covers whole 128-byte lines of every row (the nontemporal
        // weight stream then fetches each line once).
        if (M <= 8) launch_dec_t<1, 1, 2, 4, true>(a, y_dt, stream);
        else if (M <= 16) launch_dec_t<4, 1, 2, 2, true>(a, y_dt, stream);
        else if (dec_rows_112(N)) launch_dec_t<7, 2, 2, 2, true>(a, y_dt, stream);
        else launch_dec_t<8, 2, 2, 2, true>(a, y_dt, stream);
        return;
    }
    if (pipe) {
        switch (tile) {
            case 0: launch_pipe_t<256, 256, 4, 2, 2, 2, false>(a, y_dt, stream); break;
            case 1: launch_pipe_t<256, 128, 4, 2, 3, 3, false>(a, y_dt, stream); break;
            case 3: launch_pk_t<128, 128, 3>(a, y_dt, stream); break;
            default: launch_pipe_t<128, 128, 2, 2, 2, 2, false>(a, y_dt, stream); break;
        }
        return;
    }
    switch (tile) {  // (3, the K-split pairs, needs K % 128 == 0: as 1 here)
        case 0: launch_tile_t<256, 256, 2, 2, false>(a, y_dt, stream); break;
        case 1: case 3: launch_tile_t<256, 128, 2, 2, false>(a, y_dt, stream); break;
        default: launch_tile_t<128, 128, 2, 2, false>(a, y_dt, stream); break;
    }
}

// e4m3 x e4m3 -> fp32 GEMM with the same dequant epilogue (K % 128 == 0):
// the decode kernel for M <= 32 (same ring shapes as int8), else the
// pipelined one.
void launch_gemm_fp8(const uint8_t *xq, const uint8_t *wq, int64_t M, int64_t N, int64_t K,
                     const float *x_scale, int per_row, const float *w_scale, void *y, int y_dt,
                     hipStream_t stream, int force_tile) {
    if (M <= 0 || N <= 0 || K <= 0) return;  // tail loads clamp to the last stage
    GemmArgs a{};
    a.xq = reinterpret_cast<const int8_t *>(xq);
    a.wq = reinterpret_cast<const int8_t *>(wq);
    a.M = (int)M; a.N = (int)N; a.K = (int)K;
    a.xs = x_scale; a.xs_per_row = per_row; a.ws = w_scale; a.y = y;
    if (M <= 32) {
        if (M <= 8) launch_dec_t<1, 1, 2, 4, true, true>(a, y_dt, stream);
        else if (M <= 16) launch_dec_t<4, 1, 2, 2, true, true>(a, y_dt, stream);
        else if (dec_rows_112(N)) launch_dec_t<7, 2, 2, 2, true, true>(a, y_dt, stream);
        else launch_dec_t<8, 2, 2, 2, true, true>(a, y_dt, stream);
        return;
    }
    // (the K-split pairs, tile 3, are int8 only: their choice keeps 256 x 128)
    const int t = force_tile >= 0 && force_tile <= 2 ? force_tile : pick_tile(M, N, K);
    const int tile = t == 3 ? 1 : t;
    switch (tile) {
        case 0: launch_pipe_t<256, 256, 4, 2, 2, 2, false, true>(a, y_dt, stream); break;
        case 1: launch_pipe_t<256, 128, 4, 2, 3, 3, false, true>(a, y_dt, stream); break;
        default: launch_pipe_t<128, 128, 2, 2, 2, 2, false, true>(a, y_dt, stream); break;
    }
}

}  // namespace sq
