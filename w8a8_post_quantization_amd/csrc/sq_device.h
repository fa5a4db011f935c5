// Device-side helpers shared by the gfx950 kernels: 16-byte vector loads,
// element widening, wave-level reductions and the int8 quantizer step.
// Compiled with -ffp-contract=off: every a*b and a+b below is its own
// IEEE binary32 operation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sq {

constexpr int kWave = 64;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef int int4v __attribute__((ext_vector_type(4)));
typedef int int16v __attribute__((ext_vector_type(16)));

enum Dt { F32 = 0, F16 = 1, BF16 = 2 };

// Element count of one 16-byte vector of each type, and bytes per element.
template <int DT> struct Vec { static constexpr int n = DT == F32 ? 4 : 8; };
constexpr int dt_bytes(int dt) { return dt == F32 ? 4 : 2; }

// Widen the elements of one 16-byte vector to fp32 (exact for all types).
template <int DT>
__device__ __forceinline__ void widen16(const uint4 &v, float *out) {
    if constexpr (DT == F32) {
        out[0] = __uint_as_float(v.x);
        out[1] = __uint_as_float(v.y);
        out[2] = __uint_as_float(v.z);
        out[3] = __uint_as_float(v.w);
    } else if constexpr (DT == F16) {
        half8 h = __builtin_bit_cast(half8, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = (float)h[i];
    } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = __uint_as_float(w[i] << 16);
            out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
}

typedef unsigned int u4v __attribute__((ext_vector_type(4)));

// 16-byte load with the nontemporal hint, for data each kernel reads once
// (streamed weights and activations): it keeps the streams from displacing
// reused data in the caches and measurably raises the sustained HBM read rate.
__device__ __forceinline__ uint4 ld_nt(const uint4 *p) {
    const u4v v = __builtin_nontemporal_load(reinterpret_cast<const u4v *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// A 16-byte load of an input that is read once (NTL: nontemporal, for
// inputs larger than the caches) or that the next kernel reads again (a
// plain load, so it stays cached: LLM.int8() reads X in its outlier
// detection and again in its quantizer).  Inputs above this many bytes
// take the nontemporal form.
constexpr int64_t kNtLoadBytes = (int64_t)64 << 20;
template <bool NTL>
__device__ __forceinline__ uint4 ld16(const uint4 *p) {
    if constexpr (NTL) return ld_nt(p);
    else return *p;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

// Narrow fp32 to the output type with round-to-nearest-even.
template <int DT> struct OutT;
template <> struct OutT<F32> { using T = float; };
template <> struct OutT<F16> { using T = _Float16; };
template <> struct OutT<BF16> { using T = __bf16; };

// The empty asm pins the fp32 value in a register: without it the compiler
// may fold "fp32 multiply, then convert to fp16" into one mixed-precision
// fma that rounds the exact product once, which differs from rounding to
// fp32 first whenever the fp32 result is an fp16 tie.
__device__ __forceinline__ float materialize(float v) {
    asm volatile("" : "+v"(v));
    return v;
}

template <int DT>
__device__ __forceinline__ typename OutT<DT>::T narrow(float v) {
    if constexpr (DT == F32) return v;
    else return (typename OutT<DT>::T)materialize(v);
}

}  // namespace sq
