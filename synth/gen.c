/*
 * Seeded synthetic input generator shared by the GPU path's tests/bench and
 * by the CPU oracle's tests.  It holds none of the quantization method's
 * arithmetic: it only draws numbers.
 *
 * Generator: SplitMix64 (Steele, Lea & Flood, "Fast Splittable Pseudorandom
 * Number Generators", OOPSLA 2014; the 64-bit finaliser as published by
 * Vigna in splitmix64.c).  SplitMix64's i-th output (i = 0, 1, ...) from
 * state `key` is mix64(key + (i + 1) * GAMMA), so it is used here as a
 * counter-based generator: element i of a stream can be computed on its own,
 * which makes the fill parallel and independent of the thread count.
 *
 * Stream key: key = mix64(seed * 1000 + stream_id).
 * Uniform:    u = (r >> 11) * 2^-53, in [0, 1).
 * Normal:     Box-Muller in double from counters 2i and 2i+1:
 *             z_i = sqrt(-2 ln(1 - u_{2i})) * cos(2 pi u_{2i+1}).
 */
#include <math.h>
#include <stdint.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static uint64_t stream_key(uint64_t seed, uint64_t stream_id) {
    return mix64(seed * 1000ULL + stream_id);
}

static double u01(uint64_t key, uint64_t counter) {
    uint64_t r = mix64(key + (counter + 1ULL) * GAMMA);
    return (double)(r >> 11) * (1.0 / 9007199254740992.0);
}

static double normal_at(uint64_t key, uint64_t i) {
    const double two_pi = 6.283185307179586476925286766559;
    double u1 = 1.0 - u01(key, 2 * i); /* (0, 1] */
    double u2 = u01(key, 2 * i + 1);
    return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

/* out[i] = (float)(mean + std * z_i), i in [0, n).  Rounded once to fp32. */
void synth_normal_f32(uint64_t seed, uint64_t stream_id, double mean, double std,
                      float *out, int64_t n) {
    uint64_t key = stream_key(seed, stream_id);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = (float)(mean + std * normal_at(key, (uint64_t)i));
}

/* out[i] = u_i in [0, 1), in double. */
void synth_uniform_f64(uint64_t seed, uint64_t stream_id, double *out, int64_t n) {
    uint64_t key = stream_key(seed, stream_id);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = u01(key, (uint64_t)i);
}

/* Raw 64-bit outputs, for tests of the generator itself. */
void synth_raw_u64(uint64_t key, uint64_t *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        out[i] = mix64(key + ((uint64_t)i + 1ULL) * GAMMA);
}
