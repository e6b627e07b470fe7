/*
 * Seeded synthetic inputs for the DSA lightning indexer workloads.
 *
 * This file draws random numbers and nothing else: it holds none of the
 * indexer's arithmetic.  Both the HIP path and the CPU oracle receive the
 * very same bytes from it.
 *
 * Generator: element i of the stream (seed, tensor, layer) is produced from
 * SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014; the finaliser constants are the published
 * ones) applied to a counter, so every element can be drawn independently
 * and in parallel.  Normal variates use the Box-Muller transform on two
 * 53-bit uniforms; the fp64 sample is narrowed to fp32 and then to bf16
 * with round-to-nearest-even on the bit pattern.  That double narrowing is
 * deliberate and harmless for a generator (it only fixes which bf16 values
 * appear); it is not the rounding the method itself specifies.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static uint64_t sm64(uint64_t z) {
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* Key of one stream; streams for different (seed, tensor, layer) are unrelated. */
static uint64_t stream_key(uint64_t seed, uint64_t tensor, uint64_t layer) {
    return sm64(sm64(sm64(seed) ^ (tensor * 0xD1B54A32D192ED03ull)) ^ (layer * 0x8CB92BA72F3D8DD7ull));
}

/* Uniform in [0, 1) with 53 random bits, for counter c of the stream. */
static double unif53(uint64_t key, uint64_t c) {
    return (double)(sm64(key ^ sm64(c)) >> 11) * 0x1.0p-53;
}

static uint16_t narrow_bf16(double v) {
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)(u >> 16); /* inf stays inf */
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* out[i] = bf16(mean + std * N_{first + i}), N_j standard normal, i in [0, n): elements
 * first .. first + n - 1 of the stream (pair p of Box-Muller gives elements 2p and 2p + 1). */
void synth_normal_bf16_range(uint64_t seed, uint64_t tensor, uint64_t layer, double mean,
                             double std, int64_t first, int64_t n, uint16_t *out) {
    const uint64_t key = stream_key(seed, tensor, layer);
    const double two_pi = 6.283185307179586476925286766559;
    const int64_t p0 = first / 2, p1 = (first + n + 1) / 2;
#pragma omp parallel for schedule(static)
    for (int64_t p = p0; p < p1; ++p) {
        double u1 = unif53(key, 2 * (uint64_t)p);
        double u2 = unif53(key, 2 * (uint64_t)p + 1);
        double r = sqrt(-2.0 * log(1.0 - u1));
        double a = two_pi * u2;
        const int64_t e = 2 * p - first;
        if (e >= 0 && e < n) out[e] = narrow_bf16(mean + std * r * cos(a));
        if (e + 1 >= 0 && e + 1 < n) out[e + 1] = narrow_bf16(mean + std * r * sin(a));
    }
}

/* out[i] = bf16(mean + std * N_i), i in [0, n). */
void synth_normal_bf16(uint64_t seed, uint64_t tensor, uint64_t layer, double mean, double std,
                       int64_t n, uint16_t *out) {
    synth_normal_bf16_range(seed, tensor, layer, mean, std, 0, n, out);
}

/* out[i] uniform in [0, 1) (53-bit), i in [0, n). */
void synth_uniform_f64(uint64_t seed, uint64_t tensor, uint64_t layer, int64_t n, double *out) {
    const uint64_t key = stream_key(seed, tensor, layer);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = unif53(key, (uint64_t)i);
}

/* out[i] uniform integer in [lo, hi] inclusive, i in [0, n). */
void synth_uniform_int(uint64_t seed, uint64_t tensor, uint64_t layer, int64_t lo, int64_t hi,
                       int64_t n, int64_t *out) {
    const uint64_t key = stream_key(seed, tensor, layer);
    const uint64_t span = (uint64_t)(hi - lo) + 1u;
    for (int64_t i = 0; i < n; ++i) {
        /* 128-bit multiply-high maps 64 random bits onto [0, span) */
        unsigned __int128 m = (unsigned __int128)sm64(key ^ sm64((uint64_t)i)) * span;
        out[i] = lo + (int64_t)(uint64_t)(m >> 64);
    }
}
