/*
 * synth.c -- seeded synthetic input generator shared by the tests, the
 * benchmark and the oracle's callers.  It draws inputs only: it holds none of
 * the projection's arithmetic (no ternarisation, no scaling, no products).
 *
 * Generators, each written from its published definition:
 *   - SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
 *     generators", OOPSLA 2014): the i-th output of the stream with seed s is
 *     mix(s + (i + 1) * 0x9E3779B97F4A7C15), so every element is a pure
 *     function of (stream seed, index) and the fill is parallel and
 *     independent of the thread count;
 *   - uniform doubles in (0, 1]: the top 53 bits plus one, times 2^-53;
 *   - normals: the Box-Muller transform (Box and Muller 1958) on the draw pair
 *     (2p, 2p + 1), cosine branch for element 2p and sine branch for 2p + 1;
 *   - integers in [lo, hi]: Lemire's multiply-shift range reduction of the top
 *     32 bits (Lemire 2019);
 *   - bf16: round-to-nearest-even of the fp32 value.
 * Stream seeds are SplitMix64 mixes of (base seed, config, projection, tensor).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t draw(uint64_t seed, uint64_t i) { return mix64(seed + (i + 1) * GOLDEN); }

static inline double unit_open0(uint64_t x) { /* (0, 1] */
    return ((double)(x >> 11) + 1.0) * (1.0 / 9007199254740992.0);
}

static inline double normal_at(uint64_t seed, int64_t i) {
    uint64_t p = (uint64_t)i >> 1;
    double u1 = unit_open0(draw(seed, 2 * p));
    double u2 = unit_open0(draw(seed, 2 * p + 1));
    double rad = sqrt(-2.0 * log(u1));
    double ang = 6.283185307179586476925286766559 * u2;
    return (i & 1) ? rad * sin(ang) : rad * cos(ang);
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

uint64_t synth_stream_seed(uint64_t base, uint64_t config_id, uint64_t proj_id, uint64_t tensor_id) {
    uint64_t s = mix64(base + GOLDEN);
    s = mix64(s ^ (config_id + 1) * GOLDEN);
    s = mix64(s ^ (proj_id + 1) * 0xD1B54A32D192ED03ULL);
    s = mix64(s ^ (tensor_id + 1) * 0xAEF17502108EF2D9ULL);
    return s;
}

uint64_t synth_u64(uint64_t seed, uint64_t i) { return draw(seed, i); }

void synth_normal_f32(uint64_t seed, int64_t n, double mean, double std, float *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = (float)(mean + std * normal_at(seed, i));
}

void synth_normal_bf16(uint64_t seed, int64_t n, double mean, double std, uint16_t *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = f32_to_bf16_rne((float)(mean + std * normal_at(seed, i)));
}

void synth_uniform_f32(uint64_t seed, int64_t n, double lo, double hi, float *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = (float)(lo + (hi - lo) * unit_open0(draw(seed, (uint64_t)i)));
}

void synth_lognormal_f32(uint64_t seed, int64_t n, double mu, double sigma, float *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = (float)exp(mu + sigma * normal_at(seed, i));
}

static inline int64_t int_at(uint64_t seed, uint64_t i, int64_t lo, int64_t hi) {
    uint64_t range = (uint64_t)(hi - lo + 1);
    uint64_t top = draw(seed, i) >> 32;
    return lo + (int64_t)((top * range) >> 32);
}

void synth_int8_uniform(uint64_t seed, int64_t n, int32_t lo, int32_t hi, int8_t *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = (int8_t)int_at(seed, (uint64_t)i, lo, hi);
}

/* zero with probability p_zero, else sign * magnitude with the sign fair and
 * the magnitude uniform in [mag_lo, mag_hi]; three draws per element */
void synth_int8_zero_or_pm(uint64_t seed, int64_t n, double p_zero, int32_t mag_lo, int32_t mag_hi,
                           int8_t *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        uint64_t b = 3 * (uint64_t)i;
        double u = unit_open0(draw(seed, b));
        if (u <= p_zero) { out[i] = 0; continue; }
        int64_t mag = int_at(seed, b + 1, mag_lo, mag_hi);
        int neg = (int)(draw(seed, b + 2) >> 63);
        out[i] = (int8_t)(neg ? -mag : mag);
    }
}

void synth_f32_to_bf16(const float *src, int64_t n, uint16_t *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = f32_to_bf16_rne(src[i]);
}

void synth_sample_indices(uint64_t seed, int64_t n, int64_t range, int64_t *out) {
    /* n distinct-ish indices in [0, range): one draw each, sorted by caller */
    for (int64_t i = 0; i < n; i++) out[i] = int_at(seed, (uint64_t)i, 0, range - 1);
}
