/*
 * Seeded synthetic input generator (host only, no GPU code).
 *
 * Holds none of the decoder arithmetic: it only draws the random weights,
 * activations, context lengths and KV fills that both the HIP path and the
 * CPU oracle consume, so every tensor is reproducible on its own.
 *
 * Generator: counter-based splitmix64. Element i of stream s takes the
 * 64-bit words w(2i) and w(2i+1), where
 *     w(c) = mix64(key(s) + (c + 1) * 0x9E3779B97F4A7C15)
 *     key(s) = mix64(seed ^ mix64(s + 0xD1B54A32D192ED03))
 * and mix64 is the splitmix64 finaliser (Steele, Lea, Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014). The two words
 * become uniforms u1 in (0,1], u2 in [0,1) and a standard normal by the
 * Box-Muller transform, z = sqrt(-2 ln u1) cos(2 pi u2), all in fp64.
 * Values leave as fp32: mean + std * z rounded to nearest even.
 * bf16 conversion (round to nearest even on the fp32 bits) is separate.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
    return mix64(seed ^ mix64(stream + 0xD1B54A32D192ED03ULL));
}

static inline uint64_t word(uint64_t key, uint64_t counter) {
    return mix64(key + (counter + 1) * 0x9E3779B97F4A7C15ULL);
}

static inline double normal_at(uint64_t key, uint64_t i) {
    const double two_m53 = 1.1102230246251565e-16; /* 2^-53 */
    const double u1 = ((double)(word(key, 2 * i) >> 11) + 1.0) * two_m53;
    const double u2 = (double)(word(key, 2 * i + 1) >> 11) * two_m53;
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

/* out[j] = (float)(mean + std * z(offset + j)), j < n. */
void sttd_synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n, double mean, double std,
                           float *out) {
    const uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        out[j] = (float)(mean + std * normal_at(key, offset + (uint64_t)j));
    }
}

/* out[j] uniform integer in [lo, hi] (inclusive), from the top 53 bits of w(j). */
void sttd_synth_uniform_int(uint64_t seed, uint64_t stream, int64_t n, int32_t lo, int32_t hi, int32_t *out) {
    const uint64_t key = stream_key(seed, stream);
    const double span = (double)hi - (double)lo + 1.0;
    for (int64_t j = 0; j < n; ++j) {
        const double u = (double)(word(key, (uint64_t)j) >> 11) * 1.1102230246251565e-16;
        int64_t v = (int64_t)lo + (int64_t)floor(u * span);
        if (v > hi) v = hi;
        out[j] = (int32_t)v;
    }
}

/* fp32 -> bf16 bits, round to nearest even; NaN stays NaN (quiet). */
void sttd_synth_f32_to_bf16(const float *in, uint16_t *out, int64_t n) {
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        uint32_t u;
        memcpy(&u, &in[j], 4);
        if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) {
            out[j] = (uint16_t)((u >> 16) | 0x40u);
            continue;
        }
        const uint32_t bias = 0x7FFFu + ((u >> 16) & 1u);
        out[j] = (uint16_t)((u + bias) >> 16);
    }
}
