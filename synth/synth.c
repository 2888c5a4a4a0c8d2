/*
 * Seeded synthetic inputs for the MoE layer: host side.
 *
 * This file holds no arithmetic of the MoE method.  It only turns
 * (seed, stream, index) into bytes, codes, scales and normal variates, so
 * that the CPU oracle and the HIP path can be fed identical tensors.  The
 * device twin in synth_dev.hip implements the same integer definitions
 * (it has no normals: those are drawn here only and copied over, so no
 * transcendental function ever differs between the two sides).
 *
 * Generator: SplitMix64 (G. L. Steele, D. Lea, C. H. Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014).  The i-th
 * output of a SplitMix64 stream seeded with `key` is
 *     mix(key + (i + 1) * GAMMA)
 * with GAMMA = 0x9E3779B97F4A7C15 and mix() the published finaliser.
 * Each tensor gets its own key:  key = mix(mix(seed + GAMMA) ^ stream).
 *
 * Derived values (index i counts elements of the tensor):
 *   raw byte b      : byte (b & 7) of word(b >> 3), little-endian.  For
 *                     packed int4 / int2 weights this byte IS the packed
 *                     code byte: any byte is a valid pair of two's-complement
 *                     nibbles in [-8,7] or four 2-bit fields in [-2,1], each
 *                     uniform.
 *   int8 code i     : v = 16-bit field (i & 3) of word(i >> 2);
 *                     code = ((v * 255) >> 16) - 127, in [-127, 127].
 *   scale i         : (float)((0.5 + (word(i) >> 40) * 2^-24) * c), where c
 *                     is a double the caller passes (1/sqrt(in_dim)); the
 *                     fp64 multiply is exact-rounded on every IEEE machine.
 *   normal i        : Box-Muller on u1 = ((word(2i) >> 11) + 1) * 2^-53 and
 *                     u2 = (word(2i+1) >> 11) * 2^-53:
 *                     (float)(sigma * sqrt(-2 ln u1) * cos(2 pi u2)).
 *   uniform i       : (word(i) >> 11) * 2^-53, a double in [0, 1).
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t synth_mix(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, uint64_t stream)
{
    return synth_mix(synth_mix(seed + SYNTH_GAMMA) ^ stream);
}

uint64_t synth_word(uint64_t key, uint64_t i)
{
    return synth_mix(key + (i + 1) * SYNTH_GAMMA);
}

/* out[j] = raw byte (b0 + j), j < n */
void synth_bytes(uint64_t key, uint64_t b0, uint64_t n, uint8_t *out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < (int64_t)n; j++) {
        uint64_t b = b0 + (uint64_t)j;
        out[j] = (uint8_t)(synth_word(key, b >> 3) >> (8 * (b & 7)));
    }
}

/* out[j] = int8 code (i0 + j), j < n */
void synth_int8_codes(uint64_t key, uint64_t i0, uint64_t n, int8_t *out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < (int64_t)n; j++) {
        uint64_t i = i0 + (uint64_t)j;
        uint64_t v = (synth_word(key, i >> 2) >> (16 * (i & 3))) & 0xFFFFULL;
        out[j] = (int8_t)((int)((v * 255ULL) >> 16) - 127);
    }
}

/* out[j] = scale (i0 + j), j < n */
void synth_scales(uint64_t key, uint64_t i0, uint64_t n, double c, float *out)
{
    for (uint64_t j = 0; j < n; j++) {
        uint64_t u24 = synth_word(key, i0 + j) >> 40;
        out[j] = (float)((0.5 + (double)u24 * 0x1p-24) * c);
    }
}

/* out[j] = uniform (i0 + j), j < n */
void synth_uniforms(uint64_t key, uint64_t i0, uint64_t n, double *out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < (int64_t)n; j++)
        out[j] = (double)(synth_word(key, i0 + (uint64_t)j) >> 11) * 0x1p-53;
}

/* out[j] = normal (i0 + j) * sigma, j < n */
void synth_normals(uint64_t key, uint64_t i0, uint64_t n, double sigma, float *out)
{
    const double two_pi = 6.283185307179586476925286766559;
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < (int64_t)n; j++) {
        uint64_t i = i0 + (uint64_t)j;
        double u1 = ((double)(synth_word(key, 2 * i) >> 11) + 1.0) * 0x1p-53;
        double u2 = (double)(synth_word(key, 2 * i + 1) >> 11) * 0x1p-53;
        out[j] = (float)(sigma * sqrt(-2.0 * log(u1)) * cos(two_pi * u2));
    }
}
