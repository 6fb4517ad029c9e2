/*
 * Seeded synthetic inputs for the attention workloads: i.i.d. standard
 * normal values rounded to bfloat16.
 *
 * This file holds no attention arithmetic.  It is shared by the CPU oracle
 * and by the GPU path only as a source of identical input bytes.
 *
 * Generator (counter based, so any element can be produced on its own):
 *   state_0 = seed * 2^8 + tensor_id
 *   u64_i   = splitmix64_mix(state_0 + (i + 1) * GOLDEN_GAMMA)
 *   u1 = (hi32(u64_i) + 0.5) / 2^32,  u2 = lo32(u64_i) / 2^32
 *   z  = sqrt(-2 ln u1) * cos(2 pi u2)          (Box-Muller, fp64)
 *   out = bf16_rne(float(z))
 * SplitMix64 is the mixing function of Steele, Lea and Flood, "Fast
 * splittable pseudorandom number generators" (OOPSLA 2014).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* float -> bfloat16 bits, round to nearest, ties to even (finite inputs). */
static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* Fill out[0..n) with elements [first, first+n) of stream (seed, tensor_id). */
void synth_gaussian_bf16(uint64_t seed, uint32_t tensor_id, uint64_t first, uint64_t n,
                         uint16_t* out) {
    const uint64_t state0 = seed * 256u + (uint64_t)tensor_id;
    const double two_pi = 6.283185307179586476925286766559;
    #pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < (int64_t)n; ++k) {
        uint64_t i = first + (uint64_t)k;
        uint64_t h = mix64(state0 + (i + 1u) * GOLDEN_GAMMA);
        double u1 = ((double)(h >> 32) + 0.5) * (1.0 / 4294967296.0);
        double u2 = (double)(h & 0xFFFFFFFFu) * (1.0 / 4294967296.0);
        double z = sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
        out[k] = f32_to_bf16_rne((float)z);
    }
}
