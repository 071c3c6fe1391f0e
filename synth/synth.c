/*
 * synth.c -- seeded, counter-based generators for synthetic decoder inputs.
 *
 * This file holds NO arithmetic of the decode method. It only draws numbers:
 * bf16 weights from a normal distribution, token ids from a uniform one, and
 * the N(0,1) key/value prefill of the long-context workloads. Both the CPU
 * oracle and the GPU path consume the bytes written here, so they see exactly
 * the same inputs.
 *
 * Generator definition (stable; changing it changes every workload):
 *   key(seed, name)  = mix64(mix64(seed + G) ^ fnv1a64(name))
 *   u64(key, i)      = mix64(key + (i + 1) * G),   G = 0x9E3779B97F4A7C15
 *   mix64            = the SplitMix64 output finaliser (Steele, Lea, Flood,
 *                      "Fast splittable pseudorandom number generators",
 *                      OOPSLA 2014): xor-shift 30, * 0xBF58476D1CE4E5B9,
 *                      xor-shift 27, * 0x94D049BB133111EB, xor-shift 31.
 *   uniform(key, i)  = ((u64(key, i) >> 11) + 0.5) * 2^-53      in (0, 1)
 *   normal(key, i)   = Box-Muller on the pair (2*(i/2), 2*(i/2)+1):
 *                      r = sqrt(-2 ln u_a), phi = 2 pi u_b,
 *                      even i -> r cos(phi), odd i -> r sin(phi)
 *   value            = bf16_rne((float)(mean + std * normal))
 *   token(key, i)    = floor(uniform(key, i) * V)
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SYN_G 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ULL;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBULL;
    z ^= z >> 31;
    return z;
}

static inline double uni(uint64_t key, uint64_t i) {
    uint64_t x = mix64(key + (i + 1) * SYN_G);
    return ((double)(x >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

uint64_t syn_key(uint64_t seed, const char *name) {
    uint64_t h = 0xcbf29ce484222325ULL;
    for (const unsigned char *p = (const unsigned char *)name; *p; ++p) {
        h ^= *p;
        h *= 0x100000001b3ULL;
    }
    return mix64(mix64(seed + SYN_G) ^ h);
}

/* out[i] = bf16(mean + std * normal(key, i)) for i in [0, n). */
void syn_normal_bf16(uint64_t key, double mean, double std, int64_t n, uint16_t *out) {
    const double two_pi = 6.283185307179586476925286766559;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < (n + 1) / 2; ++j) {
        double ua = uni(key, (uint64_t)(2 * j));
        double ub = uni(key, (uint64_t)(2 * j + 1));
        double r = sqrt(-2.0 * log(ua));
        double phi = two_pi * ub;
        out[2 * j] = f32_to_bf16_rne((float)(mean + std * (r * cos(phi))));
        if (2 * j + 1 < n) out[2 * j + 1] = f32_to_bf16_rne((float)(mean + std * (r * sin(phi))));
    }
}

/* out[i] = floor(uniform(key, i) * vocab), in [0, vocab). */
void syn_tokens(uint64_t key, int64_t n, int32_t vocab, int32_t *out) {
    for (int64_t i = 0; i < n; ++i) {
        int32_t t = (int32_t)(uni(key, (uint64_t)i) * (double)vocab);
        out[i] = t < vocab ? t : vocab - 1;
    }
}

/* Raw draws, exposed so a test can re-derive the stream independently. */
void syn_uniform(uint64_t key, int64_t n, double *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = uni(key, (uint64_t)i);
}
