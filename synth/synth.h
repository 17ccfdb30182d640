/*
 * synth.h -- seeded, counter-based generator for the synthetic inputs of the
 * int4 MoE FFN layer (router weights, router bias, expert weights, tokens).
 *
 * This module produces INPUTS only. It holds none of the layer's arithmetic
 * (no quantisation, routing, activation or combine): both the CPU checker and
 * the GPU library consume what it produces, and nothing else is shared
 * between them.
 *
 * Definition (published algorithms, written out here):
 *   - SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable pseudorandom
 *     number generators", OOPSLA 2014): state advances by the golden-ratio
 *     constant 0x9E3779B97F4A7C15; the output is the state passed through the
 *     variant-13 finaliser (shift 30, mul 0xBF58476D1CE4E5B9, shift 27,
 *     mul 0x94D049BB133111EB, shift 31).  Used counter-style: output number
 *     i of the stream with key k is mix(k + (i+1) * golden).
 *   - Gaussian by the Irwin-Hall sum of twelve uniforms: S = sum of twelve
 *     16-bit uniforms (three 64-bit outputs, four 16-bit lanes each),
 *     z = (float)(2S - 786420) * (sigma * 2^-17).  2S - 786420 is an exact
 *     integer below 2^24 and the factor sigma * 2^-17 is an exact power-of-two
 *     scaling of sigma, so z is one IEEE fp32 multiply and is bit-identical on
 *     any IEEE machine.  Var(S) = 12 * (2^32 - 1) / 12 ~ 2^32, so z has
 *     standard deviation sigma (to 1 part in 2^33) and support +-6 sigma.
 *
 * Plain C99, static inline, no globals: includable from C and (under clang's
 * host-device pragma) from HIP device code.
 */
#ifndef SYNTH_H
#define SYNTH_H

#include <stdint.h>

#define SYNTH_GOLDEN 0x9E3779B97F4A7C15ull

/* tensor ids of the stream key */
enum {
    SYNTH_T_ROUTER_W = 1,
    SYNTH_T_ROUTER_B = 2,
    SYNTH_T_X = 3,
    SYNTH_T_GATE = 4,
    SYNTH_T_UP = 5,
    SYNTH_T_DOWN = 6,
    SYNTH_T_PERM = 7
};

static inline uint64_t synth_mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* Stream key for (seed, layer, tensor, expert). The shared expert of a layer
 * uses expert index n_experts + s. */
static inline uint64_t synth_key(uint64_t seed, uint32_t layer, uint32_t tensor,
                                 uint32_t expert)
{
    uint64_t h = synth_mix64(seed + SYNTH_GOLDEN);
    h = synth_mix64(h ^ ((uint64_t)layer + 0x1000003ull));
    h = synth_mix64(h ^ ((uint64_t)tensor << 32 ^ 0xA5A5A5A5ull));
    h = synth_mix64(h ^ ((uint64_t)expert + 0x2000005ull));
    return h;
}

/* Output number idx (0-based) of the SplitMix64 stream seeded with key. */
static inline uint64_t synth_u64(uint64_t key, uint64_t idx)
{
    return synth_mix64(key + (idx + 1ull) * SYNTH_GOLDEN);
}

/* Element idx of a ~N(0, sigma) stream (Irwin-Hall(12) approximation). */
static inline float synth_gauss(uint64_t key, uint64_t idx, float sigma)
{
    uint64_t a = synth_u64(key, 3ull * idx + 0ull);
    uint64_t b = synth_u64(key, 3ull * idx + 1ull);
    uint64_t c = synth_u64(key, 3ull * idx + 2ull);
    uint32_t s = 0;
    for (int j = 0; j < 4; ++j) {
        s += (uint32_t)((a >> (16 * j)) & 0xFFFFu);
        s += (uint32_t)((b >> (16 * j)) & 0xFFFFu);
        s += (uint32_t)((c >> (16 * j)) & 0xFFFFu);
    }
    int32_t centred = 2 * (int32_t)s - 786420;
    float factor = sigma * 0x1p-17f;
    return (float)centred * factor;
}

#endif /* SYNTH_H */
