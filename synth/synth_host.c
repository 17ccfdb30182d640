/*
 * synth_host.c -- host (CPU) fills for the seeded synthetic inputs defined in
 * synth.h.  Input generation only: nothing here quantises, routes or
 * computes any part of the MoE layer.
 *
 * The Zipf hot-expert term of the router bias is an input recipe (skewed
 * routing as a stand-in for the skew of a trained router): for a seeded
 * Fisher-Yates permutation p of the experts, expert p[r] (rank r+1) gets
 * c * (r+1)^(-s) added to its N(0, sigma_b) bias, evaluated in double on
 * the host and rounded once to fp32, so every consumer sees the same bytes.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include "synth.h"

void synth_fill_gauss(float *out, uint64_t n, uint64_t key, float sigma, uint64_t idx0)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i)
        out[i] = synth_gauss(key, idx0 + (uint64_t)i, sigma);
}

uint64_t synth_key_c(uint64_t seed, uint32_t layer, uint32_t tensor, uint32_t expert)
{
    return synth_key(seed, layer, tensor, expert);
}

uint64_t synth_u64_c(uint64_t key, uint64_t idx) { return synth_u64(key, idx); }

float synth_gauss_c(uint64_t key, uint64_t idx, float sigma)
{
    return synth_gauss(key, idx, sigma);
}

/* Seeded Fisher-Yates permutation of 0..n-1 (perm[r] = expert of rank r+1). */
void synth_permutation(int32_t *perm, int n, uint64_t key)
{
    for (int i = 0; i < n; ++i) perm[i] = i;
    for (int i = n - 1; i > 0; --i) {
        int j = (int)(synth_u64(key, (uint64_t)i) % (uint64_t)(i + 1));
        int32_t t = perm[i];
        perm[i] = perm[j];
        perm[j] = t;
    }
}

/* bias[e] = N(0, sigma_b) draw + Zipf(s) hot term of weight c (c = 0: none). */
void synth_router_bias(float *bias, int n_experts, uint64_t seed, uint32_t layer,
                       float sigma_b, double zipf_c, double zipf_s)
{
    uint64_t kb = synth_key(seed, layer, SYNTH_T_ROUTER_B, 0);
    double *acc = (double *)malloc(sizeof(double) * (size_t)n_experts);
    for (int e = 0; e < n_experts; ++e) acc[e] = (double)synth_gauss(kb, (uint64_t)e, sigma_b);
    if (zipf_c != 0.0) {
        int32_t *perm = (int32_t *)malloc(sizeof(int32_t) * (size_t)n_experts);
        synth_permutation(perm, n_experts, synth_key(seed, layer, SYNTH_T_PERM, 0));
        for (int r = 0; r < n_experts; ++r)
            acc[perm[r]] += zipf_c * pow((double)(r + 1), -zipf_s);
        free(perm);
    }
    for (int e = 0; e < n_experts; ++e) bias[e] = (float)acc[e];
    free(acc);
}
