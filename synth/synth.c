/*
 * synth.c - seeded, counter-based synthetic inputs for the MoE expert layer.
 *
 * This module only draws numbers. It holds none of the layer's arithmetic and
 * is shared by both sides of every parity check (the CPU oracle and the HIP
 * library), so both see byte-identical inputs.
 *
 * Definition (the one place it is stated):
 *   value i of tensor tau under seed S is
 *     h1 = splitmix64(S ^ (tau << 40) ^ (2i)),  h2 = splitmix64(S ^ (tau << 40) ^ (2i+1))
 *     u1 = ((h1 >> 11) + 1) * 2^-53   in (0, 1]
 *     u2 =  (h2 >> 11)      * 2^-53   in [0, 1)
 *     z  = sqrt(-2 ln u1) * cos(2 pi u2)          (Box-Muller, cosine branch)
 *     v  = (float)(sigma * z)                     (computed in double, rounded once)
 *   and for bf16 storage v is rounded again, float -> bf16, to nearest-even.
 * splitmix64 is the mixer of Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators" (OOPSLA 2014), with Vigna's constants.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC synth.c -o libsynth.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t splitmix64(uint64_t z)
{
    z += 0x9e3779b97f4a7c15ULL;
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

static inline double synth_z(uint64_t seed, uint32_t tensor, uint64_t i)
{
    const uint64_t base = seed ^ ((uint64_t)tensor << 40);
    const uint64_t h1 = splitmix64(base ^ (2 * i));
    const uint64_t h2 = splitmix64(base ^ (2 * i + 1));
    const double u1 = (double)((h1 >> 11) + 1) * 0x1.0p-53;
    const double u2 = (double)(h2 >> 11) * 0x1.0p-53;
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
}

/* float -> bf16 bits, round to nearest, ties to even (finite inputs). */
static inline uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u) /* inf / nan: truncate, keep a nan a nan */
        return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

void synth_normal_f32(uint64_t seed, uint32_t tensor, double sigma, float *out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = (float)(sigma * synth_z(seed, tensor, (uint64_t)i));
}

void synth_normal_bf16(uint64_t seed, uint32_t tensor, double sigma, uint16_t *out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = f32_to_bf16_rne((float)(sigma * synth_z(seed, tensor, (uint64_t)i)));
}

void synth_f32_to_bf16(const float *in, uint16_t *out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = f32_to_bf16_rne(in[i]);
}

/* Zipf-like per-expert bias for the skewed-routing workload:
 * logits[t, e] += (float)(c * ln(1 / (e + 1))), added in fp32. */
void synth_add_rank_bias(float *logits, int64_t T, int64_t E, double c)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t e = 0; e < E; ++e)
            logits[t * E + e] += (float)(c * log(1.0 / (double)(e + 1)));
}
