/*
 * synth.c -- seeded, counter-based synthetic activations for Lightning
 * Attention runs.  This file holds no attention arithmetic: it only turns
 * (seed, tensor, batch, head, token, feature) into a number, so that the
 * oracle and the GPU path can be fed the very same bytes, and so that any
 * slice of a million-token input can be regenerated on its own.
 *
 * Recipe (the pages give the workload only as "activations of a 64-head,
 * d=128 lightning layer"; this recipe is our stand-in for them):
 *   stream key   K = mix(mix(mix(mix(seed) + tensor) + b) + h)
 *   raw draw n   R(n) = mix(K + (n + 1) * GOLDEN)           (SplitMix64,
 *                Steele, Lea & Flood, "Fast splittable pseudorandom number
 *                generators", OOPSLA 2014: state_n = K + n*GOLDEN, output =
 *                mix(state_n + GOLDEN))
 *   element e = t*d + i of the stream, pair p = e/2:
 *                u1 = (R(2p) >> 11 + 1) * 2^-53 in (0,1]
 *                u2 = (R(2p+1) >> 11) * 2^-53 in [0,1)
 *                z  = sqrt(-2 ln u1) * (cos | sin)(2 pi u2)   (Box & Muller 1958;
 *                     even e takes cos, odd e takes sin)
 *   tensor 0 (Q), 1 (K): x = z / (1 + exp(-z))   (SiLU), computed in double
 *   tensor 2 (V):        x = z
 *   x is rounded once to float32; the bf16 form is float32 -> bf16 with
 *   round-to-nearest-even.
 */
#include <math.h>
#include <stdint.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t tensor, uint64_t b, uint64_t h)
{
    return mix64(mix64(mix64(mix64(seed) + tensor) + b) + h);
}

static inline uint64_t draw(uint64_t key, uint64_t n)
{
    return mix64(key + (n + 1) * GOLDEN);
}

/* Values of elements 2p and 2p+1 of the stream (Box-Muller pair), after SiLU for Q/K. */
static inline void element_pair(uint64_t key, int tensor, uint64_t p, double* z0, double* z1)
{
    const double u1 = (double)((draw(key, 2 * p) >> 11) + 1) * 0x1.0p-53;
    const double u2 = (double)(draw(key, 2 * p + 1) >> 11) * 0x1.0p-53;
    const double r = sqrt(-2.0 * log(u1));
    const double a = 6.283185307179586476925286766559 * u2;
    double c = r * cos(a), s = r * sin(a);
    if (tensor != 2) {
        c = c / (1.0 + exp(-c));
        s = s / (1.0 + exp(-s));
    }
    *z0 = c;
    *z1 = s;
}

static inline uint16_t f32_to_bf16_rne(float f)
{
    union { float f; uint32_t u; } c;
    c.f = f;
    uint32_t u = c.u;
    if ((u & 0x7F800000u) == 0x7F800000u) /* inf / nan: keep, quiet nan */
        return (uint16_t)((u >> 16) | ((u & 0x007FFFFFu) ? 0x40u : 0u));
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/*
 * Fill out[nb][nh][nt][d] with the tensor's values at batch b0.., head h0..,
 * token t0.. (all features).  as_bf16 != 0 writes uint16 bf16 bits, else
 * float32.  Returns 0, or -1 on bad arguments (odd d, negative sizes).
 */
int synth_fill(void* out, int as_bf16, uint64_t seed, int tensor,
               int64_t b0, int64_t nb, int64_t h0, int64_t nh,
               int64_t t0, int64_t nt, int64_t d)
{
    if (!out || d <= 0 || (d & 1) || nb < 0 || nh < 0 || nt < 0 || t0 < 0 || b0 < 0 || h0 < 0)
        return -1;
    if (tensor < 0 || tensor > 2) return -1;
    const int64_t rows = nb * nh * nt;
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < rows; ++row) {
        const int64_t t = row % nt;
        const int64_t h = (row / nt) % nh;
        const int64_t b = row / (nt * nh);
        const uint64_t key = stream_key(seed, (uint64_t)tensor, (uint64_t)(b0 + b), (uint64_t)(h0 + h));
        const uint64_t e0 = (uint64_t)(t0 + t) * (uint64_t)d;
        for (int64_t i = 0; i < d; i += 2) {
            double z0, z1;
            element_pair(key, tensor, (e0 + (uint64_t)i) >> 1, &z0, &z1);
            if (as_bf16) {
                uint16_t* o = (uint16_t*)out + row * d + i;
                o[0] = f32_to_bf16_rne((float)z0);
                o[1] = f32_to_bf16_rne((float)z1);
            } else {
                float* o = (float*)out + row * d + i;
                o[0] = (float)z0;
                o[1] = (float)z1;
            }
        }
    }
    return 0;
}

/* Raw draw, exported so tests can check the SplitMix64 stream against its definition. */
uint64_t synth_draw(uint64_t seed, int tensor, int64_t b, int64_t h, uint64_t n)
{
    return draw(stream_key(seed, (uint64_t)tensor, (uint64_t)b, (uint64_t)h), n);
}

/* The SplitMix64 output for a given state (exported for a published-value check). */
uint64_t synth_mix64_next(uint64_t state)
{
    return mix64(state + GOLDEN);
}
