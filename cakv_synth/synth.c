/*
 * synth.c -- seeded, counter-based synthetic inputs shared by the tests, the
 * benchmark and the smoke check. It holds no attention arithmetic: it only
 * turns (seed, tensor id, element index) into a value.
 *
 * Generator: SplitMix64 (G. L. Steele, D. Lea, C. H. Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014). For a stream
 * seeded with key K, output n (n = 0, 1, ...) is mix(K + (n + 1) * GAMMA),
 * GAMMA = 0x9E3779B97F4A7C15, mix = the two xor-shift-multiply rounds of the
 * paper's finaliser. Random access by n lets any slice of a tensor be made
 * alone and come out bit-identical to the same slice of the whole tensor.
 * The stream key for (seed, tensor) is mix(seed * 2^16 + tensor).
 *
 * Distributions (the value is computed in double, then rounded once):
 *   normal:  Box-Muller, z = sqrt(-2 ln u1) cos(2 pi u2) with u1 in (0, 1]
 *            from the top 24 bits and u2 in [0, 1) from the next 24 bits;
 *   uniform: u in [-1, 1) as 2 * (top 24 bits) / 2^24 - 1.
 * Each value is multiplied by `mul` times a per-head factor (head = (n / D)
 * mod H for a [.., H, D] tensor) in fp32, then stored as fp32 or rounded to
 * bfloat16 with round-to-nearest-even.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t synth_stream_key(uint64_t seed, uint64_t tensor) {
    return mix64(seed * 65536ULL + tensor + GAMMA);
}

uint64_t synth_raw(uint64_t key, uint64_t n) { return mix64(key + (n + 1) * GAMMA); }

static uint16_t f32_to_bf16_rne(float f) {
    uint32_t x;
    memcpy(&x, &f, sizeof x);
    if ((x & 0x7F800000u) == 0x7F800000u) /* inf / nan: keep, quiet nan */
        return (uint16_t)((x >> 16) | ((x & 0xFFFFu) ? 0x40u : 0u));
    uint32_t lsb = (x >> 16) & 1u;
    x += 0x7FFFu + lsb;
    return (uint16_t)(x >> 16);
}

static float draw(uint64_t key, uint64_t n, int dist) {
    const uint64_t r = synth_raw(key, n);
    const double two24 = 16777216.0;
    if (dist == 0) {
        const double u1 = ((double)(r >> 40) + 1.0) / two24;          /* (0,1] */
        const double u2 = (double)((r >> 16) & 0xFFFFFFULL) / two24;  /* [0,1) */
        return (float)(sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2));
    }
    return (float)(2.0 * ((double)(r >> 40) / two24) - 1.0);
}

/*
 * Fill out[0..count) with elements n0 .. n0+count-1 of the stream
 * (seed, tensor). dtype 0 = fp32, 1 = bf16 (uint16 bits). dist 0 = N(0,1),
 * 1 = U[-1,1). head_mul (nullable, length H) scales head (n / D) % H.
 */
int synth_fill(void* out, int64_t count, int dtype, int dist, uint64_t seed,
               uint64_t tensor, int64_t n0, float mul, const float* head_mul,
               int64_t H, int64_t D) {
    if (count < 0 || n0 < 0 || (dtype != 0 && dtype != 1) || (dist != 0 && dist != 1))
        return -1;
    if (head_mul && (H <= 0 || D <= 0)) return -1;
    const uint64_t key = synth_stream_key(seed, tensor);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        const int64_t n = n0 + i;
        float x = draw(key, (uint64_t)n, dist) * mul;
        if (head_mul) x *= head_mul[(n / D) % H];
        if (dtype == 0)
            ((float*)out)[i] = x;
        else
            ((uint16_t*)out)[i] = f32_to_bf16_rne(x);
    }
    return 0;
}

/* bf16 bits -> fp32 (exact), for host-side inspection of generated data */
void synth_bf16_to_f32(const uint16_t* in, float* out, int64_t count) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        uint32_t x = ((uint32_t)in[i]) << 16;
        memcpy(&out[i], &x, sizeof x);
    }
}
