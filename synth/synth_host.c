/*
 * Seeded synthetic tensors on the host (plain C, OpenMP).
 *
 * Test and benchmark infrastructure: this file produces inputs, it holds none
 * of the MoE layer's arithmetic.  The same element generator is implemented a
 * second time for the GPU in synth_gpu.hip; both follow the definition below
 * and must give bit-identical values (checked by the test suite).
 *
 * Element generator (counter based, one 64-bit draw per element):
 *   z_i   = mix64(key + (i + 1) * GAMMA)            (SplitMix64, Steele, Lea and
 *                                                    Flood, OOPSLA 2014; the
 *                                                    finaliser is Stafford's
 *                                                    "Mix13" variant)
 *   s_i   = sum of the four 16-bit fields of z_i     (Irwin-Hall sum, n = 4)
 *   v_i   = float(s_i - 131070) * c                  (one fp32 multiply)
 * where c = std / sqrt(4 * (65536^2 - 1) / 12) rounded to fp32 by the caller.
 * v_i has mean 0 and standard deviation std (up to the rounding of c); it is a
 * bounded (+-3.46 std) approximation of a normal variate.  bf16 output is the
 * round-to-nearest-even of v_i to the upper 16 bits.
 */
#include <stdint.h>
#include <stddef.h>

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline float synth_value(uint64_t key, uint64_t i, float c) {
    uint64_t z = mix64(key + (i + 1) * SYNTH_GAMMA);
    int32_t s = (int32_t)(z & 0xFFFFu) + (int32_t)((z >> 16) & 0xFFFFu) +
                (int32_t)((z >> 32) & 0xFFFFu) + (int32_t)(z >> 48);
    return (float)(s - 131070) * c;
}

static inline uint16_t f32_to_bf16_rne(float f) {
    union { float f; uint32_t u; } b;
    b.f = f;
    uint32_t u = b.u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* out[j] = value of element (first + j), j < n, as fp32. */
void synth_fill_f32(uint64_t key, uint64_t first, uint64_t n, float c, float* out) {
    long long nn = (long long)n;
#pragma omp parallel for schedule(static)
    for (long long j = 0; j < nn; ++j) out[j] = synth_value(key, first + (uint64_t)j, c);
}

/* out[j] = bf16 bits of element (first + j), j < n. */
void synth_fill_bf16(uint64_t key, uint64_t first, uint64_t n, float c, uint16_t* out) {
    long long nn = (long long)n;
#pragma omp parallel for schedule(static)
    for (long long j = 0; j < nn; ++j) out[j] = f32_to_bf16_rne(synth_value(key, first + (uint64_t)j, c));
}

/* Gather form: out[j] = value of element idx[j] (used to sample large tensors). */
void synth_gather_f32(uint64_t key, const uint64_t* idx, uint64_t n, float c, float* out) {
    long long nn = (long long)n;
#pragma omp parallel for schedule(static)
    for (long long j = 0; j < nn; ++j) out[j] = synth_value(key, idx[j], c);
}
