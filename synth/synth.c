/*
 * synth.c - seeded synthetic inputs for the ternary bit-plane GEMV workloads.
 *
 * This module only draws random inputs. It holds none of the GEMV's arithmetic:
 * no packing into bit planes, no validation, no select-accumulate, no dequantisation.
 * Both the CPU oracle and the GPU path receive the same arrays from here.
 *
 * Random source: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014), used counter-style: draw i of
 * stream `seed` is mix(seed + (i + 1) * golden_gamma), which is exactly the i-th
 * output of the sequential generator started from state `seed`. Because every
 * element is a pure function of (seed, index), threads may fill disjoint ranges
 * and the result never depends on the thread count.
 *
 * Workload recipe (the pages' model is BitNet b1.58 2B4T; its checkpoint is not
 * used - shapes and zero densities are copied, values are drawn):
 *   - ternary weights i.i.d.: P(0) = z, P(+1) = P(-1) = (1 - z) / 2, row-major;
 *   - activations: v ~ N(0,1) by Box-Muller, then the absmax int8 code
 *     q = rint(127 v / max|v|) (ties to even), scale max|v| / 127;
 *   - per-tensor weight scale ~ U(0.5, 2);
 *   - dense head: W ~ N(0, 0.02) and x ~ N(0, 1), rounded to bfloat16 (RNE).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SM64_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t sm64_at(uint64_t seed, uint64_t i) {
    return sm64_mix(seed + (i + 1) * SM64_GAMMA);
}

/* 53-bit uniform in [0, 1). */
static inline double sm64_u01(uint64_t r) { return (double)(r >> 11) * 0x1.0p-53; }

/* Raw draws [start, start + n) of stream `seed`. */
void synth_u64(uint64_t seed, uint64_t start, int64_t n, uint64_t *out) {
#pragma omp parallel for schedule(static) if (n > (1 << 16))
    for (int64_t i = 0; i < n; ++i) out[i] = sm64_at(seed, start + (uint64_t)i);
}

/* Uniform doubles in [0, 1) from draws [0, n). */
void synth_uniform(uint64_t seed, int64_t n, double *out) {
#pragma omp parallel for schedule(static) if (n > (1 << 16))
    for (int64_t i = 0; i < n; ++i) out[i] = sm64_u01(sm64_at(seed, (uint64_t)i));
}

/* n ternary values in {-1, 0, +1}: u < z -> 0, u < z + (1 - z)/2 -> +1, else -1. */
void synth_trits(uint64_t seed, int64_t n, double p_zero, int8_t *out) {
    const double t_pos = p_zero + 0.5 * (1.0 - p_zero);
#pragma omp parallel for schedule(static) if (n > (1 << 16))
    for (int64_t i = 0; i < n; ++i) {
        double u = sm64_u01(sm64_at(seed, (uint64_t)i));
        out[i] = (int8_t)(u < p_zero ? 0 : (u < t_pos ? 1 : -1));
    }
}

/* n normals (mean, std) as float; element i uses draws 2i and 2i+1 (Box-Muller, cosine branch). */
void synth_normal_f32(uint64_t seed, int64_t n, double mean, double std, float *out) {
    const double two_pi = 6.283185307179586476925286766559;
#pragma omp parallel for schedule(static) if (n > (1 << 14))
    for (int64_t i = 0; i < n; ++i) {
        double u1 = 1.0 - sm64_u01(sm64_at(seed, 2 * (uint64_t)i)); /* (0, 1] */
        double u2 = sm64_u01(sm64_at(seed, 2 * (uint64_t)i + 1));
        double z = sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
        out[i] = (float)(mean + std * z);
    }
}

/*
 * The activation recipe of the workload: int8 codes q = rint((127 * v) / m), m = max|v|,
 * evaluated in float with ties to even and clamped to [-127, 127]; scale = m / 127.
 * m == 0 gives all-zero codes and scale 0.
 */
void synth_absmax_codes(const float *v, int64_t n, int8_t *q, float *scale) {
    float m = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(v[i]);
        if (a > m) m = a;
    }
    if (m == 0.0f) {
        memset(q, 0, (size_t)n);
        *scale = 0.0f;
        return;
    }
    for (int64_t i = 0; i < n; ++i) {
        float t = (127.0f * v[i]) / m;
        float r = rintf(t);
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        q[i] = (int8_t)r;
    }
    *scale = m / 127.0f;
}

/* Per-tensor weight scale, U(0.5, 2): 0.5f + 1.5f * (float)u with u the first draw. */
float synth_weight_scale(uint64_t seed) {
    double u = sm64_u01(sm64_at(seed, 0));
    return 0.5f + 1.5f * (float)u;
}

/* float -> bfloat16 bits, round to nearest even (inputs here are finite). */
void synth_bf16_from_f32(const float *in, int64_t n, uint16_t *out) {
#pragma omp parallel for schedule(static) if (n > (1 << 16))
    for (int64_t i = 0; i < n; ++i) {
        uint32_t b;
        memcpy(&b, &in[i], 4);
        uint32_t lsb = (b >> 16) & 1u;
        out[i] = (uint16_t)((b + 0x7FFFu + lsb) >> 16);
    }
}

/* n bf16 values drawn N(mean, std) and rounded, straight from the stream. */
void synth_normal_bf16(uint64_t seed, int64_t n, double mean, double std, uint16_t *out) {
    const double two_pi = 6.283185307179586476925286766559;
#pragma omp parallel for schedule(static) if (n > (1 << 14))
    for (int64_t i = 0; i < n; ++i) {
        double u1 = 1.0 - sm64_u01(sm64_at(seed, 2 * (uint64_t)i));
        double u2 = sm64_u01(sm64_at(seed, 2 * (uint64_t)i + 1));
        float f = (float)(mean + std * (sqrt(-2.0 * log(u1)) * cos(two_pi * u2)));
        uint32_t b;
        memcpy(&b, &f, 4);
        uint32_t lsb = (b >> 16) & 1u;
        out[i] = (uint16_t)((b + 0x7FFFu + lsb) >> 16);
    }
}
