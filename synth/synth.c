/*
 * Seeded synthetic inputs for the draft-head sampler, the accept-rate
 * reduction and the prefix scheduler.
 *
 * This file draws random numbers and nothing else: it holds none of the
 * method's arithmetic (no bias, no softmax, no argmax, no scheduling).  Both
 * the GPU path and the CPU oracle read the buffers it fills, so their parity
 * never depends on it.
 *
 * Generator: a counter-based SplitMix64 stream (Steele, Lea & Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014; finaliser
 * constants as in Vigna's public-domain splitmix64.c).  Element i of the
 * stream with key K is mix64(K + (i + 1) * 0x9E3779B97F4A7C15), so any
 * element can be drawn independently and in parallel.
 *
 *   uniform on the open interval (0,1):  ((x >> 11) + 0.5) * 2^-53
 *   standard normal: Box-Muller on consecutive uniform pairs;
 *       element 2p uses R cos(theta), element 2p+1 uses R sin(theta), with
 *       R = sqrt(-2 ln u_{2p}), theta = 2 pi u_{2p+1}
 *   Gumbel: -ln(-ln u)
 *
 * Values are formed in double, rounded once to binary32 (round to nearest
 * even), and, for bf16 outputs, rounded again from binary32 to bfloat16
 * (round to nearest even on the upper 16 bits).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* Key of an independent sub-stream: a master seed and a tag (tensor id,
 * anchor id, ...). */
uint64_t synth_key(uint64_t seed, uint64_t tag) {
    return mix64(seed ^ mix64(tag * 0xD1B54A32D192ED03ULL + 0x632BE59BD9B4E019ULL));
}

uint64_t synth_raw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GOLDEN); }

static inline double u01(uint64_t key, uint64_t i) {
    return ((double)(synth_raw(key, i) >> 11) + 0.5) * 0x1p-53;
}

static inline double std_normal(uint64_t key, uint64_t i) {
    uint64_t p = i >> 1;
    double u1 = u01(key, 2 * p), u2 = u01(key, 2 * p + 1);
    double R = sqrt(-2.0 * log(u1));
    double th = 6.283185307179586476925286766559 * u2;
    return (i & 1) ? R * sin(th) : R * cos(th);
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static inline float bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* out[i] = fp32(mean + std * N_i), elements start .. start+n-1 of the stream */
void synth_normal_f32(uint64_t key, uint64_t start, int64_t n, double mean, double sd, float* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = (float)(mean + sd * std_normal(key, start + (uint64_t)i));
}

void synth_normal_bf16(uint64_t key, uint64_t start, int64_t n, double mean, double sd, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = f32_to_bf16_rne((float)(mean + sd * std_normal(key, start + (uint64_t)i)));
}

/* out[i] = bf16(fp32(scale * float(base[i]) + mean + sd * N_i)): a tensor
 * correlated with a bf16 base tensor (the accept-rate target logits). */
void synth_affine_noise_bf16(uint64_t key, uint64_t start, int64_t n, const uint16_t* base, double scale,
                             double mean, double sd, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        double v = scale * (double)bf16_to_f32(base[i]) + mean + sd * std_normal(key, start + (uint64_t)i);
        out[i] = f32_to_bf16_rne((float)v);
    }
}

void synth_affine_noise_f32(uint64_t key, uint64_t start, int64_t n, const float* base, double scale,
                            double mean, double sd, float* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = (float)(scale * (double)base[i] + mean + sd * std_normal(key, start + (uint64_t)i));
}

/* Gumbel(0,1) noise -ln(-ln u), u on the open interval (0,1), fp32. */
void synth_gumbel_f32(uint64_t key, uint64_t start, int64_t n, float* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = (float)(-log(-log(u01(key, start + (uint64_t)i))));
}

/* Uniform integers in [lo, hi) by Lemire's multiply-shift on the top 32 bits
 * (range < 2^32; the bias is below 2^-32 * range). */
void synth_uniform_int(uint64_t key, uint64_t start, int64_t n, int64_t lo, int64_t hi, int32_t* out) {
    uint64_t range = (uint64_t)(hi - lo);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        uint64_t x = synth_raw(key, start + (uint64_t)i) >> 32;
        out[i] = (int32_t)(lo + (int64_t)((x * range) >> 32));
    }
}

/* Uniforms on the open interval (0,1) in double. */
void synth_uniform_f64(uint64_t key, uint64_t start, int64_t n, double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = u01(key, start + (uint64_t)i);
}

/* Confidence values for the scheduler workload: c = fp32(1 / (1 + exp(-z))),
 * z = mean - slope * k + sd * N, k = 1..gamma along the last axis.  The
 * logistic here only shapes the input distribution. */
void synth_logistic_conf(uint64_t key, int64_t B, int64_t gamma, double mean, double sd, double slope,
                         float* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < B * gamma; ++i) {
        int64_t k = i % gamma + 1;
        double z = mean + sd * std_normal(key, (uint64_t)i) - slope * (double)k;
        out[i] = (float)(1.0 / (1.0 + exp(-z)));
    }
}
