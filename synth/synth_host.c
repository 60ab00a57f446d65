/*
 * Seeded synthetic inputs, host side.
 *
 * This module only produces input values. It contains none of the arithmetic
 * of the gradient reduction itself; both the CPU oracle and the GPU path are
 * fed from it. The device twin (synth_dev.hip) implements the same
 * definition and must agree with this file bit for bit.
 *
 * Definition
 * ----------
 * word(key, n)  = mix64(key + (n + 1) * GAMMA): the (n+1)-th output of a
 *                 SplitMix64 generator whose state starts at `key`
 *                 (Steele, Lea and Flood, "Fast splittable pseudorandom
 *                 number generators", OOPSLA 2014; mix64 is the variant-13
 *                 finaliser used by Vigna's splitmix64.c).
 * key(seed, s)  = mix64(seed ^ (s * STREAM_MUL)).
 * Element e of stream s draws the four words n = 4e .. 4e+3.
 *
 * normal(e)     : S = sum of the twelve 16-bit fields of words 4e..4e+2
 *                 (Irwin-Hall with 12 terms, mean 6, variance 1);
 *                 z = (S - 6*65536) / 65536, exact in fp32;
 *                 v = z * sigma, one fp32 multiply (round to nearest even);
 *                 with probability thr / 2^32 (high half of word 4e+3 below
 *                 thr) v is replaced by +mag or -mag (bit 0 of that word
 *                 set = negative);
 *                 the stored bf16 is v rounded to nearest even.
 * uniform_int(e): lo + floor(hi32(word 4e) * (hi - lo + 1) / 2^32).
 */
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL
#define STREAM_MUL 0xD1B54A32D192ED03ULL

static uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static uint64_t key_of(uint64_t seed, uint64_t stream) {
    return mix64(seed ^ (stream * STREAM_MUL));
}

static uint64_t word_at(uint64_t key, uint64_t n) {
    return mix64(key + (n + 1) * GAMMA);
}

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* fp32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN. */
static uint16_t to_bf16(float f) {
    uint32_t u = f32_bits(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static float normal_value(uint64_t key, uint64_t e, float sigma,
                          uint32_t thr, float mag) {
    int32_t s = 0;
    for (int w = 0; w < 3; ++w) {
        uint64_t x = word_at(key, 4 * e + (uint64_t)w);
        s += (int32_t)(x & 0xFFFF) + (int32_t)((x >> 16) & 0xFFFF) +
             (int32_t)((x >> 32) & 0xFFFF) + (int32_t)((x >> 48) & 0xFFFF);
    }
    float z = (float)(s - 6 * 65536) * (1.0f / 65536.0f);
    float v = z * sigma;
    if (thr != 0) {
        uint64_t x = word_at(key, 4 * e + 3);
        if ((uint32_t)(x >> 32) < thr) v = (x & 1u) ? -mag : mag;
    }
    return v;
}

static int32_t uniform_int(uint64_t key, uint64_t e, int32_t lo, int32_t hi) {
    uint64_t m = (uint64_t)((int64_t)hi - (int64_t)lo + 1);
    uint64_t x = word_at(key, 4 * e);
    return (int32_t)((int64_t)lo + (int64_t)(((x >> 32) * m) >> 32));
}

void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t start, uint64_t count,
                       float sigma, uint32_t thr, float mag, uint16_t* out) {
    uint64_t key = key_of(seed, stream);
    for (uint64_t i = 0; i < count; ++i)
        out[i] = to_bf16(normal_value(key, start + i, sigma, thr, mag));
}

void synth_points_normal_bf16(uint64_t seed, const uint64_t* streams, const uint64_t* idx,
                              uint64_t n, float sigma, uint32_t thr, float mag, uint16_t* out) {
    for (uint64_t i = 0; i < n; ++i)
        out[i] = to_bf16(normal_value(key_of(seed, streams[i]), idx[i], sigma, thr, mag));
}

void synth_uniform_int_f32(uint64_t seed, uint64_t stream, uint64_t start, uint64_t count,
                           int32_t lo, int32_t hi, float* out) {
    uint64_t key = key_of(seed, stream);
    for (uint64_t i = 0; i < count; ++i)
        out[i] = (float)uniform_int(key, start + i, lo, hi);
}

void synth_uniform_int_bf16(uint64_t seed, uint64_t stream, uint64_t start, uint64_t count,
                            int32_t lo, int32_t hi, uint16_t* out) {
    uint64_t key = key_of(seed, stream);
    for (uint64_t i = 0; i < count; ++i)
        out[i] = to_bf16((float)uniform_int(key, start + i, lo, hi));
}

/* Raw 64-bit words, for host-side metadata (fragment sizes) and tests. */
void synth_words(uint64_t seed, uint64_t stream, uint64_t start, uint64_t count, uint64_t* out) {
    uint64_t key = key_of(seed, stream);
    for (uint64_t i = 0; i < count; ++i) out[i] = word_at(key, start + i);
}
