/*
 * synth.c -- seeded, counter-based generator of synthetic inputs.
 *
 * Test and benchmark infrastructure shared by the GPU library's tests and the
 * CPU oracle.  It holds none of the MoE layer's arithmetic: it only draws
 * numbers.  Every value is a pure function of (seed, tensor_id, index), so any
 * slice of any tensor can be regenerated independently and in parallel.
 *
 * Generator: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used in counter mode.  The
 * stream key is derived from (seed, tensor_id) by two finaliser rounds; the
 * i-th raw 64-bit word of a stream is mix64(key + (i + 1) * GAMMA).
 *
 *   uniform(i)  = ((word(i) >> 11) + 0.5) * 2^-53            in (0, 1)
 *   normal pair j (elements 2j, 2j+1), Box-Muller (Box & Muller 1958):
 *       r = sqrt(-2 ln uniform(2j)),  th = 2 pi uniform(2j+1)
 *       z(2j) = r cos th,  z(2j+1) = r sin th                 (in double)
 *   a value with standard deviation sd and mean mu is (float)(mu + sd * z),
 *   bf16 values are the round-to-nearest-even of that float.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t tensor_id) {
    return mix64(mix64(seed + GAMMA) ^ (tensor_id * 0xD1B54A32D192ED03ULL + 1ULL));
}

static inline uint64_t word_at(uint64_t key, uint64_t i) { return mix64(key + (i + 1ULL) * GAMMA); }

static inline double unit_open(uint64_t w) { return ((double)(w >> 11) + 0.5) * (1.0 / 9007199254740992.0); }

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t b;
    memcpy(&b, &f, 4);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

/* Fill out[k] = f(value number first + k), k < n, one Box-Muller pair per step. */
#define NORMAL_FILL(STORE)                                                                 \
    uint64_t key = stream_key(seed, tid);                                                  \
    uint64_t lo = first, hi = first + n;                                                   \
    int64_t p0 = (int64_t)(lo >> 1), p1 = (int64_t)((hi + 1) >> 1);                        \
    _Pragma("omp parallel for schedule(static)")                                           \
    for (int64_t p = p0; p < p1; ++p) {                                                    \
        double u1 = unit_open(word_at(key, 2 * (uint64_t)p));                              \
        double u2 = unit_open(word_at(key, 2 * (uint64_t)p + 1));                          \
        double r = sqrt(-2.0 * log(u1)), th = 6.283185307179586476925 * u2;                \
        double z[2] = {r * cos(th), r * sin(th)};                                          \
        for (int q = 0; q < 2; ++q) {                                                      \
            uint64_t i = 2 * (uint64_t)p + (uint64_t)q;                                    \
            if (i >= lo && i < hi) { uint64_t k = i - lo; STORE; }                         \
        }                                                                                  \
    }

void synth_normal_f32(uint64_t seed, uint64_t tid, uint64_t first, uint64_t n, double mean, double sd,
                      float* out) {
    NORMAL_FILL(out[k] = (float)(mean + sd * z[q]))
}

void synth_normal_bf16(uint64_t seed, uint64_t tid, uint64_t first, uint64_t n, double mean, double sd,
                       uint16_t* out) {
    NORMAL_FILL(out[k] = f32_to_bf16_rne((float)(mean + sd * z[q])))
}

void synth_uniform_f32(uint64_t seed, uint64_t tid, uint64_t first, uint64_t n, double lo, double hi,
                       float* out) {
    uint64_t key = stream_key(seed, tid);
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < (int64_t)n; ++k)
        out[k] = (float)(lo + (hi - lo) * unit_open(word_at(key, first + (uint64_t)k)));
}

/* Raw 64-bit words (used for seeded permutations and subsets on the host). */
void synth_words(uint64_t seed, uint64_t tid, uint64_t first, uint64_t n, uint64_t* out) {
    uint64_t key = stream_key(seed, tid);
    for (uint64_t k = 0; k < n; ++k) out[k] = word_at(key, first + k);
}
