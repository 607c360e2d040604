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

/*
 * Weights stored in 8 bits (an input format: how a weight tensor is handed to an FP8
 * layer; no layer arithmetic).  OCP FP8 E4M3 codes (sign, 4 exponent bits with bias 7,
 * 3 mantissa bits; exponent 0 is subnormal, m * 2^-9; no infinities; S.1111.111 is NaN;
 * largest finite 448) with one E8M0 scale byte s per 32 consecutive elements of a row,
 * meaning a factor 2^(s - 127).  Per block: s = 127 + ceil(log2(amax / 448)) (127 for an
 * all-zero block), clamped to [1, 254]; each element w becomes the E4M3 value nearest to
 * w / 2^(s - 127), ties to even mantissa.
 */
static uint8_t e4m3_nearest(double x) {
    const uint8_t sign = x < 0 ? 0x80 : 0;
    const double a = fabs(x);
    if (a == 0.0) return sign;
    if (a < 0.015625) {                       /* below 2^-6: the subnormal grid m * 2^-9 */
        const double m = nearbyint(a * 512.0);
        return m >= 8.0 ? (uint8_t)(sign | 0x08) : (uint8_t)(sign | (uint8_t)m);
    }
    int e;
    const double f = frexp(a, &e);            /* a = f * 2^e, f in [0.5, 1) */
    int E = e + 6;                            /* a = (1 + m/8) * 2^(E - 7) */
    double m = nearbyint((2.0 * f - 1.0) * 8.0);
    if (m == 8.0) { m = 0.0; E += 1; }
    if (E > 15 || (E == 15 && m > 6.0)) { E = 15; m = 6.0; }   /* 448; the block scale keeps |x| <= 448 */
    return (uint8_t)(sign | (uint8_t)(E << 3) | (uint8_t)m);
}

static double bf16_bits_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* w [rows, cols] bf16 bit patterns (cols % 32 == 0) -> codes [rows, cols], scales [rows, cols/32] */
void synth_quant_e4m3(const uint16_t* w, uint64_t rows, uint64_t cols, uint8_t* codes, uint8_t* scales) {
    const int64_t nblk = (int64_t)(rows * (cols / 32));
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nblk; ++b) {
        const uint16_t* src = w + (uint64_t)b * 32;
        double amax = 0.0;
        for (int i = 0; i < 32; ++i) {
            const double v = fabs(bf16_bits_to_double(src[i]));
            if (v > amax) amax = v;
        }
        int s = 127;
        if (amax > 0.0) {
            int e;
            const double f = frexp(amax / 448.0, &e);
            s = 127 + (f == 0.5 ? e - 1 : e);
            if (s < 1) s = 1;
            if (s > 254) s = 254;
        }
        scales[b] = (uint8_t)s;
        const double inv = ldexp(1.0, 127 - s);
        for (int i = 0; i < 32; ++i) codes[(uint64_t)b * 32 + i] = e4m3_nearest(bf16_bits_to_double(src[i]) * inv);
    }
}

/*
 * Weights stored in 4 bits (MXFP4; an input format, no layer arithmetic).  OCP FP4 E2M1
 * codes (sign, 2 exponent bits with bias 1, 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2,
 * 3, 4, 6; no infinities or NaN), two per byte with the even element in bits 0..3, and one
 * E8M0 scale byte s per 32 consecutive elements of a row.  Per block: s = 127 +
 * ceil(log2(amax / 6)) (127 for an all-zero block), clamped to [1, 254]; each element w
 * becomes the E2M1 value nearest to w / 2^(s - 127), ties to the even code.
 */
static uint8_t e2m1_nearest(double x) {
    static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    const uint8_t sign = x < 0 ? 8 : 0;
    const double a = fabs(x);
    int best = 0;
    for (int c = 1; c < 8; ++c) {
        const double d = fabs(a - mag[c]), db = fabs(a - mag[best]);
        if (d < db || (d == db && (c & 1) == 0)) best = c;
    }
    return (uint8_t)(sign | best);
}

/* w [rows, cols] bf16 bit patterns (cols % 32 == 0) -> codes [rows, cols/2], scales [rows, cols/32] */
void synth_quant_e2m1(const uint16_t* w, uint64_t rows, uint64_t cols, uint8_t* codes, uint8_t* scales) {
    const int64_t nblk = (int64_t)(rows * (cols / 32));
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nblk; ++b) {
        const uint16_t* src = w + (uint64_t)b * 32;
        double amax = 0.0;
        for (int i = 0; i < 32; ++i) {
            const double v = fabs(bf16_bits_to_double(src[i]));
            if (v > amax) amax = v;
        }
        int s = 127;
        if (amax > 0.0) {
            int e;
            const double f = frexp(amax / 6.0, &e);
            s = 127 + (f == 0.5 ? e - 1 : e);
            if (s < 1) s = 1;
            if (s > 254) s = 254;
        }
        scales[b] = (uint8_t)s;
        const double inv = ldexp(1.0, 127 - s);
        for (int i = 0; i < 32; i += 2) {
            const uint8_t lo = e2m1_nearest(bf16_bits_to_double(src[i]) * inv);
            const uint8_t hi = e2m1_nearest(bf16_bits_to_double(src[i + 1]) * inv);
            codes[(uint64_t)b * 16 + i / 2] = (uint8_t)(lo | (hi << 4));
        }
    }
}
