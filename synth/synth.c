/*
 * Seeded synthetic input generators shared by the oracle-side tests and the
 * GPU-side tests/benchmark.  Nothing of the quantized-MoE computation lives
 * here: only random bits, uniform and normal draws, and the rounding of a
 * drawn fp64 value to the storage type an input is kept in (bf16 or fp32).
 *
 * Random source: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used as a counter-based
 * generator: draw n of a stream whose state is `key` is the SplitMix64
 * finaliser applied to key + (n+1)*gamma, which is exactly the (n+1)-th
 * output of SplitMix64 seeded with `key`.  Any element of any stream can be
 * produced independently, so the tensors can be filled in parallel and a
 * consumer can regenerate just the slice it needs.
 *
 * Normals: Box-Muller in fp64 (Box and Muller, 1958) on the draw pair
 * (2j, 2j+1); element 2j takes the cosine branch, element 2j+1 the sine
 * branch.  u1 = ((d0 >> 11) + 1) * 2^-53 lies in (0, 1], u2 = (d1 >> 11) * 2^-53
 * in [0, 1).
 */
#include <stdint.h>
#include <string.h>
#include <math.h>

#define SM_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t sm_draw(uint64_t key, uint64_t n) {
    return sm_mix(key + (n + 1) * SM_GAMMA);
}

/* Stream key for the tuple (seed, a, b, c, d, e): a hash chain of the finaliser. */
uint64_t synth_key(uint64_t seed, uint64_t a, uint64_t b, uint64_t c, uint64_t d, uint64_t e) {
    uint64_t s = sm_mix(seed + SM_GAMMA);
    s = sm_mix(s ^ sm_mix(a + SM_GAMMA));
    s = sm_mix(s ^ sm_mix(b + 2 * SM_GAMMA));
    s = sm_mix(s ^ sm_mix(c + 3 * SM_GAMMA));
    s = sm_mix(s ^ sm_mix(d + 4 * SM_GAMMA));
    s = sm_mix(s ^ sm_mix(e + 5 * SM_GAMMA));
    return s;
}

uint64_t synth_draw(uint64_t key, uint64_t n) { return sm_draw(key, n); }

/* out[i] = byte ((start+i) mod 8) of draw (start+i)/8, little-endian: uniform bytes. */
void synth_bytes(uint64_t key, uint64_t start, uint64_t count, uint8_t* out) {
    uint64_t i = 0;
    for (; i < count && ((start + i) & 7); ++i) {
        uint64_t j = start + i;
        out[i] = (uint8_t)(sm_draw(key, j >> 3) >> (8 * (j & 7)));
    }
    for (; i + 8 <= count; i += 8) {
        uint64_t d = sm_draw(key, (start + i) >> 3);
        for (int b = 0; b < 8; ++b) out[i + b] = (uint8_t)(d >> (8 * b));
    }
    for (; i < count; ++i) {
        uint64_t j = start + i;
        out[i] = (uint8_t)(sm_draw(key, j >> 3) >> (8 * (j & 7)));
    }
}

/* out[i] = table[floor(draw(start+i) * ntable / 2^64)]: uniform choice from a table. */
void synth_choice_bytes(uint64_t key, uint64_t start, uint64_t count,
                        const uint8_t* table, uint32_t ntable, uint8_t* out) {
    for (uint64_t i = 0; i < count; ++i) {
        unsigned __int128 p = (unsigned __int128)sm_draw(key, start + i) * ntable;
        out[i] = table[(uint32_t)(p >> 64)];
    }
}

static double sm_normal(uint64_t key, uint64_t i) {
    uint64_t j = i >> 1;
    uint64_t d0 = sm_draw(key, 2 * j), d1 = sm_draw(key, 2 * j + 1);
    double u1 = (double)((d0 >> 11) + 1) * 0x1.0p-53;
    double u2 = (double)(d1 >> 11) * 0x1.0p-53;
    double r = sqrt(-2.0 * log(u1));
    double a = 6.283185307179586476925286766559 * u2;
    return (i & 1) ? r * sin(a) : r * cos(a);
}

static double sm_uniform(uint64_t key, uint64_t i) {
    return (double)(sm_draw(key, i) >> 11) * 0x1.0p-53;
}

/* fp64 -> bf16 bits, one round-to-nearest-even to 8 significant bits.
 * Valid for the normal bf16 range, which is all these generators produce. */
static uint16_t f64_to_bf16_rne(double v) {
    if (v == 0.0) return signbit(v) ? 0x8000u : 0u;
    int e;
    double m = frexp(v, &e);
    double r = ldexp(nearbyint(ldexp(m, 8)), e - 8);
    float f = (float)r; /* exact: r has 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* bf16 values: v = mu + sigma*n, or |sigma*n| + mu when fold != 0. */
void synth_bf16_normal(uint64_t key, uint64_t start, uint64_t count,
                       double mu, double sigma, int fold, uint16_t* out) {
    for (uint64_t i = 0; i < count; ++i) {
        double n = sigma * sm_normal(key, start + i);
        if (fold) n = fabs(n);
        out[i] = f64_to_bf16_rne(mu + n);
    }
}

/* fp32 values: v = mu + sigma*n rounded once to fp32. */
void synth_f32_normal(uint64_t key, uint64_t start, uint64_t count,
                      double mu, double sigma, float* out) {
    for (uint64_t i = 0; i < count; ++i) out[i] = (float)(mu + sigma * sm_normal(key, start + i));
}

/* fp32 values: v = lo + (hi - lo)*u, u uniform in [0, 1), rounded once to fp32. */
void synth_f32_uniform(uint64_t key, uint64_t start, uint64_t count,
                       double lo, double hi, float* out) {
    for (uint64_t i = 0; i < count; ++i) out[i] = (float)(lo + (hi - lo) * sm_uniform(key, start + i));
}

/* fp64 normals (unrounded), for statistical checks of the generator itself. */
void synth_f64_normal(uint64_t key, uint64_t start, uint64_t count, double* out) {
    for (uint64_t i = 0; i < count; ++i) out[i] = sm_normal(key, start + i);
}
