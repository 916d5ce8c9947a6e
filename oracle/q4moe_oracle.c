/*
 * q4moe oracle: plain fp64 CPU statement of the routed-MoE decode path.
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline timing).
 * Definitions, sources and readings: see q4moe_oracle.h.
 *
 * Every function is the definition written out, loop by loop, with fp64
 * accumulation.  The only concession to speed is an OpenMP pragma on
 * independent outer loops, which does not change any arithmetic.
 */
#include "q4moe_oracle.h"

#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------------- */
/* Element formats                                                         */
/* ---------------------------------------------------------------------- */

/* E2M1 (OCP MX v1.0): sign bit 3, exponent bits 2..1 with bias 1, mantissa
 * bit 0.  Exponent 0 is subnormal: 0.5 * m.  Otherwise 2^(e-1) * (1 + m/2). */
double q4o_e2m1(uint32_t code) {
    uint32_t s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
    double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
    return s ? -mag : mag;
}

/* E4M3FN (OCP OFP8): sign bit 7, exponent bits 6..3 with bias 7, mantissa
 * bits 2..0.  Exponent 0 is subnormal: 2^-6 * m/8.  S.1111.111 is NaN; there
 * are no infinities, so S.1111.110 = 448 is the largest magnitude. */
double q4o_e4m3fn(uint32_t byte) {
    uint32_t s = (byte >> 7) & 1u, e = (byte >> 3) & 15u, m = byte & 7u;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, -6);
    else
        mag = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return s ? -mag : mag;
}

/* Symmetric int4 code: two's complement nibble. */
double q4o_int4(uint32_t code) {
    int v = (int)(code & 15u);
    return (double)(v >= 8 ? v - 16 : v);
}

/* bf16 is the upper half of an IEEE binary32 pattern. */
double q4o_bf16(uint32_t bits) {
    uint32_t u = (bits & 0xFFFFu) << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Element c of a packed row: element 2j is the low nibble of byte j. */
uint32_t q4o_nibble(const uint8_t* row_codes, int64_t c) {
    uint8_t b = row_codes[c / 2];
    return (c % 2 == 0) ? (b & 15u) : (b >> 4);
}

/* ---------------------------------------------------------------------- */
/* Weight dequantization                                                   */
/* ---------------------------------------------------------------------- */

/* Value of element (r, c) of a quantized matrix, as the fp32 number the
 * format defines ([W] Step 1: NVFP4 group 16; [G] What was changed: int4,
 * group 64, symmetric).  NVFP4: e2m1 * e4m3fn is exact in fp64, times the
 * fp32 per-tensor scale is still exact (at most 30 significant bits), and
 * the one cast to float is the single RNE rounding of the definition. */
static double deq_elem(int32_t fmt, int32_t cols, const uint8_t* codes, const void* scales,
                       float g, int64_t r, int64_t c) {
    uint32_t code = q4o_nibble(codes + r * (cols / 2), c);
    if (fmt == Q4O_NVFP4) {
        const uint8_t* s = (const uint8_t*)scales;
        double v = q4o_e2m1(code) * q4o_e4m3fn(s[r * (cols / 16) + c / 16]) * (double)g;
        return (double)(float)v;
    } else {
        const uint16_t* s = (const uint16_t*)scales;
        double v = q4o_int4(code) * q4o_bf16(s[r * (cols / 64) + c / 64]);
        return (double)(float)v;
    }
}

void q4o_dequant(int32_t fmt, int32_t rows, int32_t cols, const uint8_t* codes,
                 const void* scales, float g, float* out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] = (float)deq_elem(fmt, cols, codes, scales, g, r, c);
}

/* One row of a quantized matrix as fp64 values (the fp32 values, widened). */
static void deq_row(int32_t fmt, int32_t cols, const uint8_t* codes, const void* scales,
                    float g, int64_t r, double* out) {
    for (int64_t c = 0; c < cols; ++c) out[c] = deq_elem(fmt, cols, codes, scales, g, r, c);
}

/* Pointers to expert e's up or down matrix inside a bank. */
static void expert_mat(const q4o_bank* b, int32_t e, int up, const uint8_t** codes,
                       const void** scales, float* g, int32_t* rows, int32_t* cols) {
    int32_t blk = (b->fmt == Q4O_NVFP4) ? 16 : 64;
    size_t sbytes = (b->fmt == Q4O_NVFP4) ? 1 : 2;
    int32_t R = up ? b->I : b->H, C = up ? b->H : b->I;
    const uint8_t* cbase = up ? b->up_codes : b->down_codes;
    const uint8_t* sbase = (const uint8_t*)(up ? b->up_scales : b->down_scales);
    *codes = cbase + (size_t)e * R * (C / 2);
    *scales = sbase + (size_t)e * R * (C / blk) * sbytes;
    *g = (b->fmt == Q4O_NVFP4) ? (up ? b->up_g[e] : b->down_g[e]) : 1.0f;
    *rows = R;
    *cols = C;
}

/* ---------------------------------------------------------------------- */
/* Router ([Q] Precision Recipes: router compute in FP32; [G] Left at       */
/* bfloat16: fp32 e_score_correction_bias; [S] The setup: 6 of 128)        */
/* ---------------------------------------------------------------------- */

/* a ranks before b: larger key first, equal keys -> lower index first. */
static int ranks_before(const double* key, int32_t a, int32_t b) {
    return key[a] > key[b] || (key[a] == key[b] && a < b);
}

void q4o_router(int32_t E, int32_t H, int32_t T, int32_t k, const float* wg,
                const float* bias, const uint16_t* x, double* logits, double* scores,
                int32_t* ids, double* w, double* gap) {
    double* key = (double*)malloc(sizeof(double) * (size_t)E);
    char* taken = (char*)malloc((size_t)E);
    for (int32_t t = 0; t < T; ++t) {
        for (int32_t e = 0; e < E; ++e) {
            double l = 0.0;
            for (int32_t c = 0; c < H; ++c)
                l += (double)wg[(size_t)e * H + c] * q4o_bf16(x[(size_t)t * H + c]);
            double s = 1.0 / (1.0 + exp(-l));
            logits[(size_t)t * E + e] = l;
            scores[(size_t)t * E + e] = s;
            key[e] = s + (double)bias[e];
            taken[e] = 0;
        }
        /* Selection by repeated maximum: the i-th pick is the best expert not
         * yet picked, so ids come out in (key desc, index asc) order. */
        double ssum = 0.0;
        for (int32_t i = 0; i < k; ++i) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || ranks_before(key, e, best))) best = e;
            taken[best] = 1;
            ids[(size_t)t * k + i] = best;
            ssum += scores[(size_t)t * E + best];
        }
        for (int32_t i = 0; i < k; ++i)
            w[(size_t)t * k + i] = scores[(size_t)t * E + ids[(size_t)t * k + i]] / ssum;
        if (gap) {
            int32_t next = -1;
            for (int32_t e = 0; e < E; ++e)
                if (!taken[e] && (next < 0 || ranks_before(key, e, next))) next = e;
            gap[t] = (next < 0) ? 0.0 : key[ids[(size_t)t * k + k - 1]] - key[next];
        }
    }
    free(key);
    free(taken);
}

/* ---------------------------------------------------------------------- */
/* W4A16 decode ([W] Step 1 and Interlude; [G] Checkpoint layout)          */
/* ---------------------------------------------------------------------- */

void q4o_moe_w4a16(const q4o_bank* b, int32_t T, int32_t k, const uint16_t* x,
                   const int32_t* ids, const double* w, double* u_tap, double* y) {
    const int32_t H = b->H, I = b->I;
    for (size_t i = 0; i < (size_t)T * H; ++i) y[i] = 0.0;
    for (int32_t t = 0; t < T; ++t) {
        double* xt = (double*)malloc(sizeof(double) * (size_t)H);
        for (int32_t c = 0; c < H; ++c) xt[c] = q4o_bf16(x[(size_t)t * H + c]);
        for (int32_t i = 0; i < k; ++i) {
            int32_t e = ids[(size_t)t * k + i];
            const uint8_t* codes;
            const void* scales;
            float g;
            int32_t R, C;
            double* h = (double*)malloc(sizeof(double) * (size_t)I);
            /* u = W_up x ; h = relu(u)^2 */
            expert_mat(b, e, 1, &codes, &scales, &g, &R, &C);
#pragma omp parallel for schedule(static)
            for (int32_t r = 0; r < I; ++r) {
                double row[C];
                deq_row(b->fmt, C, codes, scales, g, r, row);
                double u = 0.0;
                for (int32_t c = 0; c < C; ++c) u += row[c] * xt[c];
                if (u_tap) u_tap[((size_t)t * k + i) * I + r] = u;
                double rl = u > 0.0 ? u : 0.0;
                h[r] = rl * rl;
            }
            /* y += w_i * W_down h */
            expert_mat(b, e, 0, &codes, &scales, &g, &R, &C);
#pragma omp parallel for schedule(static)
            for (int32_t r = 0; r < H; ++r) {
                double row[C];
                deq_row(b->fmt, C, codes, scales, g, r, row);
                double z = 0.0;
                for (int32_t c = 0; c < C; ++c) z += row[c] * h[c];
                y[(size_t)t * H + r] += w[(size_t)t * k + i] * z;
            }
            free(h);
        }
        free(xt);
    }
}

/* ---------------------------------------------------------------------- */
/* NVFP4 activation quantizer ([W] Step 3: dynamic NVFP4 input quantizer   */
/* on the routed experts, block 16)                                        */
/* ---------------------------------------------------------------------- */

/* Nearest E4M3FN byte to v >= 0 by exhaustive search over the 127 finite
 * non-negative values; equal distance -> the even byte (mantissa LSB 0);
 * above 448 -> 448. */
uint32_t q4o_e4m3fn_from(float v) {
    double d = (double)v;
    if (d >= 448.0) return 0x7Eu;
    uint32_t best = 0;
    double bestdist = INFINITY;
    for (uint32_t b = 0; b <= 0x7Eu; ++b) {
        double dist = fabs(q4o_e4m3fn(b) - d);
        if (dist < bestdist || (dist == bestdist && (b & 1u) == 0)) {
            best = b;
            bestdist = dist;
        }
    }
    return best;
}

/* E2M1 magnitudes in code order. */
static const double kGrid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* Code of |v| on the grid scaled by s: nearest point, ties to the even code,
 * saturating at 6*s.  The comparisons m*s are exact in fp64. */
static uint32_t e2m1_magnitude_code(double mag, double s) {
    if (s == 0.0) return 0;
    uint32_t idx = 0;
    for (uint32_t j = 0; j < 7; ++j) {
        double mid = 0.5 * (kGrid[j] + kGrid[j + 1]) * s;
        int up = (mag > mid) || (mag == mid && ((j + 1) % 2 == 0));
        if (!up) break;
        idx = j + 1;
    }
    return idx;
}

void q4o_quant_nvfp4(int32_t rows, int32_t cols, const float* v, uint8_t* codes, uint8_t* scales) {
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t blk = 0; blk < cols / 16; ++blk) {
            const float* vb = v + r * cols + blk * 16;
            float amax = 0.0f;
            for (int j = 0; j < 16; ++j)
                if (fabsf(vb[j]) > amax) amax = fabsf(vb[j]);
            float d = amax / 6.0f; /* one fp32 division, RNE */
            uint32_t sb = q4o_e4m3fn_from(d);
            double s = q4o_e4m3fn(sb);
            scales[r * (cols / 16) + blk] = (uint8_t)sb;
            for (int j = 0; j < 16; ++j) {
                uint32_t code = e2m1_magnitude_code(fabs((double)vb[j]), s);
                if (signbit(vb[j])) code |= 8u;
                int64_t c = blk * 16 + j;
                uint8_t* byte = codes + r * (cols / 2) + c / 2;
                if (c % 2 == 0)
                    *byte = (uint8_t)((*byte & 0xF0u) | code);
                else
                    *byte = (uint8_t)((*byte & 0x0Fu) | (code << 4));
            }
        }
    }
}

/* Value of quantized activation element c of a row: e2m1 * e4m3fn (exact). */
static double act_elem(const uint8_t* row_codes, const uint8_t* row_scales, int64_t c) {
    return q4o_e2m1(q4o_nibble(row_codes, c)) * q4o_e4m3fn(row_scales[c / 16]);
}

/* ---------------------------------------------------------------------- */
/* W4A4 chunk ([W] Step 3 and its prefill comparison)                      */
/* ---------------------------------------------------------------------- */

void q4o_w4a4_up(const q4o_bank* b, int32_t T, int32_t k, const int32_t* ids,
                 const uint8_t* xq_codes, const uint8_t* xq_scales, double* u) {
    const int32_t H = b->H, I = b->I;
    for (int32_t t = 0; t < T; ++t) {
        double* xt = (double*)malloc(sizeof(double) * (size_t)H);
        for (int32_t c = 0; c < H; ++c)
            xt[c] = act_elem(xq_codes + (size_t)t * (H / 2), xq_scales + (size_t)t * (H / 16), c);
        for (int32_t i = 0; i < k; ++i) {
            const uint8_t* codes;
            const void* scales;
            float g;
            int32_t R, C;
            expert_mat(b, ids[(size_t)t * k + i], 1, &codes, &scales, &g, &R, &C);
#pragma omp parallel for schedule(static)
            for (int32_t r = 0; r < I; ++r) {
                double row[C];
                deq_row(b->fmt, C, codes, scales, g, r, row);
                double acc = 0.0;
                for (int32_t c = 0; c < C; ++c) acc += row[c] * xt[c];
                u[((size_t)t * k + i) * I + r] = acc;
            }
        }
        free(xt);
    }
}

void q4o_w4a4_down_combine(const q4o_bank* b, int32_t T, int32_t k, const int32_t* ids,
                           const double* w, const uint8_t* hq_codes, const uint8_t* hq_scales,
                           double* y) {
    const int32_t H = b->H, I = b->I;
    for (size_t i = 0; i < (size_t)T * H; ++i) y[i] = 0.0;
    for (int32_t t = 0; t < T; ++t) {
        for (int32_t i = 0; i < k; ++i) {
            size_t ri = (size_t)t * k + i;
            double* ht = (double*)malloc(sizeof(double) * (size_t)I);
            for (int32_t c = 0; c < I; ++c)
                ht[c] = act_elem(hq_codes + ri * (I / 2), hq_scales + ri * (I / 16), c);
            const uint8_t* codes;
            const void* scales;
            float g;
            int32_t R, C;
            expert_mat(b, ids[ri], 0, &codes, &scales, &g, &R, &C);
#pragma omp parallel for schedule(static)
            for (int32_t r = 0; r < H; ++r) {
                double row[C];
                deq_row(b->fmt, C, codes, scales, g, r, row);
                double z = 0.0;
                for (int32_t c = 0; c < C; ++c) z += row[c] * ht[c];
                y[(size_t)t * H + r] += w[ri] * z;
            }
            free(ht);
        }
    }
}

void q4o_moe_w4a4(const q4o_bank* b, int32_t T, int32_t k, const uint16_t* x,
                  const int32_t* ids, const double* w, uint8_t* xq_codes, uint8_t* xq_scales,
                  double* u, float* h32, uint8_t* hq_codes, uint8_t* hq_scales, double* y) {
    const int32_t H = b->H, I = b->I;
    size_t nrow = (size_t)T * k;
    float* xf = (float*)malloc(sizeof(float) * (size_t)T * H);
    uint8_t* xqc = xq_codes ? xq_codes : (uint8_t*)malloc((size_t)T * (H / 2));
    uint8_t* xqs = xq_scales ? xq_scales : (uint8_t*)malloc((size_t)T * (H / 16));
    double* uu = u ? u : (double*)malloc(sizeof(double) * nrow * I);
    float* hh = h32 ? h32 : (float*)malloc(sizeof(float) * nrow * I);
    uint8_t* hqc = hq_codes ? hq_codes : (uint8_t*)malloc(nrow * (I / 2));
    uint8_t* hqs = hq_scales ? hq_scales : (uint8_t*)malloc(nrow * (I / 16));
    /* x is bf16, so its fp32 value is exact. */
    for (size_t i = 0; i < (size_t)T * H; ++i) xf[i] = (float)q4o_bf16(x[i]);
    q4o_quant_nvfp4(T, H, xf, xqc, xqs);
    q4o_w4a4_up(b, T, k, ids, xqc, xqs, uu);
    /* h = relu(u)^2, held as the fp32 number the activation quantizer reads. */
    for (size_t i = 0; i < nrow * I; ++i) {
        double rl = uu[i] > 0.0 ? uu[i] : 0.0;
        hh[i] = (float)(rl * rl);
    }
    q4o_quant_nvfp4((int32_t)nrow, I, hh, hqc, hqs);
    q4o_w4a4_down_combine(b, T, k, ids, w, hqc, hqs, y);
    free(xf);
    if (!xq_codes) free(xqc);
    if (!xq_scales) free(xqs);
    if (!u) free(uu);
    if (!h32) free(hh);
    if (!hq_codes) free(hqc);
    if (!hq_scales) free(hqs);
}

/* ---------------------------------------------------------------------- */
/* NVFP4 lm_head GEMV and argmax ([W] Step 4; Step 5 four-token verify;    */
/* [C] precision table: lm_head NVFP4 weight-only, block 16)               */
/* ---------------------------------------------------------------------- */

void q4o_gemv_nvfp4(int32_t rows, int32_t cols, const uint8_t* codes, const uint8_t* scales,
                    float g, int32_t T, const uint16_t* x, double* logits, int32_t* argmax,
                    double* gap) {
    double* xt = (double*)malloc(sizeof(double) * (size_t)T * cols);
    for (size_t i = 0; i < (size_t)T * cols; ++i) xt[i] = q4o_bf16(x[i]);
#pragma omp parallel for schedule(static)
    for (int32_t r = 0; r < rows; ++r) {
        double row[cols];
        deq_row(Q4O_NVFP4, cols, codes, scales, g, r, row);
        for (int32_t t = 0; t < T; ++t) {
            double acc = 0.0;
            for (int32_t c = 0; c < cols; ++c) acc += row[c] * xt[(size_t)t * cols + c];
            logits[(size_t)t * rows + r] = acc;
        }
    }
    for (int32_t t = 0; t < T; ++t) {
        const double* l = logits + (size_t)t * rows;
        int32_t best = 0;
        for (int32_t r = 1; r < rows; ++r)
            if (l[r] > l[best]) best = r;
        double second = -INFINITY;
        for (int32_t r = 0; r < rows; ++r)
            if (r != best && l[r] > second) second = l[r];
        if (argmax) argmax[t] = best;
        if (gap) gap[t] = l[best] - second;
    }
    free(xt);
}

/* Nearest bf16 (RNE): round |v| to a multiple of its bf16 quantum, which is
 * 2^(e-8) for |v| in [2^(e-1), 2^e) and 2^-133 in the subnormal range. */
uint32_t q4o_bf16_from(double v) {
    if (isnan(v)) return 0x7FC0u;
    uint32_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);
    int qexp = e - 8 < -133 ? -133 : e - 8;
    double q = ldexp(nearbyint(ldexp(a, -qexp)), qexp);
    float f = (float)q; /* exact, or +inf past the bf16 range */
    uint32_t u;
    memcpy(&u, &f, 4);
    return sign | (u >> 16);
}

int32_t q4o_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void q4o_set_threads(int32_t n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ---- Shared expert, FP8 per-tensor W8A8 -------------------------------
 * [W] Step 3 (shared experts go to FP8) and the precision table of [C]
 * (shared experts: FP8 per-tensor W8A8).  Readings: weights are E4M3FN
 * codes with one fp32 scale per tensor; each activation (x into up, h into
 * down) is quantized with one static fp32 input scale per tensor, the
 * calibrated value the recipe stores; code = E4M3FN nearest-even of
 * fl32(v / s), saturating at 448, sign of v kept (finite v).  The expert MLP
 * is the routed one, relu(up x)^2 then down, and its output joins y
 * unweighted before the one bf16 rounding. */

uint32_t q4o_fp8_code(float v, float s) {
    float q = v / s; /* one fp32 division, rounded to nearest */
    uint32_t sign = signbit(q) ? 0x80u : 0u;
    return sign | q4o_e4m3fn_from(fabsf(q));
}

void q4o_fp8_quant(int32_t n, const float* v, float s, uint8_t* codes) {
    for (int32_t i = 0; i < n; ++i) codes[i] = (uint8_t)q4o_fp8_code(v[i], s);
}

/* out[r] = (sum_c e4m3(w[r][c]) * e4m3(a[c])) * s_w * s_in in fp64.  Each
 * product has at most 8 significant bits and is a multiple of 2^-18 below
 * 2^18, so for up to 2^15 columns every partial sum is exact in fp64. */
void q4o_fp8_gemv(int32_t rows, int32_t cols, const uint8_t* w, const uint8_t* a, float s_w,
                  float s_in, double* out) {
    double* av = (double*)malloc(sizeof(double) * (size_t)cols);
    for (int32_t c = 0; c < cols; ++c) av[c] = q4o_e4m3fn(a[c]);
#pragma omp parallel for schedule(static)
    for (int32_t r = 0; r < rows; ++r) {
        const uint8_t* wr = w + (size_t)r * cols;
        double acc = 0.0;
        for (int32_t c = 0; c < cols; ++c) acc += q4o_e4m3fn(wr[c]) * av[c];
        out[r] = acc * (double)s_w * (double)s_in;
    }
    free(av);
}

void q4o_shared_fp8(const q4o_shared* sh, const uint16_t* x, uint8_t* xq, double* u, float* h32,
                    uint8_t* hq, double* z) {
    const int32_t H = sh->H, S = sh->S;
    float* xf = (float*)malloc(sizeof(float) * (size_t)H);
    for (int32_t k = 0; k < H; ++k) xf[k] = (float)q4o_bf16(x[k]);
    q4o_fp8_quant(H, xf, sh->up_iscale, xq);
    q4o_fp8_gemv(S, H, sh->up_codes, xq, sh->up_wscale, sh->up_iscale, u);
    for (int32_t j = 0; j < S; ++j) {
        double r = u[j] > 0.0 ? u[j] : 0.0;
        h32[j] = (float)(r * r);
    }
    q4o_fp8_quant(S, h32, sh->down_iscale, hq);
    q4o_fp8_gemv(H, S, sh->down_codes, hq, sh->down_wscale, sh->down_iscale, z);
    free(xf);
}

/* ---- NVFP4 weight quantizer ---------------------------------------------
 * [W] Step 1 (NVFP4: 4-bit E2M1 values, an FP8 scale per 16, built with
 * ModelOpt) and the recipe table's weight-scale selection (max-based, or an
 * MSE per-block search over FP8 scale values).  Readings:
 *  - per-tensor scale g = fl32(amax / 2688) (2688 = 6 * 448, the largest
 *    E2M1 value times the largest E4M3FN value), g = 1 for an all-zero
 *    tensor; decoded weight = e2m1 * e4m3(b) * g (as the GEMVs decode it);
 *  - eff(b) = fl32(e4m3(b) * g); the code of w under b is the E2M1 magnitude
 *    nearest the exact quotient |w| / eff(b), ties to the even code,
 *    saturating at 6, with w's sign bit;
 *  - max-based: b = E4M3FN nearest-even (saturating) of
 *    fl32(bamax / fl32(6 * g)), bamax the block's largest |w|;
 *  - MSE: b minimises the block's exact squared error
 *    sum_k (|w_k| - q_k(b))^2, q_k(b) = e2m1(code_k) * eff(b), over every
 *    positive finite E4M3FN byte 0x01..0x7E; the lowest byte among equal
 *    minima; an all-zero block takes b = 0. */

static const float kMid32[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};

/* Nearest E2M1 magnitude code of the exact quotient mag / eff (mid * eff is
 * exact in fp64: 3 + 24 significant bits). */
static uint32_t wq_code(float mag, float eff) {
    uint32_t c = 0;
    for (int j = 0; j < 7; ++j) {
        double t = (double)kMid32[j] * (double)eff;
        int up = ((double)mag > t) || ((double)mag == t && ((j + 1) % 2 == 0));
        if (up) c = (uint32_t)(j + 1);
    }
    return c;
}

/* Twice the E2M1 magnitude of code c (an integer: 0, 1, 2, 3, 4, 6, 8, 12). */
static const int kTwiceE2m1[8] = {0, 1, 2, 3, 4, 6, 8, 12};

/* The MSE objective, exactly.  Expanding the square,
 *   sum_k (|w_k| - q_k)^2 = sum_k w_k^2 + F(b),  F(b) = sum_k q_k (q_k - 2 |w_k|),
 * and the first sum does not depend on b, so comparing F compares errors.
 * A term is 0 unless code_k != 0, which needs |w_k| > eff / 4.  Write
 * eff = M * 2^E (M an integer below 2^24); every such |w_k| (8 significant
 * bits, at least 2^-2 of eff) is then an integer multiple W_k of 2^E, and
 * with c_k = 2 e2m1(code_k):
 *   F(b) = P * 2^(2E - 2),  P = sum_k c_k M (c_k M - 4 W_k),
 * an exact integer: c_k M < 2^28 and, for the tensor's own g (bamax <= 2688 g,
 * eff >= 2^-9 g), W_k < 2^45, so P < 2^80 (values that would leave the
 * checked range W_k < 2^50 stop the program).  The value is held as (P, E);
 * for one g the exponents E of the 126 scale bytes span at most 19 binades,
 * so aligning two values multiplies P by at most 2^38 and stays below 2^127. */
typedef struct {
    __int128 p;
    int e;
} wq_obj;

static wq_obj wq_objective(const float* mag, float eff) {
    wq_obj o = {0, 0};
    if (!(eff > 0.0f)) return o; /* an underflowed scale decodes every code to 0: F = 0 */
    int ex;
    double f = frexp((double)eff, &ex);           /* eff = f * 2^ex, f in [0.5, 1) */
    int64_t M = (int64_t)ldexp(f, 24);            /* exact: eff has at most 24 bits */
    o.e = ex - 24;
    for (int k = 0; k < 16; ++k) {
        uint32_t code = wq_code(mag[k], eff);
        if (code == 0) continue;
        double wq = ldexp((double)mag[k], -o.e);  /* W_k, exact (see above) */
        if (wq != floor(wq) || wq >= 0x1p50) {
            fprintf(stderr, "q4o_wq: block value outside the exact range of the MSE objective\n");
            abort();
        }
        __int128 cm = (__int128)kTwiceE2m1[code] * M;
        o.p += cm * (cm - 4 * (__int128)(int64_t)wq);
    }
    return o;
}

/* a - b for F values, exactly, as (P, E) at the smaller exponent. */
static wq_obj wq_sub(wq_obj a, wq_obj b) {
    if (a.p == 0) a.e = b.e;
    if (b.p == 0) b.e = a.e;
    wq_obj d;
    d.e = a.e < b.e ? a.e : b.e;
    __int128 pa = a.p, pb = b.p;
    for (int i = 0; i < 2 * (a.e - d.e); ++i) pa *= 2;
    for (int i = 0; i < 2 * (b.e - d.e); ++i) pb *= 2;
    d.p = pa - pb;
    return d;
}

static int wq_less(wq_obj a, wq_obj b) { return wq_sub(a, b).p < 0; }

static double wq_to_double(wq_obj a) { return ldexp((double)a.p, 2 * a.e - 2); }

float q4o_wq_gscale(int64_t n, const uint16_t* w) {
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float v = fabsf((float)q4o_bf16(w[i]));
        if (v > amax) amax = v;
    }
    return amax > 0.0f ? amax / 2688.0f : 1.0f;
}

/* One block of 16 bf16 weights: scale byte and 16 codes (low nibble first
 * in 8 bytes). */
uint32_t q4o_wq_block(const uint16_t* w, float g, int mse, uint8_t* codes8) {
    float mag[16];
    float bamax = 0.0f;
    uint32_t sign[16];
    for (int k = 0; k < 16; ++k) {
        float v = (float)q4o_bf16(w[k]);
        mag[k] = fabsf(v);
        sign[k] = signbit(v) ? 8u : 0u;
        if (mag[k] > bamax) bamax = mag[k];
    }
    uint32_t b = 0;
    if (bamax > 0.0f) {
        volatile float six_g = 6.0f * g;
        volatile float t = bamax / six_g;
        b = q4o_e4m3fn_from(t);
        if (mse) {
            wq_obj best = {0, 0};
            for (uint32_t c = 1; c <= 0x7Eu; ++c) {
                volatile float eff = (float)q4o_e4m3fn(c) * g;
                wq_obj o = wq_objective(mag, eff);
                if (c == 1 || wq_less(o, best)) { /* strictly less: the lowest byte keeps a tie */
                    best = o;
                    b = c;
                }
            }
        }
    }
    volatile float eff = (float)q4o_e4m3fn(b) * g;
    for (int k = 0; k < 8; ++k) codes8[k] = 0;
    for (int k = 0; k < 16; ++k) {
        uint32_t c = (b == 0 ? 0u : wq_code(mag[k], eff)) | sign[k];
        codes8[k / 2] |= (uint8_t)(k % 2 == 0 ? c : c << 4);
    }
    return b;
}

void q4o_quant_weights_nvfp4(int32_t rows, int32_t cols, const uint16_t* w, int32_t mse, uint8_t* codes,
                             uint8_t* scales, float* gscale) {
    const float g = q4o_wq_gscale((int64_t)rows * cols, w);
    *gscale = g;
    const int64_t nb = (int64_t)rows * cols / 16;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nb; ++i) scales[i] = (uint8_t)q4o_wq_block(w + 16 * i, g, mse, codes + 8 * i);
}

/* Codes of a block under a given scale byte b (the rule above), and the
 * amount by which b's exact squared error exceeds the block's exact MSE
 * minimum (F(b) - min F, exact, rounded once to fp64).  For checking a
 * quantizer that takes the same decision by another evaluation. */
double q4o_wq_codes_excess(const uint16_t* w, float g, uint32_t b, uint8_t* codes8) {
    float mag[16];
    uint32_t sign[16];
    for (int k = 0; k < 16; ++k) {
        float v = (float)q4o_bf16(w[k]);
        mag[k] = fabsf(v);
        sign[k] = signbit(v) ? 8u : 0u;
    }
    volatile float eff = (float)q4o_e4m3fn(b) * g;
    for (int k = 0; k < 8; ++k) codes8[k] = 0;
    for (int k = 0; k < 16; ++k) {
        uint32_t c = (b == 0 ? 0u : wq_code(mag[k], eff)) | sign[k];
        codes8[k / 2] |= (uint8_t)(k % 2 == 0 ? c : c << 4);
    }
    if (b == 0 || b > 0x7Eu) return 0.0;
    wq_obj mine = wq_objective(mag, eff), best = mine;
    for (uint32_t c = 1; c <= 0x7Eu; ++c) {
        volatile float e2 = (float)q4o_e4m3fn(c) * g;
        wq_obj o = wq_objective(mag, e2);
        if (wq_less(o, best)) best = o;
    }
    return wq_to_double(wq_sub(mine, best));
}

void q4o_wq_codes_excess_blocks(int64_t nblocks, const uint16_t* w, float g, const uint8_t* scales,
                                uint8_t* codes, double* excess) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nblocks; ++i)
        excess[i] = q4o_wq_codes_excess(w + 16 * i, g, scales[i], codes + 8 * i);
}
