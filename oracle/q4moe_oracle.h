/*
 * q4moe oracle: a plain, slow CPU statement of what the routed-MoE decode
 * path computes, in fp64.  TEST INFRASTRUCTURE ONLY: it is called by the
 * tests, by the package's smoke check and by the benchmark's CPU-baseline
 * leg, never by the library it checks.  It shares no source, header, table
 * or helper with the HIP library; its types below are its own.
 *
 * Sources (web pages, cited by title and section):
 *  [W]  "Let's optimize Nemotron 3.5 Lightning - a worklog" (itsnav.com):
 *       Step 1 (W4A16, NVFP4 group 16), Step 3 (routed experts W4A4 with a
 *       dynamic NVFP4 input quantizer), Step 4 (NVFP4 lm_head), Interlude
 *       (batch-1 GEMM is a weight read), Step 5 (k=3 drafts, 4-token verify).
 *  [C]  model card "naveenrajk/nemotron35-w4a4-v13": precision table
 *       (routed experts NVFP4 block 16; lm_head NVFP4 weight-only).
 *  [G]  "NVIDIA-Nemotron-3.5-Lightning-30B-A3B-W4A16" README: "What was
 *       changed" (int4, group 64, symmetric, weight-only), "Group size 64"
 *       (down_proj input 1856 wide), "Checkpoint layout" (per-expert 2-D
 *       up_proj / down_proj), "Left at bfloat16" (fp32 e_score_correction_bias).
 *  [Q]  "Quantization (PTQ + QAD)" (Nemotron 3.5 Super docs): Precision
 *       Recipes table, row "Router / gate (compute)": FP32.
 *  [S]  "The Model Card's Recommended Config Was 1.9x Slower Than No Config":
 *       The setup (128 routed experts, 6 active).
 * Element formats, which the pages name but do not define, follow the public
 * OCP specifications: E2M1 from "OCP Microscaling Formats (MX) v1.0",
 * E4M3FN from "OCP 8-bit Floating Point Specification (OFP8)".
 *
 * Readings where the pages are silent (each one listed in the design notes):
 *  - router: sigmoid scores s = 1/(1+exp(-l)); selection key s + bias; top-k
 *    by key descending, equal keys -> lower expert index first; gate weights
 *    are the selected s renormalised to sum 1 (bias not in the weights);
 *  - expert MLP: y = sum_i w_i * down_i(relu(up_i x)^2);
 *  - nibble order: element 2j in bits 3..0 of byte j, element 2j+1 in 7..4;
 *  - NVFP4 weight value: fl32((e2m1(code) * e4m3fn(scale)) * g), g an fp32
 *    per-tensor scale; int4-g64 value: int4(code) * bf16(scale);
 *  - NVFP4 activation quantizer (W4A4): per 16-block, scale byte =
 *    E4M3FN round-to-nearest-even (saturating at 448) of fl32(amax / 6);
 *    code = nearest E2M1 magnitude of |v| / scale, ties to the even code,
 *    saturating at 6, sign bit = sign bit of v; scale 0 -> magnitude 0;
 *  - shared expert (FP8 per-tensor W8A8): E4M3FN weights with an fp32 scale
 *    per tensor, static fp32 input scales per tensor, activation code =
 *    E4M3FN nearest-even of fl32(v / s) saturating at 448; relu^2 like the
 *    routed experts; its output joins y with weight 1, before the rounding.
 */
#ifndef Q4MOE_ORACLE_H
#define Q4MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { Q4O_NVFP4 = 1, Q4O_INT4_G64 = 2 };

/* One expert bank, expert-major, logical row-major layout.
 * up:   codes [E][I][H/2], scales [E][I][H/blk];  down: codes [E][H][I/2],
 * scales [E][H][I/blk].  blk = 16 (NVFP4, scales are E4M3FN bytes) or 64
 * (int4-g64, scales are bf16 bit patterns).  up_g / down_g: fp32 per-tensor
 * scale per expert (NVFP4 only; ignored for int4). */
typedef struct {
    int32_t fmt, E, H, I;
    const uint8_t* up_codes;
    const void* up_scales;
    const float* up_g;
    const uint8_t* down_codes;
    const void* down_scales;
    const float* down_g;
} q4o_bank;

/* Element decoders (closed forms of the OCP definitions). */
double q4o_e2m1(uint32_t code);      /* 4-bit code -> value in {0,.5,...,6} with sign */
double q4o_e4m3fn(uint32_t byte);    /* NaN for S.1111.111, no infinities */
double q4o_int4(uint32_t code);      /* two's complement nibble, -8..7 */
double q4o_bf16(uint32_t bits);      /* bf16 bit pattern -> value */
uint32_t q4o_nibble(const uint8_t* row_codes, int64_t c);

/* Dequantize one matrix [rows][cols] to fp32 (the exact per-element values). */
void q4o_dequant(int32_t fmt, int32_t rows, int32_t cols, const uint8_t* codes,
                 const void* scales, float g, float* out);

/* Router for T tokens: logits [T][E], scores [T][E] (fp64), ids [T][k] in
 * selection order, w [T][k], gap [T] = key(k-th) - key(k+1-th) (0 if k == E). */
void q4o_router(int32_t E, int32_t H, int32_t T, int32_t k, const float* wg,
                const float* bias, const uint16_t* x, double* logits, double* scores,
                int32_t* ids, double* w, double* gap);

/* W4A16 routed-MoE decode for T tokens given ids/w [T][k].
 * u_tap (nullable) [T][k][I]: up outputs; y [T][H]: unrounded outputs. */
void q4o_moe_w4a16(const q4o_bank* bank, int32_t T, int32_t k, const uint16_t* x,
                   const int32_t* ids, const double* w, double* u_tap, double* y);

/* E4M3FN byte nearest to v (RNE, saturating to 448), found by exhaustive search. */
uint32_t q4o_e4m3fn_from(float v);

/* NVFP4 activation quantizer over rows of `cols` fp32 values (cols % 16 == 0):
 * codes [rows][cols/2] (same nibble order as weights), scales [rows][cols/16]. */
void q4o_quant_nvfp4(int32_t rows, int32_t cols, const float* v, uint8_t* codes, uint8_t* scales);

/* W4A4 routed-MoE chunk for T tokens given ids/w.  Taps (all nullable):
 * xq_codes [T][H/2], xq_scales [T][H/16]; u [T][k][I] (fp64); h32 [T][k][I]
 * (fl32 of relu(u)^2, the quantizer input); hq_codes [T][k][I/2],
 * hq_scales [T][k][I/16].  y [T][H] unrounded. */
void q4o_moe_w4a4(const q4o_bank* bank, int32_t T, int32_t k, const uint16_t* x,
                  const int32_t* ids, const double* w, uint8_t* xq_codes, uint8_t* xq_scales,
                  double* u, float* h32, uint8_t* hq_codes, uint8_t* hq_scales, double* y);

/* Stage-wise pieces of the W4A4 chunk: down projection and combine from a
 * given quantized h (rows ordered (t, slot)), and up projection from a given
 * quantized x. */
void q4o_w4a4_down_combine(const q4o_bank* bank, int32_t T, int32_t k, const int32_t* ids,
                           const double* w, const uint8_t* hq_codes, const uint8_t* hq_scales,
                           double* y);
void q4o_w4a4_up(const q4o_bank* bank, int32_t T, int32_t k, const int32_t* ids,
                 const uint8_t* xq_codes, const uint8_t* xq_scales, double* u);

/* NVFP4 GEMV: logits[t][r] = sum_c W[r][c] * bf16(x[t][c]) (fp64);
 * argmax[t] = lowest row index among the maxima; gap[t] = top1 - top2. */
void q4o_gemv_nvfp4(int32_t rows, int32_t cols, const uint8_t* codes, const uint8_t* scales,
                    float g, int32_t T, const uint16_t* x, double* logits, int32_t* argmax,
                    double* gap);

/* Shared expert, FP8 per-tensor W8A8 ([W] Step 3; [C] precision table).
 * up_codes E4M3FN [S][H], down_codes E4M3FN [H][S]; per-tensor fp32 weight
 * scales and static fp32 input scales (x into up, h into down). */
typedef struct {
    int32_t H, S;
    const uint8_t* up_codes;
    const uint8_t* down_codes;
    float up_wscale, up_iscale, down_wscale, down_iscale;
} q4o_shared;

/* E4M3FN code of fl32(v / s): nearest-even, saturating at 448, sign kept. */
uint32_t q4o_fp8_code(float v, float s);
void q4o_fp8_quant(int32_t n, const float* v, float s, uint8_t* codes);

/* out[r] = (sum_c e4m3(w[r][c]) e4m3(a[c])) * s_w * s_in, fp64 (exact sums). */
void q4o_fp8_gemv(int32_t rows, int32_t cols, const uint8_t* w, const uint8_t* a, float s_w,
                  float s_in, double* out);

/* The whole shared expert for one token: xq [H] codes; u [S] fp64;
 * h32 [S] = fl32(relu(u)^2), the h quantizer's input; hq [S] codes;
 * z [H] fp64, the expert's output (joins y with weight 1). */
void q4o_shared_fp8(const q4o_shared* sh, const uint16_t* x, uint8_t* xq, double* u, float* h32,
                    uint8_t* hq, double* z);

/* NVFP4 weight quantizer of a bf16 matrix [rows][cols] (cols % 16 == 0):
 * codes [rows][cols/2], scales [rows][cols/16], per-tensor g.  mse = 0:
 * max-based block scales; mse = 1: per-block search over every positive
 * finite E4M3FN scale (readings in q4moe_oracle.c).  Also its pieces. */
void q4o_quant_weights_nvfp4(int32_t rows, int32_t cols, const uint16_t* w, int32_t mse, uint8_t* codes,
                             uint8_t* scales, float* gscale);
float q4o_wq_gscale(int64_t n, const uint16_t* w);
uint32_t q4o_wq_block(const uint16_t* w, float g, int mse, uint8_t* codes8);
/* The codes of one block under scale byte b, and how much b's exact squared
 * error exceeds the block's exact minimum over the bytes 0x01..0x7E. */
double q4o_wq_codes_excess(const uint16_t* w, float g, uint32_t b, uint8_t* codes8);
void q4o_wq_codes_excess_blocks(int64_t nblocks, const uint16_t* w, float g, const uint8_t* scales,
                                uint8_t* codes, double* excess);

/* bf16 bit pattern nearest to v (RNE), for chaining an oracle output. */
uint32_t q4o_bf16_from(double v);

/* Threads the oracle's parallel loops use (1 without OpenMP), and a way to
 * set them (n > 0). */
int32_t q4o_threads(void);
void q4o_set_threads(int32_t n);

#ifdef __cplusplus
}
#endif
#endif
