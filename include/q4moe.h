/*
 * libq4moe: batch-1 / few-token decode of the routed mixture-of-experts
 * layers of a 4-bit block-quantized hybrid MoE language model, on one
 * AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages, cited by title and section):
 *  [W] "Let's optimize Nemotron 3.5 Lightning - a worklog": Step 1 (W4A16:
 *      NVFP4 weights, group 16, 16-bit activations, dequantized in-kernel),
 *      Step 3 (routed experts W4A4 with a dynamic NVFP4 input quantizer;
 *      router kept at 16/32 bits), Step 4 (NVFP4 lm_head [131072 x 2688]),
 *      Interlude (a batch-1 GEMM is a weight read), Step 5 (k = 3 drafts:
 *      the verifier runs 4 tokens per step).
 *  [G] "NVIDIA-Nemotron-3.5-Lightning-30B-A3B-W4A16" README: What was
 *      changed (int4, group 64, symmetric, weight-only; 128 routed experts
 *      per MoE layer, 23 layers), Group size 64 (down_proj input is 1856
 *      wide), Checkpoint layout (per-expert 2-D up_proj and down_proj, no
 *      gate projection), Left at bfloat16 (router .gate with an fp32
 *      e_score_correction_bias).
 *  [Q] "Quantization (PTQ + QAD)": Precision Recipes, router compute FP32.
 *  [S] "The Model Card's Recommended Config Was 1.9x Slower Than No
 *      Config": The setup (128 routed experts, 6 active).
 *
 * Readings where the pages are silent (the library and its tests use them):
 *  - router: logits l = W_g x in fp32; scores s = sigmoid(l); experts are
 *    selected by the key s + bias, largest first, equal keys -> lower expert
 *    index first; gate weights are the selected scores divided by their sum
 *    (the bias only selects);
 *  - expert MLP: y = sum_i w_i * down_i( relu(up_i x)^2 ), accumulated in
 *    fp32, h kept in fp32, y rounded once to bf16 (nearest even);
 *  - NVFP4 element: E2M1 code (OCP MX v1.0) times an E4M3FN block scale (OCP
 *    OFP8) per 16 consecutive input elements, times an fp32 per-tensor
 *    scale; int4-g64 element: two's complement nibble times a bf16 scale per
 *    64 consecutive input elements;
 *  - packing: element (r, 2j) is the low nibble (bits 3..0) of byte
 *    r*cols/2 + j, element (r, 2j+1) the high nibble.
 *
 * Conventions for every entry point:
 *  - All pointers inside descriptors and all array arguments are DEVICE
 *    pointers, except the descriptors themselves (host structs, read during
 *    the call only).  The caller owns every buffer and the stream; the
 *    library never allocates, frees, copies host<->device or synchronizes.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is
 *    enqueued asynchronously on it.
 *  - Arguments are validated on the host before anything is enqueued; on a
 *    non-OK status nothing was enqueued and q4moe_last_error() describes the
 *    problem.  Nothing throws, aborts or prints.
 *  - Alignment: code arrays, x, y, logits and workspaces 16-byte aligned;
 *    scale arrays 4-byte aligned.
 *  - Workspaces: size from the matching *_ws_bytes() call; zero-filled once
 *    before the first use (q4moe_ws_init).  Every workspace starts with the
 *    same prefix at the same offsets: control words, then the epoch-tagged
 *    hand-off values of the one-launch decode, sized for the largest
 *    supported shapes (about 2.4 MB).  Only the one-launch decode writes the
 *    prefix, and each of its calls accepts only values tagged with its own
 *    epoch (one more than the last completed call's); every other entry
 *    point keeps its scratch after the prefix.  So one workspace, sized for
 *    the largest call it serves, takes any sequence of calls of any entry
 *    points, shapes and token counts issued in order on one stream; calls
 *    that overlap in time must use different workspaces.
 *  - The one-launch decode (n_tok = 1 in q4moe_w4a16_decode and its shared
 *    and W4A4 variants) is a persistent kernel whose workgroups wait on one
 *    another: it launches one workgroup per compute unit and needs all of
 *    them resident at once, so the device must not be shared with work that
 *    holds compute units for the whole call.  Every wait is bounded: if one
 *    expires (a workgroup that never became resident, or a workspace that is
 *    not zero-filled), the kernel still ends and the call has returned OK,
 *    but bit 0 of the workspace flags is set and y is not valid.  Read the
 *    flags with q4moe_ws_check (sticky until q4moe_ws_init).  A workspace
 *    whose control words were disturbed (shared by calls that overlapped,
 *    or overwritten) keeps failing this way until q4moe_ws_init.
 */
#ifndef Q4MOE_H
#define Q4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q4MOE_ABI_VERSION 1

typedef enum {
    Q4MOE_OK = 0,
    Q4MOE_EINVAL = 1,       /* null pointer, bad size or shape */
    Q4MOE_EALIGN = 2,       /* misaligned pointer */
    Q4MOE_EUNSUPPORTED = 3, /* valid but not implemented (format / shape) */
    Q4MOE_EWORKSPACE = 4,   /* workspace too small */
    Q4MOE_EDEVICE = 5       /* HIP runtime or kernel-side failure */
} q4moe_status;

typedef enum { Q4MOE_NVFP4 = 1, Q4MOE_INT4_G64 = 2 } q4moe_fmt;

/* One quantized matrix, logical row-major [rows x cols]; y = W x.
 * codes:  rows*cols/2 bytes (two elements per byte, low nibble first).
 * scales: NVFP4 -> uint8 E4M3FN [rows][cols/16];
 *         INT4_G64 -> bf16 bit patterns (uint16) [rows][cols/64].
 * gscale: NVFP4 -> device pointer to one fp32 per-tensor scale;
 *         INT4_G64 -> must be NULL. */
typedef struct {
    int32_t fmt, rows, cols;
    const uint8_t* codes;
    const void* scales;
    const float* gscale;
} q4moe_qmat;

/* An expert bank, expert-major, every expert the same shape ([G] Checkpoint
 * layout: per-expert up_proj [inter x hidden] and down_proj [hidden x inter]).
 *  up_codes   [E][inter][hidden/2]    up_scales   [E][inter][hidden/blk]
 *  down_codes [E][hidden][inter/2]    down_scales [E][hidden][inter/blk]
 *  up_gscale, down_gscale: fp32 [E] (NVFP4) or NULL (INT4_G64).
 * blk = 16 (NVFP4) or 64 (INT4_G64).  Supported: hidden and inter multiples
 * of 32 (NVFP4) or 64 (INT4_G64), each at most 4096. */
typedef struct {
    int32_t fmt, n_experts, hidden, inter;
    const uint8_t* up_codes;
    const void* up_scales;
    const float* up_gscale;
    const uint8_t* down_codes;
    const void* down_scales;
    const float* down_gscale;
} q4moe_experts;

/* Router ([Q] router compute FP32; [G] fp32 e_score_correction_bias):
 * w_g fp32 [n_experts][hidden] row-major, bias fp32 [n_experts];
 * 1 <= top_k <= min(8, n_experts), n_experts <= 256. */
typedef struct {
    const float* w_g;
    const float* bias;
    int32_t n_experts, hidden, top_k;
} q4moe_router;

/* Router top-k for n_tok bf16 tokens x [n_tok][hidden] (1 <= n_tok <= 65536).
 * Outputs ids int32 [n_tok][top_k] in selection order and w fp32
 * [n_tok][top_k]; logits (nullable) fp32 [n_tok][n_experts]. */
size_t q4moe_router_topk_ws_bytes(const q4moe_router* r, int32_t n_tok);
q4moe_status q4moe_router_topk(const q4moe_router* r, const uint16_t* x_bf16, int32_t n_tok,
                               int32_t* ids, float* w, float* logits, void* ws, size_t ws_bytes,
                               void* stream);

/* Reference dequantization of one matrix to fp32 [rows][cols], element for
 * element the value the format defines: NVFP4 fl32((e2m1 * e4m3fn) * g),
 * INT4_G64 int4 * bf16 ([W] Step 1; [G] What was changed).  No workspace. */
q4moe_status q4moe_dequant_ref(const q4moe_qmat* m, float* out, void* stream);

/* W4A16 routed-MoE decode of n_tok tokens (1 <= n_tok <= 65536) through
 * one layer ([W] Step 1 and Interlude; Step 5 for n_tok = 4; "Coming in Part
 * 2: filling the GPU" for many concurrent tokens): router top-k, up GEMV,
 * relu^2, down GEMV, weighted combine.  x bf16 [n_tok][hidden], y bf16
 * [n_tok][hidden]; ids/w (nullable) receive the routing.
 * By token count: 1 -> one persistent launch; 2-4 (NVFP4; int4: 2) ->
 * small-batch kernels that stream each selected expert once for all
 * tokens (int4: once per token and slot); more -> the grouped
 * path (per-expert dispatch lists, grouped GEMMs on fp16 MFMA with x staged
 * exactly and h carried as fp16 hi + lo, about 22 bits), which needs hidden
 * and inter multiples of 64 (else Q4MOE_EUNSUPPORTED).  Every path
 * accumulates in fp32 and rounds y once. */
size_t q4moe_w4a16_decode_ws_bytes(const q4moe_router* r, const q4moe_experts* ex, int32_t n_tok);
q4moe_status q4moe_w4a16_decode(const q4moe_router* r, const q4moe_experts* ex,
                                const uint16_t* x_bf16, int32_t n_tok, uint16_t* y_bf16,
                                int32_t* ids, float* w, void* ws, size_t ws_bytes, void* stream);

/* A stack of n_layers single-token W4A16 routed-MoE layers of one shape and
 * format (routers[l], experts[l], 1 <= n_layers <= 4096) in as few launches
 * as the device allows: one per 24 layers.  A decode step runs the model's
 * layers back to back, and its floor is the GPU work alone ([W] Step 7: one
 * graph for the drafter's passes leaves the step within ~5% of its GPU
 * work); between two launches this device idles about 3 us, a fifth of a
 * layer, so the stack runs in one persistent launch instead.  Order and
 * results are those of n_layers q4moe_w4a16_decode calls in sequence: layer
 * l + 1 starts its routing only once every row of layer l's y is written and
 * visible on the device.  x_bf16[l], y_bf16[l]: bf16 [hidden], 16-byte
 * aligned.  chain != 0: layer l + 1 takes layer l's y as its x (x_bf16[l]
 * for l > 0 is not read and may be NULL).  ids / w: NULL, or arrays of
 * n_layers (nullable) pointers receiving each layer's routing.  The
 * workspace is that of a one-token q4moe_w4a16_decode (the taps hold the last
 * layer's values).  Every workgroup of a launch must be resident at once,
 * as for the one-token decode; a shape the single launch does not fit runs
 * as one call per layer, with the same results. */
size_t q4moe_w4a16_decode_stack_ws_bytes(const q4moe_router* r, const q4moe_experts* ex);
q4moe_status q4moe_w4a16_decode_stack(const q4moe_router* routers, const q4moe_experts* experts,
                                      int32_t n_layers, const uint16_t* const* x_bf16,
                                      uint16_t* const* y_bf16, int32_t chain, int32_t* const* ids,
                                      float* const* w, void* ws, size_t ws_bytes, void* stream);

/* The grouped W4A16 path of q4moe_w4a16_decode for any token count
 * (1 <= n_tok <= 65536; hidden and inter multiples of 64, else
 * Q4MOE_EUNSUPPORTED): the same arguments, results and precision as
 * q4moe_w4a16_decode above four tokens, where that entry point takes this
 * path itself.  Exposed so that a caller can choose the backend per batch
 * size ("Quantization (PTQ + QAD)", Deployment and Serving).  Its workspace
 * holds the q4moe_w4a16_decode_taps values at the same offsets. */
size_t q4moe_w4a16_grouped_ws_bytes(const q4moe_router* r, const q4moe_experts* ex, int32_t n_tok);
q4moe_status q4moe_w4a16_grouped(const q4moe_router* r, const q4moe_experts* ex,
                                 const uint16_t* x_bf16, int32_t n_tok, uint16_t* y_bf16,
                                 int32_t* ids, float* w, void* ws, size_t ws_bytes, void* stream);

/* q4moe_w4a16_decode for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): no
 * workspace argument; the library's own static scratch of 3.5 MiB per GPU
 * (device memory held from load until the process ends) serves as the
 * workspace.  It allocates nothing.  Shapes whose workspace would exceed the
 * scratch return Q4MOE_EWORKSPACE (1-4 tokens of the 128 x 2688 x 1856
 * top-6 layer take at most 3.15 MiB).  Every call on a GPU shares that GPU's
 * scratch: calls that overlap in time on one GPU race and must not be
 * issued (calls in order on one stream are fine).  The expired-wait flag of
 * the one-launch decode is kept in the scratch and not reported. */
q4moe_status q4moe_w4a16_decode_noalloc(const q4moe_router* r, const q4moe_experts* ex,
                                        const uint16_t* x_bf16, int32_t n_tok, uint16_t* y_bf16,
                                        int32_t* ids, float* w, void* stream);

/* Byte offsets, inside a decode workspace, of values the decode leaves there
 * after each call: y32 fp32 [n_tok][hidden] (y before rounding) and
 * h fp32 [n_tok*top_k][inter] (relu(u)^2, rows ordered (token, slot)),
 * for every token count. */
typedef struct { size_t y32, h; } q4moe_decode_taps;
q4moe_status q4moe_w4a16_decode_taps(const q4moe_router* r, const q4moe_experts* ex,
                                     int32_t n_tok, q4moe_decode_taps* out);

/* FP8 per-tensor W8A8 shared expert ([W] Step 3: shared experts go to FP8,
 * they run on every token; [C] precision table: shared experts FP8
 * per-tensor W8A8).  up_codes E4M3FN [inter][hidden], down_codes E4M3FN
 * [hidden][inter], row-major, 16-byte aligned; hidden equal to the routed
 * experts', inter a multiple of 64 up to 4096.  up_wscale / down_wscale:
 * fp32 weight scale per tensor; up_iscale / down_iscale: fp32 static input
 * scale per tensor (x into up, h into down), finite and non-zero.  An
 * activation v is coded as the E4M3FN value nearest fl32(v / iscale) (ties
 * to even, saturating at 448, sign kept); u = (W q) * wscale * iscale.  The
 * MLP is relu(up x)^2 then down, as for the routed experts. */
typedef struct {
    int32_t hidden, inter;
    const uint8_t* up_codes;
    const uint8_t* down_codes;
    float up_wscale, up_iscale, down_wscale, down_iscale;
} q4moe_shared_fp8;

/* q4moe_w4a16_decode plus the FP8 shared expert: y = sum_i w_i z_i +
 * z_shared, rounded once to bf16; 1 <= n_tok <= 65536, NVFP4 or int4-g64
 * routed experts.  NVFP4 routed experts, one token: the same single launch,
 * whose shared weights are read while the router runs; 2-4 tokens: three
 * launches for the shared expert (each weight row read once for all tokens)
 * before the small-batch routed kernels, whose combine adds its output.
 * Otherwise (more tokens, or int4 routed experts): the shared expert through
 * the grouped GEMMs as a one-expert dispatch of every token (E4M3FN weights
 * and activation codes decode exactly to fp16 for the MFMA), beside the
 * routed experts' grouped path (hidden and inter multiples of 64, else
 * Q4MOE_EUNSUPPORTED). */
size_t q4moe_w4a16_decode_shared_ws_bytes(const q4moe_router* r, const q4moe_experts* ex,
                                          const q4moe_shared_fp8* sh, int32_t n_tok);
q4moe_status q4moe_w4a16_decode_shared(const q4moe_router* r, const q4moe_experts* ex,
                                       const q4moe_shared_fp8* sh, const uint16_t* x_bf16,
                                       int32_t n_tok, uint16_t* y_bf16, int32_t* ids, float* w,
                                       void* ws, size_t ws_bytes, void* stream);

/* The int4 checkpoint's form ([G] What was changed: the shared expert is
 * int4 group 64, weight-only, like the routed experts; an NVFP4 W4A16
 * checkpoint's shared expert is NVFP4): q4moe_w4a16_decode plus a 4-bit
 * W4A16 shared expert, y = sum_i w_i z_i + z_shared rounded once; sh is a
 * bank of one expert (n_experts = 1, hidden equal to the routed experts',
 * inter a multiple of 64 up to 4096, NVFP4 or INT4_G64, its own format).
 * The shared expert runs through the grouped GEMMs as a one-expert dispatch
 * of every token (x staged exactly, h as fp16 hi + lo); the routed experts
 * take the small-batch kernels (NVFP4, up to 4 tokens) or the grouped path
 * (hidden and inter multiples of 64, else Q4MOE_EUNSUPPORTED).  Taps as in
 * q4moe_shared_taps: y32, h and sh_h32 (xq and sh_hq are 0: no codes). */
size_t q4moe_w4a16_decode_shared_q4_ws_bytes(const q4moe_router* r, const q4moe_experts* ex,
                                             const q4moe_experts* sh, int32_t n_tok);
q4moe_status q4moe_w4a16_decode_shared_q4(const q4moe_router* r, const q4moe_experts* ex, const q4moe_experts* sh,
                                          const uint16_t* x_bf16, int32_t n_tok, uint16_t* y_bf16, int32_t* ids,
                                          float* w, void* ws, size_t ws_bytes, void* stream);

/* Byte offsets of the values q4moe_w4a16_decode_shared leaves in its
 * workspace: y32 and h as in q4moe_decode_taps; xq uint8 [n_tok][hidden] (x
 * codes), sh_h32 fp32 [n_tok][inter] (relu(u)^2, the h quantizer's input),
 * sh_hq uint8 [n_tok][inter] (h codes). */
typedef struct { size_t y32, h, xq, sh_h32, sh_hq; } q4moe_shared_taps;
q4moe_status q4moe_w4a16_decode_shared_taps(const q4moe_router* r, const q4moe_experts* ex,
                                            const q4moe_shared_fp8* sh, int32_t n_tok,
                                            q4moe_shared_taps* out);
q4moe_status q4moe_w4a16_decode_shared_q4_taps(const q4moe_router* r, const q4moe_experts* ex,
                                               const q4moe_experts* sh, int32_t n_tok, q4moe_shared_taps* out);

/* W4A4 routed-MoE decode of 1 <= n_tok <= 8 tokens ([W] Step 3: the
 * routed experts take 4-bit weights and activations; the MTP drafter's
 * experts are NVFP4 W4A4 too, [C] and the pages' MTP passage): as
 * q4moe_w4a16_decode, with x and h quantized to NVFP4 on the fly (per 16, an
 * E4M3FN scale amax/6 and E2M1 codes, as in q4moe_w4a4_grouped) and the
 * GEMVs run on their exact dequantized values.  One token: a single launch;
 * 2-8 tokens: the small-batch kernels, each selected expert streamed once
 * for all tokens.  NVFP4 experts and n_tok <= 8 only, else
 * Q4MOE_EUNSUPPORTED.  ids/w nullable. */
size_t q4moe_w4a4_decode_ws_bytes(const q4moe_router* r, const q4moe_experts* ex, int32_t n_tok);
q4moe_status q4moe_w4a4_decode(const q4moe_router* r, const q4moe_experts* ex, const uint16_t* x_bf16,
                               int32_t n_tok, uint16_t* y_bf16, int32_t* ids, float* w, void* ws,
                               size_t ws_bytes, void* stream);

/* Byte offsets of the values q4moe_w4a4_decode leaves in its workspace:
 * y32 fp32 [n_tok][hidden]; h32 fp32 [n_tok*top_k][inter] (relu(u)^2
 * before quantization, rows (token, slot)); xq_codes [n_tok][hidden/2],
 * xq_scales [n_tok][hidden/16]; hq_codes [n_tok*top_k][inter/2], hq_scales
 * [n_tok*top_k][inter/16] (rows (token, slot); codes low nibble first). */
typedef struct { size_t y32, h32, xq_codes, xq_scales, hq_codes, hq_scales; } q4moe_w4a4_token_taps;
q4moe_status q4moe_w4a4_decode_taps(const q4moe_router* r, const q4moe_experts* ex, int32_t n_tok,
                                    q4moe_w4a4_token_taps* out);

/* The MoE block of the W4A4 checkpoint ([W] Step 3; [C] precision table:
 * routed experts NVFP4 W4A4, shared experts FP8 per-tensor W8A8) for
 * 1 <= n_tok <= 4 tokens: q4moe_w4a4_decode plus the shared expert of
 * q4moe_w4a16_decode_shared, y = sum_i w_i z_i + z_shared rounded once.
 * One token: one launch; 2-4: the shared expert's three launches, then the
 * small-batch kernels. */
size_t q4moe_w4a4_decode_shared_ws_bytes(const q4moe_router* r, const q4moe_experts* ex,
                                         const q4moe_shared_fp8* sh, int32_t n_tok);
q4moe_status q4moe_w4a4_decode_shared(const q4moe_router* r, const q4moe_experts* ex, const q4moe_shared_fp8* sh,
                                      const uint16_t* x_bf16, int32_t n_tok, uint16_t* y_bf16, int32_t* ids,
                                      float* w, void* ws, size_t ws_bytes, void* stream);

/* Its taps: those of q4moe_w4a4_token_taps and, for the shared expert, sh_xq
 * uint8 [n_tok][hidden], sh_h32 fp32 [n_tok][inter], sh_hq uint8
 * [n_tok][inter]. */
typedef struct {
    size_t y32, h32, xq_codes, xq_scales, hq_codes, hq_scales, sh_xq, sh_h32, sh_hq;
} q4moe_w4a4_shared_taps;
q4moe_status q4moe_w4a4_decode_shared_taps(const q4moe_router* r, const q4moe_experts* ex,
                                           const q4moe_shared_fp8* sh, int32_t n_tok, q4moe_w4a4_shared_taps* out);

/* W4A4 routed-MoE layer for any token count, choosing the kernels by the
 * count (mid-batch decode: the pages point at choosing the GEMM backend per
 * batch size): up to Q4MOE_W4A4_PER_TOKEN_MAX_TOKENS tokens one
 * single-token q4moe_w4a4_decode launch per token, more tokens the grouped
 * MFMA pipeline (q4moe_w4a4_grouped).  Measured cold on MI355X at the full
 * shapes (128 x 2688 x 1856, top-6), the single-token launches (about 18 us
 * each) beat both the one-pass small-batch kernels of q4moe_w4a4_decode and
 * the grouped pipeline up to 7 tokens.  The results are those of the entry
 * point used.  ids / w are required. */
#define Q4MOE_W4A4_PER_TOKEN_MAX_TOKENS 7
size_t q4moe_w4a4_moe_ws_bytes(const q4moe_router* r, const q4moe_experts* ex, int32_t n_tok);
q4moe_status q4moe_w4a4_moe(const q4moe_router* r, const q4moe_experts* ex, const uint16_t* x_bf16, int32_t n_tok,
                            uint16_t* y_bf16, int32_t* ids, float* w, void* ws, size_t ws_bytes, void* stream);

/* FP8 per-tensor W8A8 matrix: the MTP drafter's lm_head ("Quantization
 * (PTQ + QAD)", MTP Drafter Precision: the drafter shares the checkpoint's
 * lm_head, quantized to FP8).  codes E4M3FN [rows][cols] row-major,
 * 16-byte aligned, cols a multiple of 64 in [64, 4096], rows * cols < 2^32;
 * wscale: fp32 weight scale per tensor; iscale: fp32 static input scale per
 * tensor (finite, non-zero).  The same per-tensor W8A8 format as the shared
 * expert: an activation v is coded as the E4M3FN value nearest
 * fl32(v / iscale) (ties to even, saturating at 448, sign kept). */
typedef struct {
    int32_t rows, cols;
    const uint8_t* codes;
    float wscale, iscale;
} q4moe_fp8_mat;

/* FP8 GEMV + argmax for 1 <= n_tok <= 4 bf16 tokens x [n_tok][cols]:
 * logits fp32 [n_tok][rows] = (sum_c e4m3(W[r][c]) e4m3(code(x[t][c]))) *
 * wscale * iscale (each product exact, fp32 accumulation); argmax (nullable)
 * int32 [n_tok]: the lowest row among each token's largest logits.  The
 * workspace keeps the activation codes uint8 [n_tok][cols] at the offset
 * q4moe_fp8_gemv_taps returns. */
size_t q4moe_fp8_gemv_ws_bytes(const q4moe_fp8_mat* m, int32_t n_tok);
q4moe_status q4moe_fp8_gemv(const q4moe_fp8_mat* m, const uint16_t* x_bf16, int32_t n_tok, float* logits,
                            int32_t* argmax, void* ws, size_t ws_bytes, void* stream);
q4moe_status q4moe_fp8_gemv_taps(const q4moe_fp8_mat* m, int32_t n_tok, size_t* xq);

/* NVFP4 weight quantizer ([W] Step 1: NVFP4 weights, E2M1 values with an
 * FP8 (E4M3) scale per 16, built with ModelOpt; the recipe table's
 * weight-scale selection: max-based, or an MSE per-block search over FP8
 * scale values).  bf16 w [rows][cols] (cols % 16 == 0, 16-byte aligned) ->
 * codes [rows][cols/2] (low nibble first, 8-byte aligned), E4M3FN scales
 * [rows][cols/16], and the fp32 per-tensor scale *gscale (device memory),
 * such that weight = e2m1 * e4m3 * g as every decoder here reads it.
 *   g = fl32(amax / 2688) (1 for an all-zero tensor); eff(b) = fl32(e4m3(b) g);
 *   the code of w under b is the E2M1 magnitude nearest |w| / eff(b) (the
 *   exact quotient), ties to the even code, saturating at 6, sign of w kept;
 *   Q4MOE_WQ_MAX: b = E4M3FN nearest-even of fl32(bamax / fl32(6 g));
 *   Q4MOE_WQ_MSE: b in 0x01..0x7E minimising the block's squared error
 *   sum (|w| - e2m1(code) * eff(b))^2, the lowest byte among equal minima;
 *   an all-zero block takes b = 0.  The search evaluates the error in fp32
 *   (summed in element order): where two bytes' exact errors differ by less
 *   than that evaluation's rounding (at most about 2^-15 of the block's
 *   sum w^2), it may keep the other byte.
 * Two launches; the workspace holds the first one's partial maxima. */
enum { Q4MOE_WQ_MAX = 0, Q4MOE_WQ_MSE = 1 };
size_t q4moe_quantize_weights_ws_bytes(int32_t rows, int32_t cols);
q4moe_status q4moe_quantize_weights(const uint16_t* w_bf16, int32_t rows, int32_t cols, int32_t mode,
                                    uint8_t* codes, uint8_t* scales, float* gscale, void* ws, size_t ws_bytes,
                                    void* stream);

/* W4A4 routed-MoE chunk of n_tok tokens (1 <= n_tok <= 65536), NVFP4 only
 * ([W] Step 3: routed experts take 4-bit weights and activations, the
 * activations quantized on the fly per block of 16 with an E4M3FN scale
 * amax/6).  Tokens are routed, dispatched per expert, and each expert runs
 * as a grouped GEMM on the matrix cores.  x bf16 [n_tok][hidden] -> y bf16
 * [n_tok][hidden]; ids int32 / w fp32 [n_tok][top_k] are required outputs. */
size_t q4moe_w4a4_grouped_ws_bytes(const q4moe_router* r, const q4moe_experts* ex, int32_t n_tok);
q4moe_status q4moe_w4a4_grouped(const q4moe_router* r, const q4moe_experts* ex,
                                const uint16_t* x_bf16, int32_t n_tok, uint16_t* y_bf16,
                                int32_t* ids, float* w, void* ws, size_t ws_bytes, void* stream);

/* Workspace offsets of the W4A4 stage values left after each call.
 * Rows p = 0 .. n_tok*top_k-1 are in dispatch order (expert ascending, then
 * token ascending); perm int32 [n_tok*top_k] maps row p to t*top_k + slot;
 * expert_offsets int32 [n_experts+1] are the row ranges per expert.
 *  xq_codes uint8 [n_tok][hidden/2], xq_scales uint8 [n_tok][hidden/16]
 *  h32 fp32 [rows][inter]        (relu(u)^2 before quantization)
 *  hq_codes uint8 [rows][inter/2], hq_scales uint8 [rows][inter/16]
 *  y32 fp32 [n_tok][hidden]      (y before rounding) */
typedef struct {
    size_t perm, expert_offsets, xq_codes, xq_scales, h32, hq_codes, hq_scales, y32;
} q4moe_w4a4_taps;
q4moe_status q4moe_w4a4_grouped_taps(const q4moe_router* r, const q4moe_experts* ex,
                                     int32_t n_tok, q4moe_w4a4_taps* out);

/* NVFP4 W4A16 GEMV for the lm_head ([W] Step 4; [C] precision table:
 * lm_head NVFP4 weight-only, block 16): logits fp32 [n_tok][rows] =
 * g * W x_t for bf16 x [n_tok][cols], 1 <= n_tok <= 4, cols a multiple of 32
 * up to 4096, codes under 4 GiB; argmax (nullable) int32 [n_tok] = lowest row
 * index among the largest logits.  Products and sums are fp32 on fp16 MFMA:
 * weights decode exactly; token t of x is scaled by the power of two that
 * puts its largest magnitude in [2^14, 2^15) and rounded to fp16, which is
 * exact for every element at least 2^-28 of that maximum.  Two launches (the
 * GEMV, then the argmax merge when argmax is given); no atomics, so the
 * workspace needs no clearing between calls. */
size_t q4moe_w4a16_gemv_ws_bytes(const q4moe_qmat* m, int32_t n_tok);
q4moe_status q4moe_w4a16_gemv(const q4moe_qmat* m, const uint16_t* x_bf16, int32_t n_tok,
                              float* logits, int32_t* argmax, void* ws, size_t ws_bytes,
                              void* stream);

/* Zero-fill a workspace on `stream` with a kernel (no memset node, so it can
 * be captured in a graph). */
q4moe_status q4moe_ws_init(void* ws, size_t ws_bytes, void* stream);

/* Kernel-side status word of a workspace: 0 = fine.  Reads device memory
 * synchronously on `stream` (for tests and diagnostics, not the hot path). */
q4moe_status q4moe_ws_check(const void* ws, size_t ws_bytes, void* stream, uint32_t* flags);

const char* q4moe_status_str(q4moe_status s);
/* Detail of the last non-OK status on the calling thread. */
const char* q4moe_last_error(void);
int32_t q4moe_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif
