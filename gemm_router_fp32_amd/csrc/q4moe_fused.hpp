// One-launch routed-MoE decode of a single token on gfx950.
//
// Batch-1 decode reads every active weight once and does almost no
// arithmetic per byte ("Let's optimize Nemotron 3.5 Lightning - a worklog",
// Interlude), so the whole layer runs as ONE persistent launch whose waves
// stream the selected experts' 4-bit weights over the entire chip:
//
//   R  router:  workgroup e (< E) computes logit e (its waves split the row
//               of W_g) and the sigmoid score, and publishes the score.
//   S  select:  every workgroup polls the E scores, forms the keys
//               score + bias, and each wave runs the exact fp32 top-k itself
//               (wave max, then the lowest index holding it).
//   U  up:      the K x I (slot, row) up units and the K x H down units are
//               each split evenly over all waves; each wave issues the loads
//               of its up rows, computes h = relu(W_up x)^2 for them into
//               LDS, and then issues the loads of its down rows (which do
//               not depend on h), so that the up rows every workgroup waits
//               for come first and the down weights stream during the h
//               hand-off.
//   P  publish: the workgroup publishes its h rows (one per thread), then
//               all its threads poll the h of the slots its down rows use
//               into LDS.  (A poll result counts only after every load the
//               wave issued before it, so the first poll also waits for the
//               down weights.)
//   D  down:    every wave computes z = w * g * (W_down h) from the weights
//               in registers and publishes z.
//   C  combine: one workgroup per 64-row block polls that block's z of every
//               slot and sums them in slot order (deterministic) into y.
//
// Hand-offs between workgroups carry their own readiness: every published
// value is a 64-bit (value, epoch) pair written with one device-coherent
// store (an agent-scope relaxed atomic: it bypasses the per-XCD L2 copies),
// and readers poll the values until they carry the current epoch.  No
// counters, no store-completion waits and no agent-scope fences (which
// write back or invalidate a whole L2 on this part) sit on the critical
// path.  The epoch advances by one per call (each workgroup keeps its own
// copy and advances it early in the call), so stale values of earlier calls
// never match and nothing has to be cleared.  Values many workgroups read (scores, h) and the epoch word are
// kept in kReplicas copies, copy b % kReplicas for workgroup b (which is also
// its XCD), so no single line or memory channel serves the whole chip.
// Every poll is bounded; on expiry the kernel flags the workspace and carries
// on, so it always ends.
//
// Two variants ride on the same phases ("Let's optimize Nemotron 3.5
// Lightning - a worklog", Step 3; the W4A4 model card's precision table):
//   SH  the FP8 per-tensor W8A8 shared expert: its weights stream while the
//       router runs, x is coded during the score hand-off, its h codes are
//       exchanged four per value ahead of the routed h, its down rows run
//       during the routed h hand-off, and its z is one more combine slot.
//   A4  W4A4 routed experts: x and h quantized to NVFP4 inside the launch
//       (h by the workgroup that makes it, which then publishes codes and
//       scales instead of fp32 h), the GEMVs running on the exact bf16
//       values of the quantized activations.
#pragma once

#include "q4moe_kernels.hpp"

// Phase marker for instrumented builds; expands to nothing in the library.
#ifndef Q4MOE_PHASE
#define Q4MOE_PHASE(i)
#endif
#ifndef Q4MOE_WAVE_MARK
#define Q4MOE_WAVE_MARK(i)
#endif

namespace q4moe {

constexpr int kReplicas = 8;
constexpr int kWaves = 8;    // waves per workgroup (one workgroup per CU)
constexpr int kMaxUp = 3;      // up passes (two rows each) per wave, loads in flight together
constexpr int kDownRows = 8;  // down rows per wave (one slot), loads in flight together
constexpr int kMaxWgUp = 512;        // up rows per workgroup (K * I / grid)
constexpr int kRowBlock = 64;
constexpr uint32_t kPollLimit = 200000;  // polls (each at least one memory round trip) before giving up

// LDS layouts of x and h: one 16-byte pad after every 32-element chunk (x
// and h as 16-bit values: 64 bytes, then 16 bytes of pad) or after every 32
// fp32 values (128 bytes, then 16).  A GEMV lane reads its own chunk as
// consecutive 16-byte pieces; unpadded, the chunks of all lanes start in the
// same banks and every piece read serialises (8 ways for fp32, 4 for 16-bit),
// while with the pad the chunks of any 8 consecutive lanes start 4 banks
// apart (lane strides of 36 and 20 words) and one read pass serves them all.
__device__ __forceinline__ int lds_pad_f32(int i) { return i + 4 * (i >> 5); }   // fp32 element i
__device__ __forceinline__ int lds_pad_u16(int j) { return j + 8 * (j >> 5); }   // 16-bit element j
__device__ __forceinline__ int lds_pad_u128(int t) { return t + (t >> 2); }      // 16-byte piece t of 16-bit values
constexpr int kLdsH16Lo = 2 * 4096 + 2 * 4096 / 4;  // 16-bit h: the lo halves start here (past the padded hi halves)

// Block scales reach the GEMV lanes through LDS: a row's scales (or a down
// unit's eight rows', which are adjacent) are read with one wide load per
// lane, 8 or 16 bytes at 4-byte-aligned offsets clamped into the region, and
// each wave stages them in its own kScaleStage bytes of LDS, from which a
// lane takes the 2 bytes of each of its chunks.  One load instruction per
// row pass (and one per down unit) replaces one 2-byte load per chunk and
// row: the load path pays per instruction, not per byte.
constexpr int kScaleStage = 2048;  // per wave: the 8 down rows' scales (I <= 2048), or 2 kMaxUp up rows of 256

// The 4-byte-aligned region [b4, b4 + span4) holding bytes [s, s + n) of a
// scale array (s even, n >= 8, array 4-byte aligned and a multiple of 4 long).
__device__ __forceinline__ void scale_region(uint32_t s, uint32_t n, uint32_t& b4, uint32_t& span4) {
    b4 = s & ~3u;
    span4 = ((s + n + 3u) & ~3u) - b4;
}

// Workspace control words of the fused decode.
enum : int {
    FW_EPOCH = 256,  // [grid]: workgroup b's epoch of the last call (at most CTRL_WORDS - FW_EPOCH workgroups)
};

struct FusedArgs {
    int E, H, I, K;
    const float* wg;
    const float* bias;
    const uint16_t* x;
    const uint8_t* upc;
    const void* ups;
    const float* upg;
    const uint8_t* dnc;
    const void* dns;
    const float* dng;
    uint16_t* y;
    int32_t* ids_out;             // nullable
    float* w_out;                 // nullable
    uint32_t* ctrl;
    unsigned long long* sc_tag;   // [kReplicas][E]    (score, epoch)
    unsigned long long* h_tag;    // [kReplicas][K][I] (h, epoch)
    unsigned long long* z_tag;    // [K][H]            (w * g * z, epoch)
    int32_t* ids;                 // [K]    tap
    float* w;                     // [K]    tap
    float* h;                     // [K][I] tap
    float* y32;                   // [H]
    // FP8 per-tensor W8A8 shared expert (the SH variants): up [S][H] and
    // down [H][S] E4M3FN codes, per-tensor weight scales and static input
    // scales; its output z is slot K of z_tag.
    int S;
    const uint8_t* shu;
    const uint8_t* shd;
    float su_w, su_in, sd_w, sd_in;
    unsigned long long* hq_tag;   // [kReplicas][S/4] (four h codes, epoch)
    uint8_t* sh_xq;               // [H] tap: x codes
    float* sh_h;                  // [S] tap: relu(u)^2 before quantization
    uint8_t* sh_hq;               // [S] tap: h codes
    // W4A4 (the A4 variants): taps of the NVFP4 activation codes
    uint8_t* xq_codes;            // [H/2]
    uint8_t* xq_scales;           // [H/16]
    uint8_t* hq_codes;            // [K][I/2]
    uint8_t* hq_scales;           // [K][I/16]
};

// A stack of single-token layers of one shape in one launch: the per-layer
// pointers (the rest of FusedArgs is common), at most kStackMax layers.
constexpr int kStackMax = 24;
struct StackLayer {
    const float* wg;
    const float* bias;
    const uint16_t* x;
    const uint8_t* upc;
    const void* ups;
    const float* upg;
    const uint8_t* dnc;
    const void* dns;
    const float* dng;
    uint16_t* y;
    int32_t* ids_out;  // nullable
    float* w_out;      // nullable
};
struct StackArgs {
    FusedArgs a;
    unsigned long long* y_tag;     // [kReplicas][H/2]: (two bf16 of y, epoch), chained stacks
    unsigned long long* done_tag;  // [kReplicas][64]: (0, epoch) per combined block of 64 rows of y
    int n_layers;
    int chain;  // layer l + 1 takes layer l's y as its x
    StackLayer layer[kStackMax];
};
// Where a layer of the stack stands: its index, whether it takes the
// previous layer's y as x, and the y tags (null outside a stack).
struct StackCtl {
    int layer;
    int chain;
    unsigned long long* y_tag;
    unsigned long long* done_tag;
};

__device__ __forceinline__ unsigned long long tagged(float v, uint32_t ep) {
    return ((unsigned long long)ep << 32) | __float_as_uint(v);
}
__device__ __forceinline__ void put_tag(unsigned long long* p, float v, uint32_t ep) {
    __hip_atomic_store(p, tagged(v, ep), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long get_tag(const unsigned long long* p) {
    return __hip_atomic_load(const_cast<unsigned long long*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tag_is(unsigned long long t, uint32_t ep) { return (uint32_t)(t >> 32) == ep; }
__device__ __forceinline__ float tag_value(unsigned long long t) { return __uint_as_float((uint32_t)t); }

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Exact fp32 top-k by rank, in two stages.  Each key is held as a 64-bit
// composite: the order-preserving integer image of the key in the high half
// (NaN at INT_MIN, below every key) and 2^32 - 1 - e in the low half, so
// that of two keys the one earlier in the selection order (the larger key;
// for equal keys the lower expert index) has the larger composite, and no
// two composites are equal.  An expert's rank is the number of composites
// above its own; the experts of rank < K are the selection, in rank order.
//  1. Wave w ranks the G = EP / 8 composites of experts w G .. w G + G - 1
//     among themselves (EP = E rounded up to 64, 128 or 256; slots past E
//     hold composites below every key), P = 64 / G lanes per expert, each
//     counting over G / P of them, and writes its K largest in order to its
//     list.
//  2. Each entry of the lists is counted against the entries of all lists
//     (eight lanes per entry, one list each).  For an entry whose rank among
//     all experts is below K that count is its rank (every expert above it
//     is in the first K of its own group, so in a list); for any other entry
//     the count is at least K.
// Every comparison within a stage is independent, and the lists are small.
// The gates (topk_gates) are taken later, off the path to the up loads.
__device__ __forceinline__ long long topk_comp(float key, int e) {
    const uint32_t ko = (uint32_t)key_order(key);
    return (long long)(((unsigned long long)ko << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)e));
}

template <int EP>
__device__ __forceinline__ void topk_stage1(const FusedArgs& a, const long long* s_comp, long long (*s_list)[8]) {
    constexpr int G = EP / kWaves;  // 8, 16 or 32 experts per wave
    constexpr int P = 64 / G;       // lanes per expert: 8, 4 or 2
    constexpr int NC = G / P;       // composites each lane compares: 1, 4 or 16
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e = wave * G + lane / P, part = lane % P;
    const long long ce = s_comp[e];
    const long long* src = s_comp + wave * G + part * NC;
    int rank = 0;
#pragma unroll
    for (int j = 0; j < NC; ++j) rank += src[j] > ce ? 1 : 0;
    if constexpr (P >= 2) rank += __builtin_amdgcn_mov_dpp(rank, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
    if constexpr (P >= 4) rank += __builtin_amdgcn_mov_dpp(rank, 0x4E, 0xF, 0xF, true);  // [2,3,0,1]
    if constexpr (P >= 8) rank += __builtin_amdgcn_mov_dpp(rank, 0x141, 0xF, 0xF, true);  // row_half_mirror
    if (part == 0 && rank < a.K) s_list[wave][rank] = ce;
}

__device__ __forceinline__ void topk_stage2(const FusedArgs& a, long long (*s_list)[8], const float* s_scores,
                                            int* s_ids, float* s_sc) {
    // thread t: position (t >> 3) & 7 of list t >> 6 (positions past K hold
    // nothing and write nothing), counted against list t & 7; the 8 lanes of
    // an entry are adjacent, so the 8 counts are summed with lane moves
    const int t = threadIdx.x, lst = t >> 6, pos = (t >> 3) & 7, part = t & 7;
    const bool valid = pos < a.K;
    const long long c = s_list[lst][valid ? pos : 0];
    int rank = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q)
        if (q < a.K) rank += s_list[part][q] > c ? 1 : 0;
    rank += __builtin_amdgcn_mov_dpp(rank, 0xB1, 0xF, 0xF, true);   // quad_perm [1,0,3,2]
    rank += __builtin_amdgcn_mov_dpp(rank, 0x4E, 0xF, 0xF, true);   // [2,3,0,1]
    rank += __builtin_amdgcn_mov_dpp(rank, 0x141, 0xF, 0xF, true);  // row_half_mirror: the other quad of the 8
    if (part == 0 && valid && rank < a.K) {
        const int e = (int)(0xFFFFFFFFu - (uint32_t)(unsigned long long)c);
        s_ids[rank] = e;
        s_sc[rank] = s_scores[e];
        if ((int)((unsigned long long)c >> 32) == INT_MIN) atomicOr(a.ctrl + CTRL_FLAGS, 2u);  // a NaN key chosen
    }
}

// The gates of one wave's copy: lane i < K takes the i-th selected score
// over the sum of the K selected scores, summed in selection order.
__device__ __forceinline__ void topk_gates(const FusedArgs& a, const float* s_sc, float* s_w) {
    const int lane = threadIdx.x & 63;
    const float4 p0 = reinterpret_cast<const float4*>(s_sc)[0], p1 = reinterpret_cast<const float4*>(s_sc)[1];
    const float sc[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    float ssum = 0.f, mine = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (i < a.K) ssum += sc[i];
        mine = lane == i ? sc[i] : mine;
    }
    if (lane < a.K) s_w[lane] = mine / ssum;
    __builtin_amdgcn_wave_barrier();
}

// Sums over the 64 lanes of eight values v[0..7] at once: after it, lane l
// holds the sum of v[rows8_label(l)] over all lanes.  Each level halves the
// lanes a value spans and pairs two values into one register: across the
// wave halves (lanes 0-31 keep v[2i], 32-63 v[2i+1]), across 16-lane rows,
// across 8-lane halves of a row; the last three steps sum inside each group
// of eight lanes, so every lane of the group holds the total.
__device__ __forceinline__ float add_swap32(float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_swap16(float a, float b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float rows8_sum(const float (&v)[8]) {
    const int lane = threadIdx.x & 63;
    // level 1: [v0 | v1], [v2 | v3], [v4 | v5], [v6 | v7] (by wave half)
    const float p0 = add_swap32(v[0], v[1]), p1 = add_swap32(v[2], v[3]);
    const float p2 = add_swap32(v[4], v[5]), p3 = add_swap32(v[6], v[7]);
    // level 2: by 16-lane row, q0 = [v0, v2, v1, v3], q1 = [v4, v6, v5, v7]
    const float q0 = add_swap16(p0, p1), q1 = add_swap16(p2, p3);
    // level 3: lanes 0-7 of a row take q0, lanes 8-15 q1 (row_ror:8 pairs
    // lane i with lane i ^ 8)
    const bool hi8 = (lane & 8) != 0;
    const float x = hi8 ? q1 : q0, y = hi8 ? q0 : q1;
    float r = x + dpp_mov<0x128>(y);
    // inside each group of eight lanes: quad_perm [1,0,3,2], [2,3,0,1], then
    // row_half_mirror (lane i with lane 7 - i of its half row)
    r += dpp_mov<0xB1>(r);
    r += dpp_mov<0x4E>(r);
    r += dpp_mov<0x141>(r);
    return r;
}
// Row of the eight whose sum lane l holds after rows8_sum: 4 for lanes 8-15
// of a 16-lane row, plus [0, 2, 1, 3] by the row's index.
__device__ __forceinline__ int rows8_label(int lane) {
    return ((lane >> 3) & 1) * 4 + ((lane >> 4) & 1) * 2 + ((lane >> 5) & 1);
}

// Units of [0, total) owned by wave index `w` of `n` waves: [lo, hi).
// 32-bit: total <= 8 * 4096 and w <= 8 * (workgroups on the device), so
// w * total stays far below 2^32.
__device__ __forceinline__ int share_lo(int total, int w, int n) {
    return (int)(((uint32_t)w * (uint32_t)total) / (uint32_t)n);
}

// E4M3FN code of fl32(v / s) with v's sign (finite v): the FP8 activation
// quantizer of the shared expert.
__device__ __forceinline__ uint32_t fp8_act_code(float v, float s) {
    const float q = __fdiv_rn(v, s);
    return ((__float_as_uint(q) >> 24) & 0x80u) | e4m3fn_rne_sat(fabsf(q));
}

// Sixteen E4M3FN weights . sixteen bf16 activations (pairs in natural
// order): every fp8 value is exact in bf16, so each product is exact.
__device__ __forceinline__ float fp8_chunk_bf16(const uint4 q, const uint4 x0, const uint4 x1) {
    float p = 0.f;
    p = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, 1.0f, false), as_bf16x2(x0.x), p);
    p = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, 1.0f, true), as_bf16x2(x0.y), p);
    p = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, 1.0f, false), as_bf16x2(x0.z), p);
    p = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, 1.0f, true), as_bf16x2(x0.w), p);
    p = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.z, 1.0f, false), as_bf16x2(x1.x), p);
    p = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.z, 1.0f, true), as_bf16x2(x1.y), p);
    p = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.w, 1.0f, false), as_bf16x2(x1.z), p);
    p = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.w, 1.0f, true), as_bf16x2(x1.w), p);
    return p;
}

// Four E4M3FN codes (one dword) -> four bf16 (exact), as two dwords.
__device__ __forceinline__ uint2 fp8x4_bf16(uint32_t v) {
    return make_uint2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, false)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, true)));
}

// A4: W4A4, the activations (x into up, h into down) quantized to NVFP4 on
// the fly: x by the waves that do not poll the scores, h by every workgroup
// for the slots it uses, once the h hand-off is in; both replaced in LDS by
// their exact dequantized values, so the GEMVs themselves are unchanged.
// One single-token layer, run by every workgroup of the launch; ep is the
// layer's epoch (one more than the last layer's, on this workspace).  STK:
// the layer is one of a stack (k_decode_stack), and from the second layer on
// it starts its routing only once the previous layer's y is complete.
template <int FMT, int C, int C2, bool SH, bool A4, bool STK>
__device__ __forceinline__ void fused_layer(const FusedArgs& a, const uint32_t ep, const StackCtl& sk, const uint32_t tid,
                                            const uint32_t bid) {
    __shared__ float s_part[kWaves];
    __shared__ __attribute__((aligned(16))) long long s_comp[256];  // selection composites (key, index)
    __shared__ float s_scores[256];
    __shared__ long long s_list[kWaves][8];  // each wave's K largest composites, in order
    __shared__ int s_sel_ids[8];
    __shared__ __attribute__((aligned(16))) float s_sel_sc[8];
    __shared__ float s_w_all[kWaves][8];  // each wave's copy of the gates
    // h of the (at most two, adjacent) slots this workgroup's down rows use,
    // padded: fp32 (NVFP4), or 16-bit (int4: bf16 hi halves, then lo halves
    // from kLdsH16Lo; W4A4: bf16)
    __shared__ float s_h[kLdsH16Lo];
    uint16_t* const s_h16 = reinterpret_cast<uint16_t*>(s_h);
    __shared__ float s_hrow[kMaxWgUp];  // this workgroup's up results, before they are published
    __shared__ uint4 s_x[512 + 128];    // x (bf16, H <= 4096, padded), read once per workgroup
    __shared__ __attribute__((aligned(16))) uint8_t s_scst[kWaves][kScaleStage];  // each wave's block scales
    uint8_t* const my_sc = s_scst[tid >> 6];
    // shared expert: x and h codes decoded to bf16 (natural order), and this
    // workgroup's (at most 16) h codes before they are published
    __shared__ uint32_t s_xb[SH ? 2048 : 1], s_shb[SH ? 2048 : 1], s_shq[SH ? 4 : 1];
    const int lane = tid & 63, wave = tid >> 6;
    const int seg = lane >> 5, li = lane & 31;
    const int NW = gridDim.x * kWaves, gw = bid * kWaves + wave;
    const int nchH = a.H / 32, nchI = a.I / 32;
    // Up rows: lane li of a 32-lane segment takes chunks c * lpr + li
    // (c < C), so each load instruction reads one contiguous run of the row.
    const int lpr = (nchH + C - 1) / C;
    uint32_t* flags = a.ctrl + CTRL_FLAGS;
    const int rep = bid % kReplicas;

    Q4MOE_PHASE(0);
    // selection slots past E: composites below every key (never chosen)
    if ((int)tid >= a.E && tid < 256) s_comp[tid] = topk_comp(__builtin_nanf(""), tid);
    // Thread 128 + e polls the score of expert e: waves 2 and up store
    // nothing in the router phase, so their poll results do not wait for
    // the score stores to complete.
    const int pe = (int)tid - 128;
    const bool poller = pe >= 0 && pe < a.E;
    const float bias = a.bias[poller ? pe : 0];
    // Router row of workgroup e < E (its waves split it); every workgroup
    // issues these loads (past E it reads row 0 and ignores it), so that all
    // of the kernel's first loads leave together, before anything waits.
    const int nf4 = a.H / 4;
    const int rlo = wave * nf4 / kWaves, rhi = (wave + 1) * nf4 / kWaves;
    const float4* wr = reinterpret_cast<const float4*>(a.wg + (size_t)((int)bid < a.E ? bid : 0) * a.H);
    // a wave's share is at most 128 pieces (H <= 4096): two per lane
    // (clamped; the extra one is masked)
    float4 wv[2];
    uint2 xb[2];
    // In a chained stack, x of every layer but the first is the previous
    // layer's y, which arrives with its tags (below).
    const bool x_from_y = STK && sk.chain && sk.layer > 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int j = min(rlo + lane + 64 * i, rhi - 1);
        wv[i] = wr[j];
        if (!x_from_y) xb[i] = *reinterpret_cast<const uint2*>(a.x + 4 * j);
    }

    // x into LDS once per workgroup (the up GEMV reads it from there); the
    // store waits for the load, so in a stack it follows the y poll, whose
    // loads then leave without waiting for it
    const bool x_lds = !A4 && !x_from_y && (int)tid < a.H / 8;
    uint4 xl = make_uint4(0u, 0u, 0u, 0u);
    if (x_lds) xl = *reinterpret_cast<const uint4*>(a.x + 8 * tid);
    if (!STK && x_lds) s_x[lds_pad_u128(tid)] = xl;
    if constexpr (STK) {
        if (sk.layer > 0 && !sk.chain) {
            // Independent layers: the routing waits until every block of the
            // previous layer's y has been combined (its done tags), as the
            // next call would wait for the previous one's end.  One wave
            // polls the 42 (H / 64) tags of this workgroup's copy: a poll of
            // every y value by every workgroup would put megabytes of poll
            // traffic beside the previous layer's last hand-offs.
            if (wave == 0) {
                const int nbk = (a.H + kRowBlock - 1) / kRowBlock;
                const unsigned long long* src = sk.done_tag + (size_t)rep * 64 + min(lane, nbk - 1);
                bool have = lane >= nbk;
                for (uint32_t polls = 0; !__all(have); ++polls) {
                    const unsigned long long v = get_tag(src);
                    have = have || tag_is(v, ep - 1u);
                    if (polls > kPollLimit) {
                        if (lane == 0) atomicOr(flags, 1u);
                        break;
                    }
                    if (!__all(have)) __builtin_amdgcn_s_sleep(1);
                }
            }
        }
        if (sk.layer > 0 && sk.chain) {
            // A chain: the previous layer's y is this layer's x, its (two
            // bf16, epoch) values, one copy per workgroup, thread t polling
            // pairs t + 512 m.
            const int np = a.H / 2;
            const unsigned long long* src = sk.y_tag + (size_t)rep * np;
            const uint32_t epy = ep - 1u;
            uint32_t pend = 0;
#pragma unroll
            for (int m = 0; m < 4; ++m)
                if ((int)tid + 512 * m < np) pend |= 1u << m;
            for (uint32_t polls = 0; __any(pend != 0u); ++polls) {
                unsigned long long v[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) v[m] = (pend >> m) & 1u ? get_tag(src + tid + 512 * m) : 0ull;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    if (((pend >> m) & 1u) && tag_is(v[m], epy)) {
                        if (x_from_y) {
                            const int t = tid + 512 * m;  // elements 2t, 2t + 1
                            reinterpret_cast<uint32_t*>(&s_x[lds_pad_u128(t >> 2)])[t & 3] = (uint32_t)v[m];
                        }
                        pend &= ~(1u << m);
                    }
                }
                if (polls > kPollLimit) {
                    if (lane == 0) atomicOr(flags, 1u);
                    break;
                }
                if (__any(pend != 0u)) __builtin_amdgcn_s_sleep(1);
            }
        }
        if (x_lds) s_x[lds_pad_u128(tid)] = xl;
        __syncthreads();
        if (x_from_y) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int j = min(rlo + lane + 64 * i, rhi - 1);  // elements 4j .. 4j + 3
                xb[i] = reinterpret_cast<const uint2*>(&s_x[lds_pad_u128(j >> 1)])[j & 1];
            }
        }
    }
    // x pieces the waves that will not poll the scores quantize during the
    // score hand-off (eight values each, at most two per thread: H / 8 <= 512
    // pieces over at least four such waves), loaded now with the router's
    // loads; every thread loads, clamped into x, and the pollers' are unused
    const int npw = (a.E + 63) / 64;
    const int iw = wave < 2 ? wave : wave - npw, nidle = kWaves - npw;
    uint4 xqv[2];
    if constexpr (SH || A4) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
            xqv[i] = *reinterpret_cast<const uint4*>(a.x + 8 * min(iw * 64 + lane + i * nidle * 64, a.H / 8 - 1));
    }

    // Shared expert: its weights do not depend on the routing, so they
    // stream while the router runs (the loads leave in two bursts, below).
    // Workgroup b takes the up rows of h-code quads [sq0, sq1) (at most 16
    // rows: one per 32-lane segment, lane li reading chunks li + 32 c), and
    // wave gw the (at most two) down rows [sd0, sd1), lane l reading chunks
    // l + 64 c.  Reads past a row's end are clamped into it and masked at use.
    constexpr int CS = SH ? 2 * C : 1;  // H / 16 <= 32 * CS
    constexpr int CD = SH ? 4 : 1;      // S / 16 <= 64 * CD
    uint4 qsu[CS], qsd[2][CD];
    int sq0 = 0, sq1 = 0, shr = 0, sd0 = 0, sd1 = 0;
    if constexpr (SH) {
        const int nq = a.S / 4;
        sq0 = share_lo(nq, bid, gridDim.x);
        sq1 = share_lo(nq, bid + 1, gridDim.x);
        shr = 4 * sq0 + 2 * wave + seg;
        sd0 = share_lo(a.H, gw, NW);
        sd1 = share_lo(a.H, gw + 1, NW);
    }
    auto issue_sh_up = [&]() {
        const uint32_t rb = (uint32_t)(shr < 4 * sq1 ? shr : 0) * (uint32_t)a.H;
#pragma unroll
        for (int c = 0; c < CS; ++c) {
            const int ch = min(li + 32 * c, a.H / 16 - 1);
            qsu[c] = ldg16_stream(a.shu + (rb + (uint32_t)ch * 16u));
        }
    };
    auto issue_sh_dn = [&]() {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const uint32_t rb2 = (uint32_t)min(sd0 + p, a.H - 1) * (uint32_t)a.S;
#pragma unroll
            for (int c = 0; c < CD; ++c) {
                const int ch = min(lane + 64 * c, a.S / 16 - 1);
                qsd[p][c] = ldg16_stream(a.shd + (rb2 + (uint32_t)ch * 16u));
            }
        }
    };

    compiler_fence();  // keep every load above in the entry block

    // ---- R: workgroup e computes router logit e; its waves split the row
    if ((int)bid < a.E) {
        const int e = bid;
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if (rlo + lane + 64 * i < rhi) {
                acc = __builtin_fmaf(wv[i].x, bf16_bits_to_f32(xb[i].x & 0xffffu), acc);
                acc = __builtin_fmaf(wv[i].y, bf16_bits_to_f32(xb[i].x >> 16), acc);
                acc = __builtin_fmaf(wv[i].z, bf16_bits_to_f32(xb[i].y & 0xffffu), acc);
                acc = __builtin_fmaf(wv[i].w, bf16_bits_to_f32(xb[i].y >> 16), acc);
            }
        }
        acc = seg_sum_last<64>(acc);
        if (lane == 63) s_part[wave] = acc;
        __syncthreads();
        if (tid < kReplicas) {  // thread t publishes copy t
            float l = 0.f;
#pragma unroll
            for (int v = 0; v < kWaves; ++v) l += s_part[v];
            const float sc = 1.0f / (1.0f + expf(-l));
            put_tag(a.sc_tag + tid * a.E + e, sc, ep);
        }
    }
    Q4MOE_PHASE(1);
    // Shared expert up rows: their loads leave once the router rows are in
    // (workgroups past E wait for their unused router loads), so that the
    // router's reads do not queue behind them in the memory system.
    if constexpr (SH) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        issue_sh_up();
    }

    // unit bookkeeping (routing-independent: done while the scores travel)
    const int RU = a.K * a.I;
    int u0, u1, wu0, wu1;
    if constexpr (A4) {
        // W4A4: a workgroup owns whole 16-row blocks of h (the quantizer's
        // blocks), so that it can quantize them itself before publishing
        const int nbk = RU / 16;
        wu0 = 16 * share_lo(nbk, bid, gridDim.x);
        wu1 = 16 * share_lo(nbk, bid + 1, gridDim.x);
        u0 = wu0 + share_lo(wu1 - wu0, wave, kWaves);
        u1 = wu0 + share_lo(wu1 - wu0, wave + 1, kWaves);
    } else {
        u0 = share_lo(RU, gw, NW);
        u1 = share_lo(RU, gw + 1, NW);
        wu0 = share_lo(RU, bid * kWaves, NW);
        wu1 = share_lo(RU, (bid + 1) * kWaves, NW);
    }
    // A wave's up units span at most two slots: slot(u) = us0 + (u >= ubnd).
    const int us0 = (u1 > u0 ? u0 : 0) / a.I, ubnd = (us0 + 1) * a.I;
    const int n_up_pass = (u1 - u0 + 1) / 2;  // <= kMaxUp (checked on the host)
    // Down units are runs of kDownRows rows inside one slot: unit q covers
    // rows 8 (q % dpu) .. 8 (q % dpu) + 7 of slot q / dpu, and wave gw takes
    // unit gw (the waves past the last unit hold no down rows).
    const int dpu = (a.H + kDownRows - 1) / kDownRows, n_du = a.K * dpu;
    const bool dwave = gw < n_du;
    const int dslot = dwave ? gw / dpu : 0, drow0 = dwave ? (gw - dslot * dpu) * kDownRows : 0;
    // the workgroup's down units span slots sl0 .. sl1 (at most two: dpu >=
    // kWaves - 1 is checked on the host)
    const int wdu0 = bid * kWaves, wdu1 = min(wdu0 + kWaves, n_du);
    const int sl0 = wdu1 > wdu0 ? wdu0 / dpu : 0, sl1 = wdu1 > wdu0 ? (wdu1 - 1) / dpu : -1;

    // ---- S: poll the scores (one copy per workgroup), form the keys.  One
    // poll in flight at a time, so that the loop ends with nothing
    // outstanding: a poll left in flight would hold up the next wait on the
    // wave's memory counter (register reuse makes the compiler place one at
    // the top-k), and with it the whole workgroup at the next barrier.
    if (wave >= 2 && wave < 2 + (a.E + 63) / 64) {
        const unsigned long long* src = a.sc_tag + rep * a.E + (poller ? pe : 0);
        bool have = !poller;
        for (uint32_t polls = 0;; ++polls) {
            const unsigned long long v = get_tag(src);
            if (!have && tag_is(v, ep)) {
                const float sc = tag_value(v);
                s_scores[pe] = sc;
                s_comp[pe] = topk_comp(sc + bias, pe);
                have = true;
            }
            if (!__any(!have)) break;
            if (polls > kPollLimit) {
                if (lane == 0) atomicOr(flags, 1u);
                break;
            }
        }
    } else if constexpr (SH || A4) {
        // The waves that do not poll quantize x, eight values per thread:
        // for the shared expert to E4M3FN codes (into LDS as their bf16
        // values), for W4A4 to NVFP4 (lane pairs share a block of 16; into
        // LDS as bf16 of the exact dequantized values).
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int t = iw * 64 + lane + i * nidle * 64;
            if (t >= a.H / 8) break;
            const uint4 v = xqv[i];
            const uint32_t in[4] = {v.x, v.y, v.z, v.w};
            float f[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f[2 * j] = bf16_bits_to_f32(in[j] & 0xffffu);
                f[2 * j + 1] = bf16_bits_to_f32(in[j] >> 16);
            }
            if constexpr (SH) {
                uint32_t cw[2] = {0u, 0u};
#pragma unroll
                for (int j = 0; j < 8; ++j) cw[j >> 2] |= fp8_act_code(f[j], a.su_in) << (8 * (j & 3));
                const uint2 b0 = fp8x4_bf16(cw[0]), b1 = fp8x4_bf16(cw[1]);
                *reinterpret_cast<uint4*>(&s_xb[4 * t]) = make_uint4(b0.x, b0.y, b1.x, b1.y);
                if (bid == 0) *reinterpret_cast<uint2*>(a.sh_xq + 8 * t) = make_uint2(cw[0], cw[1]);
            }
            if constexpr (A4) {
                const Nvfp4Half b = nvfp4_quant8_pair(f);
                nvfp4_dequant8(b, f);
                uint32_t o[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    o[j] = (__float_as_uint(f[2 * j]) >> 16) | (__float_as_uint(f[2 * j + 1]) & 0xffff0000u);
                s_x[lds_pad_u128(t)] = make_uint4(o[0], o[1], o[2], o[3]);
                if (bid == 0) {
                    *reinterpret_cast<uint32_t*>(a.xq_codes + 4 * t) = b.code;
                    if ((t & 1) == 0) a.xq_scales[t / 2] = (uint8_t)b.sb;
                }
            }
        }
    }
    // Every wave holds its epoch value before this barrier (the empty asm
    // takes it as an input, so its load has returned): the workgroup's copy
    // can then advance after the next barrier without any wave reading the
    // new value.
    asm volatile("" ::"v"(ep));
    __syncthreads();
    Q4MOE_PHASE(2);
    // Shared expert down rows: after the score hand-off, for the same reason
    // (two smaller bursts delay the routing less than one).
    if constexpr (SH) issue_sh_dn();
    if (a.E <= 64)
        topk_stage1<64>(a, s_comp, s_list);
    else if (a.E <= 128)
        topk_stage1<128>(a, s_comp, s_list);
    else
        topk_stage1<256>(a, s_comp, s_list);
    __syncthreads();
    topk_stage2(a, s_list, s_scores, s_sel_ids, s_sel_sc);
    __syncthreads();
    int* ids = s_sel_ids;
    float* wsel = s_w_all[wave];
    // the workgroup's epoch copy advances now, long before the kernel ends,
    // so nothing is left for its last instructions (a stack advances it once,
    // after its last layer: inside the layer loop the compiler would wait for
    // this store's completion before the next layer's up loads)
    if (!STK && tid == 0) __hip_atomic_store(a.ctrl + FW_EPOCH + bid, ep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    Q4MOE_PHASE(3);

    // ---- U: issue the loads of this wave's up rows.  Every lane issues every
    // load (an invalid row or chunk reads a valid address and is zeroed
    // through its scale at compute time), so the loads stay in issue order
    // and each use waits only for its own data.  Offsets are 32-bit from the
    // uniform bases (the argument limits keep a bank under 2^31 bytes), and
    // each row index (< 2^20) times its row bytes (<= 2048) is a full-rate
    // 24-bit multiply: the row of unit u of slot s is u + ids[s] * rows -
    // s * rows, a select between the wave's two slots.
    const uint8_t* ups8 = reinterpret_cast<const uint8_t*>(a.ups);
    const uint8_t* dns8 = reinterpret_cast<const uint8_t*>(a.dns);
    const int us1 = min(us0 + 1, a.K - 1);
    const uint32_t urb = a.H / 2, usb = (FMT == FMT_NVFP4) ? a.H / 16 : a.H / 32;  // bytes per up row
    const uint32_t drb = a.I / 2, dsb = (FMT == FMT_NVFP4) ? a.I / 16 : a.I / 32;  // bytes per down row
    uint32_t uco[C], uso[C];  // this lane's chunk offsets within an up row
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int ch = min(c * lpr + li, nchH - 1);
        uco[c] = ch * 16;
        uso[c] = (FMT == FMT_NVFP4) ? ch * 2 : (ch >> 1) * 2;
    }
    uint4 qu[kMaxUp][C];
    uint32_t su[kMaxUp][C];
    // up scales: the 8-byte piece at offset uso8[p] of pass p's row region
    // (which starts at byte usk[p] of its 4-byte-aligned cover)
    u32x2 usc[kMaxUp];
    uint32_t uso8[kMaxUp], usk[kMaxUp];
    // per-tensor scales of the wave's two up slots
    const int idu0 = ids[us0], idu1 = ids[us1];
    float gu0 = 1.0f, gu1 = 1.0f;
    if constexpr (FMT == FMT_NVFP4) {
        gu0 = a.upg[idu0];
        gu1 = a.upg[idu1];
    }
    const int uoff0 = idu0 * a.I - us0 * a.I, uoff1 = idu1 * a.I - (us0 + 1) * a.I;
    uint32_t urow[kMaxUp];
#pragma unroll
    for (int p = 0; p < kMaxUp; ++p) {
        int u = u0 + 2 * p + seg;
        if (u >= u1) u = u1 > u0 ? u0 : 0;
        urow[p] = (uint32_t)(u + (u >= ubnd ? uoff1 : uoff0));
    }
    compiler_fence();
    // the scales first (one load per pass: each segment its row's region),
    // so that they are in by the time the codes are
#pragma unroll
    for (int p = 0; p < kMaxUp; ++p) {
        uint32_t b4, span4;
        scale_region(__umul24(urow[p], usb), usb, b4, span4);
        usk[p] = __umul24(urow[p], usb) - b4;
        uso8[p] = min(8u * (uint32_t)li, span4 - 8u);
        usc[p] = ldg8_a4(ups8 + (b4 + uso8[p]));
    }
#pragma unroll
    for (int p = 0; p < kMaxUp; ++p) {
        const uint32_t rc = __umul24(urow[p], urb);
#pragma unroll
        for (int c = 0; c < C; ++c) qu[p][c] = ldg16_stream(a.upc + (rc + uco[c]));
    }
    compiler_fence();
    Q4MOE_PHASE(8);
    // the gates, while the up rows travel
    topk_gates(a, s_sel_sc, wsel);
    if (gw == 0 && lane < a.K) {
        const int id = ids[lane];
        const float wv = wsel[lane];
        a.ids[lane] = id;
        a.w[lane] = wv;
        if (a.ids_out) a.ids_out[lane] = id;
        if (a.w_out) a.w_out[lane] = wv;
    }

    // ---- shared expert up: u = (W x) * s_w * s_in for this segment's row
    // (its weights arrived during the routing), h = relu(u)^2; the
    // workgroup's h codes are published at once, four per value, so that
    // they have travelled by the time the down rows need them
    if constexpr (SH) {
        const int nck = a.H / 16;
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < CS; ++c) {
            const int chr = li + 32 * c, ch = min(chr, nck - 1);
            const uint4* xp = reinterpret_cast<const uint4*>(&s_xb[8 * ch]);
            const float p = fp8_chunk_bf16(qsu[c], xp[0], xp[1]);
            acc += chr < nck ? p : 0.f;
        }
        acc = seg_sum_last<32>(acc);
        if (li == 31 && shr < 4 * sq1) {
            const float r = fmaxf(acc * (a.su_w * a.su_in), 0.f), h = r * r;
            const uint32_t code = fp8_act_code(h, a.sd_in);
            reinterpret_cast<uint8_t*>(s_shq)[shr - 4 * sq0] = (uint8_t)code;
            a.sh_h[shr] = h;
            a.sh_hq[shr] = (uint8_t)code;
        }
        __syncthreads();
        const int j = tid;
        if (j < sq1 - sq0) {
            const float v = __uint_as_float(s_shq[j]);
#pragma unroll
            for (int rp = 0; rp < kReplicas; ++rp) put_tag(a.hq_tag + (size_t)rp * (a.S / 4) + sq0 + j, v, ep);
        }
    }

    // activations of this lane's up chunks, from LDS
    uint32_t xa[C][16];
    float xs[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int ch = min(c * lpr + li, nchH - 1);
        uint32_t nat[16];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint4 v = s_x[5 * ch + k];
            nat[4 * k + 0] = v.x;
            nat[4 * k + 1] = v.y;
            nat[4 * k + 2] = v.z;
            nat[4 * k + 3] = v.w;
        }
        if constexpr (FMT == FMT_NVFP4) {
#pragma unroll
            for (int j = 0; j < 16; ++j) xa[c][j] = nat[j];
            xs[c] = 0.f;
        } else {
#pragma unroll
            for (int d = 0; d < 4; ++d) int4_pair_order(nat + 4 * d, xa[c] + 4 * d);
            xs[c] = pair_sum_bf16(nat);
        }
    }

    // the up scales through LDS: pass p's row region at 256 (2 p + seg)
    // (a row's scales are at most 256 bytes: H <= 4096)
#pragma unroll
    for (int p = 0; p < kMaxUp; ++p) {
        uint32_t* d = reinterpret_cast<uint32_t*>(my_sc + 256 * (2 * p + seg) + uso8[p]);
        d[0] = usc[p][0];
        d[1] = usc[p][1];
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int p = 0; p < kMaxUp; ++p) {
#pragma unroll
        for (int c = 0; c < C; ++c)
            su[p][c] = *reinterpret_cast<const uint16_t*>(my_sc + 256 * (2 * p + seg) + usk[p] + uso[c]);
    }
    __builtin_amdgcn_wave_barrier();

    // ---- U: h = relu(W_up x)^2 for this wave's rows: unit u0 + 2 p + seg
    // ends in lane 31 + 32 seg of hres[p] (for W4A4 also in LDS)
    float hres[kMaxUp];
#pragma unroll
    for (int p = 0; p < kMaxUp; ++p) {
        hres[p] = 0.f;
        if (p < n_up_pass) {
            const int u = u0 + 2 * p + seg;
            const bool ok = u < u1;
            const int slot = us0 + (u >= ubnd ? 1 : 0);
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const bool chok = li < lpr && c * lpr + li < nchH;
                if constexpr (FMT == FMT_NVFP4) {
                    const f32x2 sp = e4m3fn_x2_f32(su[p][c]);
                    const float s0 = chok ? sp[0] : 0.f, s1 = chok ? sp[1] : 0.f;
                    acc += nvfp4_chunk_bf16(qu[p][c], xa[c], s0, s1);
                } else {
                    const float sg = chok ? bf16_bits_to_f32(su[p][c]) : 0.f;
                    acc = __builtin_fmaf(sg, int4_chunk_bf16(qu[p][c], xa[c]) - 136.0f * xs[c], acc);
                }
            }
            acc = seg_sum_last<32>(acc);
            const float g = slot == us0 ? gu0 : gu1;
            const float rl = fmaxf(acc * g, 0.f);
            hres[p] = rl * rl;
            if constexpr (A4)
                if (li == 31 && ok) s_hrow[u - wu0] = hres[p];
        }
    }
    Q4MOE_PHASE(9);
    Q4MOE_WAVE_MARK(0);

    // ---- P: publish h, then issue the down loads, then poll the h of the
    // slots the workgroup's down rows use into LDS.  (A poll result counts
    // only after every load the wave issued before it, so the first poll
    // also waits for the down weights.)
    if constexpr (!A4) {
        // Every wave publishes its own (at most 2 kMaxUp) rows as soon as
        // they are done, with no workgroup barrier: lane l stores copy
        // l / (2 kMaxUp) of unit u0 + l % (2 kMaxUp), all copies in one store.
        constexpr int NU = 2 * kMaxUp;
        static_assert(NU * kReplicas <= 64, "one wave store holds every copy");
        const int k = lane % NU, rp = lane / NU;
        float v = 0.f;
#pragma unroll
        for (int p = 0; p < kMaxUp; ++p) {
            const float h0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hres[p]), 31));
            const float h1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hres[p]), 63));
            v = k == 2 * p ? h0 : v;
            v = k == 2 * p + 1 ? h1 : v;
        }
        if (rp < kReplicas && u0 + k < u1) put_tag(a.h_tag + (size_t)rp * RU + (u0 + k), v, ep);
        if (lane < NU && u0 + lane < u1) a.h[u0 + lane] = v;
    } else {
        // W4A4: the workgroup's h blocks to NVFP4 (lane pairs: half a block
        // each), published as one (8 codes, epoch) value per half block and
        // one (scale, epoch) value per block, kReplicas copies each (per
        // copy: K I / 8 code values, then K I / 16 scale values)
        __syncthreads();
        const int j = tid;
        if (j < wu1 - wu0) a.h[wu0 + j] = s_hrow[j];
        if (j < (wu1 - wu0) / 8) {
            float f[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) f[k] = s_hrow[8 * j + k];
            const Nvfp4Half b = nvfp4_quant8_pair(f);
            const int hb = wu0 / 8 + j;  // global half-block index (slot-major)
            const size_t per = (size_t)(RU / 8 + RU / 16);
#pragma unroll
            for (int rp = 0; rp < kReplicas; ++rp) {
                put_tag(a.h_tag + rp * per + hb, __uint_as_float(b.code), ep);
                if ((j & 1) == 0) put_tag(a.h_tag + rp * per + RU / 8 + hb / 2, __uint_as_float(b.sb), ep);
            }
            *reinterpret_cast<uint32_t*>(a.hq_codes + (size_t)hb * 4) = b.code;
            if ((j & 1) == 0) a.hq_scales[hb / 2] = (uint8_t)b.sb;
        }
    }

    // Then the loads of a down wave's rows, once its h has left.  They leave
    // only now: a load waits at issue while the CU's load queue is full, and
    // the queue is full of up loads until about now, so issued earlier they
    // would hold the wave (and its h) back.  The rows past the slot's end
    // (H % kDownRows != 0) read its last row and are dropped at the publish.
    // First every up load is retired (all were used by now): otherwise the
    // compiler counts them as pending past the branch and, where their
    // registers are reused, waits for the down weights as well.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    compiler_fence();
    // Shared expert: one poll of the h-code quads (t and t + 512 for thread
    // t), issued before the down loads so that its results do not wait for
    // them (the quads not yet published by then are polled again later).
    const unsigned long long* srcq = a.hq_tag + (size_t)rep * (a.S / 4);
    unsigned long long vq[2];
    if constexpr (SH) {
#pragma unroll
        for (int m = 0; m < 2; ++m) vq[m] = get_tag(srcq + min((int)tid + 512 * m, a.S / 4 - 1));
    }
    compiler_fence();
    uint4 qd[kDownRows][C2];
    uint32_t sd[kDownRows][C2];
    // down scales: the unit's kDownRows rows are adjacent (H % kDownRows ==
    // 0), so their scales are one region, read as 16-byte pieces at dso16[k]
    // of its 4-byte-aligned cover (the region starts at byte dsk of it)
    u32x4 dsc[C2];
    uint32_t dso16[C2], dso[C2], dsk = 0;
#pragma unroll
    for (int c = 0; c < C2; ++c) {
        const int ch = min(lane * C2 + c, nchI - 1);
        dso[c] = (FMT == FMT_NVFP4) ? ch * 2 : (ch >> 1) * 2;
    }
    float gdn = 1.0f;  // per-tensor scale of the down matrix (NVFP4)
    // (with the shared expert every wave issues them, the few without down
    // rows reading rows 0-7 of slot 0: loads under a branch would make the
    // compiler wait for all of them before the shared expert's h codes)
    if (SH || dwave) {
        const int drow = ids[dslot] * a.H + drow0;
        uint32_t b4, span4;
        scale_region(__umul24((uint32_t)drow, dsb), kDownRows * dsb, b4, span4);
        dsk = __umul24((uint32_t)drow, dsb) - b4;
#pragma unroll
        for (int k = 0; k < C2; ++k) {
            dso16[k] = min(16u * (uint32_t)(lane + 64 * k), span4 - 16u);
            dsc[k] = ldg16_a4(dns8 + (b4 + dso16[k]));
        }
        uint32_t dco[C2];
#pragma unroll
        for (int c = 0; c < C2; ++c) dco[c] = min(lane * C2 + c, nchI - 1) * 16;
#pragma unroll
        for (int p = 0; p < kDownRows; ++p) {
            const uint32_t rc = __umul24((uint32_t)(drow + p), drb);
#pragma unroll
            for (int c = 0; c < C2; ++c) qd[p][c] = ldg16_stream(a.dnc + (rc + dco[c]));
        }
        if constexpr (FMT == FMT_NVFP4) gdn = a.dng[ids[dslot]];
    }
    compiler_fence();
    Q4MOE_WAVE_MARK(1);
    // The polls leave once every wave's down loads have: they reach the
    // memory system behind them, by when the h they read has been published.
    __syncthreads();
    Q4MOE_PHASE(4);

    if constexpr (SH) {
        // The shared expert's h codes into LDS (from the early poll; quads
        // not yet there are polled again, which waits for the down
        // weights), then its down rows, while the routed h travels.
        uint32_t qp = 0;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int q = tid + 512 * m;
            if (q < a.S / 4) {
                if (tag_is(vq[m], ep))
                    *reinterpret_cast<uint2*>(&s_shb[2 * q]) = fp8x4_bf16((uint32_t)vq[m]);
                else
                    qp |= 1u << m;
            }
        }
        for (uint32_t polls = 0; __any(qp != 0u); ++polls) {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int q = tid + 512 * m;
                if ((qp >> m) & 1u) {
                    const unsigned long long v = get_tag(srcq + q);
                    if (tag_is(v, ep)) {
                        *reinterpret_cast<uint2*>(&s_shb[2 * q]) = fp8x4_bf16((uint32_t)v);
                        qp &= ~(1u << m);
                    }
                }
            }
            if (polls > kPollLimit) {
                if (lane == 0) atomicOr(flags, 1u);
                break;
            }
            if (__any(qp != 0u)) __builtin_amdgcn_s_sleep(1);
        }
        __syncthreads();
        const int nck2 = a.S / 16;
        float zsh[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < CD; ++c) {
                const int chr = lane + 64 * c, ch = min(chr, nck2 - 1);
                const uint4* hp = reinterpret_cast<const uint4*>(&s_shb[8 * ch]);
                const float q = fp8_chunk_bf16(qsd[p][c], hp[0], hp[1]);
                acc += chr < nck2 ? q : 0.f;
            }
            zsh[p] = seg_sum_last<64>(acc);
        }
        const float sc = a.sd_w * a.sd_in;
#pragma unroll
        for (int p = 0; p < 2; ++p)
            if (lane == 63 && sd0 + p < sd1) put_tag(a.z_tag + (uint32_t)(a.K * a.H + sd0 + p), zsh[p] * sc, ep);
    }
    if constexpr (A4) {
        // W4A4: the NVFP4 h of slots sl0 .. sl1 (one run of at most 1024
        // half blocks), thread t taking half blocks t and t + 512: its codes
        // and its block's scale, decoded exactly into LDS as fp32
        const int nhb = (sl1 - sl0 + 1) * a.I / 8, hb0 = sl0 * a.I / 8;
        const size_t per = (size_t)(RU / 8 + RU / 16);
        const unsigned long long* src = a.h_tag + rep * per;
        uint32_t pend = 0;
#pragma unroll
        for (int m = 0; m < 2; ++m)
            if ((int)tid + 512 * m < nhb) pend |= 5u << m;  // bit m: codes, bit m + 2: scale
        uint32_t cw[2] = {0u, 0u}, sw[2] = {0u, 0u};
        for (uint32_t polls = 0; __any(pend != 0u); ++polls) {
            unsigned long long v[4];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int hb = hb0 + (int)tid + 512 * m;
                v[m] = (pend >> m) & 1u ? get_tag(src + hb) : 0ull;
                v[m + 2] = (pend >> (m + 2)) & 1u ? get_tag(src + RU / 8 + hb / 2) : 0ull;
            }
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                if (((pend >> m) & 1u) && tag_is(v[m], ep)) {
                    cw[m] = (uint32_t)v[m];
                    pend &= ~(1u << m);
                }
                if (((pend >> (m + 2)) & 1u) && tag_is(v[m + 2], ep)) {
                    sw[m] = (uint32_t)v[m + 2];
                    pend &= ~(1u << (m + 2));
                }
            }
            if (polls > kPollLimit) {
                if (lane == 0) atomicOr(flags, 1u);
                break;
            }
            if (__any(pend != 0u)) __builtin_amdgcn_s_sleep(1);
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int t = (int)tid + 512 * m;
            if (t < nhb) {
                Nvfp4Half b;
                b.code = cw[m];
                b.sb = sw[m] & 0xffu;
                float f[8];
                nvfp4_dequant8(b, f);
                // as bf16 pairs (exact: at most 6 significant bits)
                uint32_t o[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    o[j] = (__float_as_uint(f[2 * j]) >> 16) | (__float_as_uint(f[2 * j + 1]) & 0xffff0000u);
                reinterpret_cast<uint4*>(s_h)[lds_pad_u128(t)] = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
    } else {
        // the slots sl0 .. sl1 are adjacent in the [K][I] layout, so their h
        // is one run of nh <= 2 * 4096 = 16 * 512 values
        const int nh = (sl1 - sl0 + 1) * a.I;
        const unsigned long long* src = a.h_tag + ((size_t)rep * a.K + sl0) * a.I;
        uint32_t pend = 0;
#pragma unroll
        for (int m = 0; m < 16; ++m)
            if ((int)tid + 512 * m < nh) pend |= 1u << m;
        for (uint32_t polls = 0; __any(pend != 0u); ++polls) {
            unsigned long long v[16];
#pragma unroll
            for (int m = 0; m < 16; ++m) v[m] = (pend >> m) & 1u ? get_tag(src + tid + 512 * m) : 0ull;
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                if (((pend >> m) & 1u) && tag_is(v[m], ep)) {
                    const int i = tid + 512 * m;
                    if constexpr (FMT == FMT_NVFP4) {
                        s_h[lds_pad_f32(i)] = tag_value(v[m]);
                    } else {
                        // int4: h as bf16 hi + lo halves (about 17 bits),
                        // each in the pair order of the nibble unpacking
                        const float hv = tag_value(v[m]);
                        const uint32_t hi = f32_to_bf16_rne(hv);
                        const uint32_t lo = f32_to_bf16_rne(hv - bf16_bits_to_f32(hi));
                        const int pi = (i & ~7) | ((i & 3) << 1) | ((i >> 2) & 1);
                        s_h16[lds_pad_u16(pi)] = (uint16_t)hi;
                        s_h16[kLdsH16Lo + lds_pad_u16(pi)] = (uint16_t)lo;
                    }
                    pend &= ~(1u << m);
                }
            }
            if (polls > kPollLimit) {
                if (lane == 0) atomicOr(flags, 1u);
                break;
            }
            if (__any(pend != 0u)) __builtin_amdgcn_s_sleep(1);
        }
    }
    // the down scales through LDS (every load of the wave is in by now)
    if (dwave) {
#pragma unroll
        for (int k = 0; k < C2; ++k) {
            uint32_t* d = reinterpret_cast<uint32_t*>(my_sc + dso16[k]);
            d[0] = dsc[k][0];
            d[1] = dsc[k][1];
            d[2] = dsc[k][2];
            d[3] = dsc[k][3];
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int p = 0; p < kDownRows; ++p) {
#pragma unroll
            for (int c = 0; c < C2; ++c)
                sd[p][c] = *reinterpret_cast<const uint16_t*>(my_sc + dsk + (uint32_t)p * dsb + dso[c]);
        }
    }
    Q4MOE_WAVE_MARK(2);
    __syncthreads();
    Q4MOE_PHASE(5);

    // ---- D: a wave computes z = w * g * (W_down h) for its 8 rows of slot
    // dslot (one block of code: each row waits only for its own weights),
    // sums the rows over the lanes together and publishes them with one
    // store.
    if (dwave) {
        float zp[kDownRows];  // this lane's part of each row
        if constexpr (A4) {
            // W4A4: h is exact in bf16, so one dot2 per weight pair
            uint32_t hb[C2][16];
#pragma unroll
            for (int c = 0; c < C2; ++c) {
                const int ch = min(lane * C2 + c, nchI - 1);
                // (a slot's h starts on a chunk boundary: I % 32 == 0)
                const uint4* hp = reinterpret_cast<const uint4*>(s_h) + 5 * ((dslot - sl0) * (a.I / 32) + ch);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint4 v = hp[k];
                    hb[c][4 * k + 0] = v.x;
                    hb[c][4 * k + 1] = v.y;
                    hb[c][4 * k + 2] = v.z;
                    hb[c][4 * k + 3] = v.w;
                }
            }
#pragma unroll
            for (int p = 0; p < kDownRows; ++p) {
                float zz = 0.f;
#pragma unroll
                for (int c = 0; c < C2; ++c) {
                    const bool chok = lane * C2 + c < nchI;
                    const f32x2 sp = e4m3fn_x2_f32(sd[p][c]);
                    const float s0 = chok ? sp[0] : 0.f, s1 = chok ? sp[1] : 0.f;
                    zz += nvfp4_chunk_bf16(qd[p][c], hb[c], s0, s1);
                }
                zp[p] = zz;
            }
        } else if constexpr (FMT == FMT_NVFP4) {
            float hv[C2][32];
#pragma unroll
            for (int c = 0; c < C2; ++c) {
                const int ch = min(lane * C2 + c, nchI - 1);
                const float4* hp = reinterpret_cast<const float4*>(&s_h[lds_pad_f32((dslot - sl0) * a.I + ch * 32)]);
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float4 v = hp[k];
                    hv[c][4 * k + 0] = v.x;
                    hv[c][4 * k + 1] = v.y;
                    hv[c][4 * k + 2] = v.z;
                    hv[c][4 * k + 3] = v.w;
                }
            }
#pragma unroll
            for (int p = 0; p < kDownRows; ++p) {
                float zz = 0.f;
#pragma unroll
                for (int c = 0; c < C2; ++c) {
                    const bool chok = lane * C2 + c < nchI;
                    const f32x2 sp = e4m3fn_x2_f32(sd[p][c]);
                    const float s0 = chok ? sp[0] : 0.f, s1 = chok ? sp[1] : 0.f;
                    zz += nvfp4_chunk_f32(qd[p][c], hv[c], s0, s1);
                }
                zp[p] = zz;
            }
        } else {
            // int4: a dot2 of the bf16 weights 136 + code with h's hi and
            // lo halves; 136 * sum(h) is taken off once per chunk
            uint32_t hq[C2][16], lq[C2][16];
            float hs[C2];
#pragma unroll
            for (int c = 0; c < C2; ++c) {
                const int ch = min(lane * C2 + c, nchI - 1);
                const int e = lds_pad_u16((dslot - sl0) * a.I + ch * 32);
                const uint4* hp = reinterpret_cast<const uint4*>(&s_h16[e]);
                const uint4* lp = reinterpret_cast<const uint4*>(&s_h16[kLdsH16Lo + e]);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint4 v = hp[k], w = lp[k];
                    hq[c][4 * k + 0] = v.x;
                    hq[c][4 * k + 1] = v.y;
                    hq[c][4 * k + 2] = v.z;
                    hq[c][4 * k + 3] = v.w;
                    lq[c][4 * k + 0] = w.x;
                    lq[c][4 * k + 1] = w.y;
                    lq[c][4 * k + 2] = w.z;
                    lq[c][4 * k + 3] = w.w;
                }
                float t = 0.f;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    t = dot2_bf16(as_bf16x2(hq[c][j]), as_bf16x2(0x3F803F80u), t);
                    t = dot2_bf16(as_bf16x2(lq[c][j]), as_bf16x2(0x3F803F80u), t);
                }
                hs[c] = 136.0f * t;
            }
#pragma unroll
            for (int p = 0; p < kDownRows; ++p) {
                float zz = 0.f;
#pragma unroll
                for (int c = 0; c < C2; ++c) {
                    const bool chok = lane * C2 + c < nchI;
                    const float sg = chok ? bf16_bits_to_f32(sd[p][c]) : 0.f;
                    zz = __builtin_fmaf(sg, int4_chunk_bf16_hl(qd[p][c], hq[c], lq[c]) - hs[c], zz);
                }
                zp[p] = zz;
            }
        }
        // the eight row sums over the 64 lanes at once: lane l ends with the
        // sum of row rows8_label(l)
        const float zs = rows8_sum(zp);
        const int rl = rows8_label(lane);
        const float wg = wsel[dslot] * gdn;
        if ((lane & 7) == 7 && drow0 + rl < a.H) put_tag(a.z_tag + (uint32_t)(dslot * a.H + drow0 + rl), wg * zs, ep);
    }
    Q4MOE_WAVE_MARK(3);
    Q4MOE_PHASE(6);

    // ---- C: block b of 64 rows is combined by workgroup b * grid / nblocks
    const int nb = (a.H + kRowBlock - 1) / kRowBlock;
    for (int b = wave; b < nb; b += kWaves) {
        if ((int)((long long)b * gridDim.x / nb) != (int)bid) continue;
        const int r = b * kRowBlock + lane;
        constexpr int NS = SH ? 9 : 8;       // routed slots, then the shared expert
        const int ns = a.K + (SH ? 1 : 0);
        float part[NS];
        uint32_t pend = 0;
        for (int s2 = 0; s2 < ns; ++s2) pend |= 1u << s2;
        if (r >= a.H) pend = 0;
        // every load of a poll leaves before any is waited for (rows and
        // slots clamped into the array, so the load count is fixed)
        const unsigned long long* zr = a.z_tag + min(r, a.H - 1);
        for (uint32_t polls = 0;; ++polls) {
            unsigned long long v[NS];
#pragma unroll
            for (int s2 = 0; s2 < NS; ++s2) v[s2] = get_tag(zr + (size_t)min(s2, ns - 1) * a.H);
#pragma unroll
            for (int s2 = 0; s2 < NS; ++s2) {
                if (((pend >> s2) & 1u) && tag_is(v[s2], ep)) {
                    part[s2] = tag_value(v[s2]);
                    pend &= ~(1u << s2);
                }
            }
            if (!__any(pend != 0u)) break;
            if (polls > kPollLimit) {
                if (lane == 0) atomicOr(flags, 1u);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        uint32_t yb = 0u;
        if (r < a.H) {
            float yv = 0.f;
#pragma unroll
            for (int s2 = 0; s2 < NS; ++s2)
                if (s2 < ns) yv += (pend >> s2) & 1u ? 0.f : part[s2];
            yb = f32_to_bf16_rne(yv);
            a.y32[r] = yv;
            a.y[r] = (uint16_t)yb;
        }
        if constexpr (STK) {
            if (sk.chain) {
                // y for the next layer of the chain: rows 2t, 2t + 1 as one
                // (two bf16, epoch) value, kReplicas copies
                const uint32_t yo = (uint32_t)__builtin_amdgcn_mov_dpp((int)yb, 0xB1, 0xF, 0xF, true);  // lane ^ 1
                if ((lane & 1) == 0 && r < a.H) {
                    const uint32_t pair = yb | (yo << 16);
#pragma unroll
                    for (int rp = 0; rp < kReplicas; ++rp)
                        put_tag(sk.y_tag + (size_t)rp * (a.H / 2) + r / 2, __uint_as_float(pair), ep);
                }
            } else if (lane < kReplicas) {
                // this block is combined (after its y stores)
                put_tag(sk.done_tag + (size_t)lane * 64 + b, 0.f, ep);
            }
        }
    }
    Q4MOE_PHASE(7);

    Q4MOE_PHASE(10);
}

// One layer for one token.
template <int FMT, int C, int C2, bool SH, bool A4>
__global__ __launch_bounds__(64 * kWaves, 1) void k_decode_fused(FusedArgs a) {
    // This call's epoch: one more than the last call's.  Each workgroup keeps
    // its own copy in word FW_EPOCH + b, which only workgroup b of each call
    // reads and writes; every call runs every workgroup once, so all copies
    // advance together and stay equal.  Every wave loads it and first uses it
    // after the router, so nothing waits for it here.
    const uint32_t ep =
        __hip_atomic_load(a.ctrl + FW_EPOCH + blockIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    fused_layer<FMT, C, C2, SH, A4, false>(a, ep, StackCtl{0, 0, nullptr, nullptr}, threadIdx.x, blockIdx.x);
}

// A stack of single-token layers of one shape in one launch, in order: layer
// l takes epoch e + 1 + l (e: the last epoch on this workspace), and from the
// second layer on each starts its routing only once the previous layer's y
// is complete on the device, the order of one launch per layer without the
// device's gap between launches.
template <int FMT, int C, int C2>
__global__ __launch_bounds__(64 * kWaves, 1) void k_decode_stack(StackArgs s) {
    const uint32_t ep0 = __hip_atomic_load(s.a.ctrl + FW_EPOCH + blockIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll 1
    for (int l = 0; l < s.n_layers; ++l) {
        FusedArgs a = s.a;
        const StackLayer& L = s.layer[l];
        a.wg = L.wg;
        a.bias = L.bias;
        a.x = L.x;
        a.upc = L.upc;
        a.ups = L.ups;
        a.upg = L.upg;
        a.dnc = L.dnc;
        a.dns = L.dns;
        a.dng = L.dng;
        a.y = L.y;
        a.ids_out = L.ids_out;
        a.w_out = L.w_out;
        // the thread and workgroup indices pass through an empty asm each
        // layer, so that nothing computed from them is hoisted out of the
        // loop and held in registers across the layers
        uint32_t tid = threadIdx.x, bid = blockIdx.x;
        asm volatile("" : "+v"(tid), "+s"(bid));
        fused_layer<FMT, C, C2, false, false, true>(a, ep0 + 1u + (uint32_t)l,
                                                    StackCtl{l, s.chain, s.y_tag, s.done_tag}, tid, bid);
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(s.a.ctrl + FW_EPOCH + blockIdx.x, ep0 + (uint32_t)s.n_layers, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace q4moe
