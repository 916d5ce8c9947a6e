// FP8 per-tensor W8A8 shared expert for 2-4 tokens ("Let's optimize Nemotron
// 3.5 Lightning - a worklog", Step 3: shared experts to FP8; the W4A4 model
// card's precision table), beside the small-batch routed kernels: every token
// runs through the shared expert, so each weight row is read once and meets
// all tokens.  Three launches: x coded to E4M3FN with the static input scale;
// up, u = (W x) s_w s_in, h = relu(u)^2, h coded the same way; down,
// z = (W h) s_w s_in.  One wave per row (lane l takes 16-byte chunks
// l + 64 c), 4 rows per wave and 16 per workgroup, all weight loads issued
// before the activation codes are staged in LDS as bf16; the products are
// exact (fp8 values are exact in bf16), the sums fp32.
#pragma once

#include "q4moe_fused.hpp"

namespace q4moe {

constexpr int kShRowsPerWg = 16;

struct SharedSmallArgs {
    int T, H, S;
    const uint16_t* x;        // [T][H] bf16
    const uint8_t* shu;       // [S][H] E4M3FN
    const uint8_t* shd;       // [H][S] E4M3FN
    float su_w, su_in, sd_w, sd_in;
    uint8_t* xq;              // [T][H] tap: x codes
    float* h;                 // [T][S] tap: relu(u)^2
    uint8_t* hq;              // [T][S] h codes (the down kernel's input)
    float* z;                 // [T][H] the shared expert's output
};

// A wave's four rows [row0, row0 + 4) of W [rows][cols] (fp8), all issued
// before anything else so that the coding of the activations overlaps them;
// rows and chunks past the end are clamped (their products are dropped).
template <int CH>
__device__ __forceinline__ void fp8_rows_load(const uint8_t* w, int row0, int rows, int cols, uint4 (&q)[4][CH]) {
    const int lane = threadIdx.x & 63;
    const int nck = cols / 16;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const size_t row = (size_t)min(row0 + k, rows - 1);
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int ch = min(lane + 64 * c, nck - 1);
            q[k][c] = ldg16_stream(w + (row * cols + (size_t)ch * 16));
        }
    }
}

// The four rows against the T activation rows act [T][cols] (bf16 pairs in
// LDS, pitch cols / 2 dwords); lane 63 returns out[k][t] (0 for t >= T).
template <int CH>
__device__ __forceinline__ void fp8_rows_dot(const uint4 (&q)[4][CH], int cols, const uint32_t* act, int T,
                                             float (&out)[4][4]) {
    const int lane = threadIdx.x & 63;
    const int nck = cols / 16;
    float acc[4][4] = {};
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int chr = lane + 64 * c, ch = min(chr, nck - 1);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (t < T) {
                const uint4* ap = reinterpret_cast<const uint4*>(act + (size_t)t * (cols / 2) + 8 * ch);
                const uint4 a0 = ap[0], a1 = ap[1];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float p = fp8_chunk_bf16(q[k][c], a0, a1);
                    acc[k][t] += chr < nck ? p : 0.f;
                }
            }
        }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int t = 0; t < 4; ++t) out[k][t] = t < T ? seg_sum_last<64>(acc[k][t]) : 0.f;
}

// The sixteen sums held by lane 63 spread over lanes 0..15 (lane 4 k + t
// takes out[k][t]), so that the epilogue runs on 16 lanes at once.
__device__ __forceinline__ float spread_sums(const float (&out)[4][4]) {
    const int lane = threadIdx.x & 63;
    float mine = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(out[k][t]), 63));
            mine = lane == 4 * k + t ? v : mine;
        }
    return mine;
}

// x of every token coded to E4M3FN once, before the up kernel (coding it in
// every up workgroup costs more than the weights' read): grid
// ceil(T H / 8 / 256), 256 threads, one 16-byte piece of x per thread.
__global__ __launch_bounds__(256) void k_shared_xcode(SharedSmallArgs a) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= a.T * a.H / 8) return;
    const uint4 v = *reinterpret_cast<const uint4*>(a.x + 8 * (size_t)i);
    const uint32_t in[4] = {v.x, v.y, v.z, v.w};
    uint32_t cw[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t bits = (e & 1) ? in[e >> 1] >> 16 : in[e >> 1] & 0xffffu;
        cw[e >> 2] |= fp8_act_code(bf16_bits_to_f32(bits), a.su_in) << (8 * (e & 3));
    }
    *reinterpret_cast<uint2*>(a.xq + 8 * (size_t)i) = make_uint2(cw[0], cw[1]);
}

// T rows of `cols` E4M3FN codes -> bf16 pairs in LDS (pitch cols / 2
// dwords), in 16-byte pieces, at most 4 per thread (4 x 4096 / 16 / 256),
// all loaded before any is decoded.
__device__ __forceinline__ void stage_codes_bf16(const uint8_t* codes, int T, int cols, uint32_t* dst) {
    const int n16 = T * cols / 16;
    uint4 cv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int i = min((int)threadIdx.x + 256 * j, n16 - 1);
        cv[j] = *reinterpret_cast<const uint4*>(codes + 16 * (size_t)i);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int i = threadIdx.x + 256 * j;
        if (i >= n16) break;
        const uint2 b0 = fp8x4_bf16(cv[j].x), b1 = fp8x4_bf16(cv[j].y), b2 = fp8x4_bf16(cv[j].z),
                    b3 = fp8x4_bf16(cv[j].w);
        uint4* d = reinterpret_cast<uint4*>(dst + 8 * (size_t)i);
        d[0] = make_uint4(b0.x, b0.y, b1.x, b1.y);
        d[1] = make_uint4(b2.x, b2.y, b3.x, b3.y);
    }
}

// up: grid ceil(S / 16), 256 threads (4 waves x 4 rows)
template <int CH>
__global__ __launch_bounds__(256) void k_shared_up(SharedSmallArgs a) {
    __shared__ __attribute__((aligned(16))) uint32_t s_x[4 * 4096 / 2];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row0 = blockIdx.x * kShRowsPerWg + wave * 4;
    uint4 q[4][CH];
    fp8_rows_load<CH>(a.shu, row0, a.S, a.H, q);
    stage_codes_bf16(a.xq, a.T, a.H, s_x);
    __syncthreads();
    float u[4][4];
    fp8_rows_dot<CH>(q, a.H, s_x, a.T, u);
    const float sc = a.su_w * a.su_in;
    const float um = spread_sums(u);
    const int row = row0 + (lane >> 2), t = lane & 3;
    if (lane < 16 && t < a.T && row < a.S) {
        const float r = fmaxf(um * sc, 0.f), hv = r * r;
        a.h[(size_t)t * a.S + row] = hv;
        a.hq[(size_t)t * a.S + row] = (uint8_t)fp8_act_code(hv, a.sd_in);
    }
}

// down: grid ceil(H / 16), 256 threads; the h codes of every token into LDS
// (as bf16), then z = (W h) s_w s_in
template <int CH>
__global__ __launch_bounds__(256) void k_shared_down(SharedSmallArgs a) {
    __shared__ __attribute__((aligned(16))) uint32_t s_h[4 * 4096 / 2];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row0 = blockIdx.x * kShRowsPerWg + wave * 4;
    uint4 q[4][CH];
    fp8_rows_load<CH>(a.shd, row0, a.H, a.S, q);
    stage_codes_bf16(a.hq, a.T, a.S, s_h);
    __syncthreads();
    float zz[4][4];
    fp8_rows_dot<CH>(q, a.S, s_h, a.T, zz);
    const float sc = a.sd_w * a.sd_in;
    const float zm = spread_sums(zz);
    const int row = row0 + (lane >> 2), t = lane & 3;
    if (lane < 16 && t < a.T && row < a.H) a.z[(size_t)t * a.H + row] = zm * sc;
}

}  // namespace q4moe
