// FP8 per-tensor W8A8 shared expert for 2-4 tokens ("Let's optimize Nemotron
// 3.5 Lightning - a worklog", Step 3: shared experts to FP8; the W4A4 model
// card's precision table), beside the small-batch routed kernels: every token
// runs through the shared expert, so each weight row is read once and meets
// all tokens.  Up: x coded to E4M3FN with the static input scale (each
// workgroup codes all tokens' x into LDS as bf16), u = (W x) s_w s_in,
// h = relu(u)^2, h coded the same way; down: z = (W h) s_w s_in.  One wave
// per row (lane l takes 16-byte chunks l + 64 c), 16 rows per workgroup; the
// products are exact (fp8 values are exact in bf16), the sums fp32.
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

// rows [16 b, 16 b + 16) of W [rows][cols] (fp8) against the T activation
// rows act [T][cols] (bf16 pairs in LDS, pitch cols / 2 dwords); lane 63 of
// each wave returns the T sums of its row in out[t]
template <int CH>
__device__ __forceinline__ void fp8_rows_dot(const uint8_t* w, int row, int cols, const uint32_t* act, int T,
                                             float (&out)[4]) {
    const int lane = threadIdx.x & 63;
    const int nck = cols / 16;
    uint4 q[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int ch = min(lane + 64 * c, nck - 1);
        q[c] = ldg16_stream(w + ((size_t)row * cols + (size_t)ch * 16));
    }
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int chr = lane + 64 * c, ch = min(chr, nck - 1);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (t < T) {
                const uint4* ap = reinterpret_cast<const uint4*>(act + (size_t)t * (cols / 2) + 8 * ch);
                const float p = fp8_chunk_bf16(q[c], ap[0], ap[1]);
                acc[t] += chr < nck ? p : 0.f;
            }
        }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) out[t] = seg_sum_last<64>(acc[t]);
}

// x of every token coded to E4M3FN (bf16 of the codes into LDS); workgroup
// (0) also stores the codes
__device__ __forceinline__ void code_rows_fp8(const uint16_t* src, int T, int cols, float s_in, uint32_t* dst,
                                              uint8_t* tap, bool write_tap) {
    const int n8 = T * cols / 8;
    for (int i = threadIdx.x; i < n8; i += blockDim.x) {
        const uint4 v = *reinterpret_cast<const uint4*>(src + 8 * (size_t)i);
        const uint32_t in[4] = {v.x, v.y, v.z, v.w};
        uint32_t cw[2] = {0u, 0u};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t bits = (j & 1) ? in[j >> 1] >> 16 : in[j >> 1] & 0xffffu;
            cw[j >> 2] |= fp8_act_code(bf16_bits_to_f32(bits), s_in) << (8 * (j & 3));
        }
        const uint2 b0 = fp8x4_bf16(cw[0]), b1 = fp8x4_bf16(cw[1]);
        *reinterpret_cast<uint4*>(dst + 4 * (size_t)i) = make_uint4(b0.x, b0.y, b1.x, b1.y);
        if (write_tap) *reinterpret_cast<uint2*>(tap + 8 * (size_t)i) = make_uint2(cw[0], cw[1]);
    }
}

// up: grid ceil(S / 16), 256 threads (4 waves x 4 rows)
template <int CH>
__global__ __launch_bounds__(256) void k_shared_up(SharedSmallArgs a) {
    __shared__ __attribute__((aligned(16))) uint32_t s_x[4 * 4096 / 2];
    code_rows_fp8(a.x, a.T, a.H, a.su_in, s_x, a.xq, blockIdx.x == 0);
    __syncthreads();
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const float sc = a.su_w * a.su_in;
#pragma unroll 1
    for (int k = 0; k < kShRowsPerWg / 4; ++k) {
        const int row = blockIdx.x * kShRowsPerWg + wave * (kShRowsPerWg / 4) + k;
        float u[4];
        fp8_rows_dot<CH>(a.shu, min(row, a.S - 1), a.H, s_x, a.T, u);
        if (lane == 63 && row < a.S) {
            for (int t = 0; t < a.T; ++t) {
                const float r = fmaxf(u[t] * sc, 0.f), hv = r * r;
                a.h[(size_t)t * a.S + row] = hv;
                a.hq[(size_t)t * a.S + row] = (uint8_t)fp8_act_code(hv, a.sd_in);
            }
        }
    }
}

// down: grid ceil(H / 16), 256 threads; the h codes of every token into LDS
// (as bf16), then z = (W h) s_w s_in
template <int CH>
__global__ __launch_bounds__(256) void k_shared_down(SharedSmallArgs a) {
    __shared__ __attribute__((aligned(16))) uint32_t s_h[4 * 4096 / 2];
    const int n4 = a.T * a.S / 4;
    for (int i = threadIdx.x; i < n4; i += blockDim.x) {
        const uint2 b = fp8x4_bf16(*reinterpret_cast<const uint32_t*>(a.hq + 4 * (size_t)i));
        *reinterpret_cast<uint2*>(s_h + 2 * (size_t)i) = b;
    }
    __syncthreads();
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const float sc = a.sd_w * a.sd_in;
#pragma unroll 1
    for (int k = 0; k < kShRowsPerWg / 4; ++k) {
        const int row = blockIdx.x * kShRowsPerWg + wave * (kShRowsPerWg / 4) + k;
        float zz[4];
        fp8_rows_dot<CH>(a.shd, min(row, a.H - 1), a.S, s_h, a.T, zz);
        if (lane == 63 && row < a.H)
            for (int t = 0; t < a.T; ++t) a.z[(size_t)t * a.H + row] = zz[t] * sc;
    }
}

}  // namespace q4moe
