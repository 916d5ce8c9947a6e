// FP8 per-tensor W8A8 GEMV + argmax for up to four tokens: the MTP drafter's
// lm_head ("Quantization (PTQ + QAD)", MTP Drafter Precision: the lm_head the
// drafter shares is FP8; the precision table's FP8 lm_head).  Weights are
// E4M3FN bytes with one fp32 scale per tensor; the activations are coded to
// E4M3FN with a static fp32 input scale, as for the shared expert.
//
// v_mfma_f32_16x16x32_f16 with the weight rows as the 16-row operand and the
// tokens as the 16-column operand (columns past T are zero).  Every E4M3FN
// value is exact in fp16, so each product is exact and only the fp32
// accumulation rounds.  A wave owns a group of 16 rows at a time: lane
// (m, kq) loads bytes 64 j + 16 kq .. +15 of row m (k 64 j + 16 kq .. +15),
// in batches of eight pieces with batch b + 1 issued before batch b is
// computed, and MFMA step (j, d) sums k 64 j + 16 kq + 8 d .. +7 on both
// operands.  The activation codes' fp16 values sit in LDS, staged while the
// first weight batch is in flight.  Persistent grid: wave w of workgroup b
// takes groups b*4+w, stepping by 4*gridDim; each workgroup leaves its best
// (logit, row) key per token for k_argmax_reduce.
#pragma once

#include "q4moe_fused.hpp"

namespace q4moe {

struct Fp8GemvArgs {
    int rows, cols, T;
    const uint8_t* codes;       // [rows][cols] E4M3FN
    float wscale, iscale;
    const uint16_t* x;          // [T][cols] bf16
    float* logits;              // [T][rows]
    uint8_t* xq;                // [T][cols] tap: the activation codes
    unsigned long long* keys;   // [gridDim][T]
};

template <int NJ8, int NT, int P, typename F>
__device__ __forceinline__ f32x4g fp8_gemv_group(const uint8_t* codes, uint32_t r, int cols, const _Float16* xs,
                                                 int m16, int kq, F&& after_first_issue) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const uint32_t rc = r * (uint32_t)cols;
    constexpr int kB = 8;
    uint4 q[NJ8];
    auto issue = [&](int j0) {
#pragma unroll
        for (int j = j0; j < (j0 + kB < NJ8 ? j0 + kB : NJ8); ++j) {
            const bool ok = 64 * j + 16 * kq < cols;
            q[j] = ldg16(codes + (rc + (ok ? 64 * j + 16 * kq : cols - 16)));
        }
    };
    f32x4g acc = {0.f, 0.f, 0.f, 0.f};
    issue(0);
    __builtin_amdgcn_sched_barrier(0);
    after_first_issue();
#pragma unroll
    for (int j0 = 0; j0 < NJ8; j0 += kB) {
        __builtin_amdgcn_sched_barrier(0);
        if (j0 + kB < NJ8) issue(j0 + kB);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = j0; j < (j0 + kB < NJ8 ? j0 + kB : NJ8); ++j) {
            const bool ok = 64 * j + 16 * kq < cols;
            const uint32_t w4[4] = {q[j].x, q[j].y, q[j].z, q[j].w};
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                const h2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w4[2 * d], 1.0f, false);
                const h2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w4[2 * d], 1.0f, true);
                const h2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w4[2 * d + 1], 1.0f, false);
                const h2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w4[2 * d + 1], 1.0f, true);
                h8 wf = {p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
                if (!ok) wf = h8{0, 0, 0, 0, 0, 0, 0, 0};
                h8 xf = {0, 0, 0, 0, 0, 0, 0, 0};
                if (m16 < NT) xf = *reinterpret_cast<const h8*>(xs + m16 * P + 64 * j + 16 * kq + 8 * d);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf, xf, acc, 0, 0, 0);
            }
        }
    }
    return acc;
}

template <int NJ8, int T>
__global__ __launch_bounds__(256, 3) void k_gemv_fp8(Fp8GemvArgs a) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    constexpr int P = kGemvMaxCols + 8;
    static_assert(64 * (NJ8 - 1) + 16 * 3 + 8 + 8 <= P, "LDS reads stay in the row");
    __shared__ __attribute__((aligned(16))) _Float16 xs[T][P];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int cols = a.cols;
    // x -> E4M3FN codes of fl32(x / iscale) -> their exact fp16 values in
    // LDS (zeros past the row); workgroup 0 also stores the codes
    auto x_setup = [&] {
        const int per = cols / 8, total = T * per;
        for (int p = threadIdx.x; p < total; p += 256) {
            const int t = p / per, k0 = (p - t * per) * 8;
            const uint4 v = *reinterpret_cast<const uint4*>(a.x + (size_t)p * 8);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
            h8 hv;
            uint32_t cw[2] = {0u, 0u};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t c0 = fp8_act_code(bf16_bits_to_f32(w[d] & 0xffffu), a.iscale);
                const uint32_t c1 = fp8_act_code(bf16_bits_to_f32(w[d] >> 16), a.iscale);
                hv[2 * d] = (_Float16)e4m3fn_to_f32(c0);
                hv[2 * d + 1] = (_Float16)e4m3fn_to_f32(c1);
                cw[d >> 1] |= (c0 | (c1 << 8)) << (16 * (d & 1));
            }
            *reinterpret_cast<h8*>(&xs[t][k0]) = hv;
            if (blockIdx.x == 0 && a.xq) *reinterpret_cast<uint2*>(a.xq + (size_t)t * cols + k0) = make_uint2(cw[0], cw[1]);
        }
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll 1
            for (int k = cols + threadIdx.x; k < P; k += 256) xs[t][k] = (_Float16)0.f;
        __syncthreads();
    };
    const int m16 = lane & 15, kq = lane >> 4;
    const int n = m16;  // token column of this lane in the 16-column operand
    unsigned long long best = 0ull;
    const int groups = (a.rows + 15) / 16;
    // every wave takes part in x_setup's barrier: a wave without a group of
    // its own computes the last group and stores nothing
    int grp = blockIdx.x * 4 + wave;
    const int grp0 = grp < groups ? grp : groups - 1;
    f32x4g acc = fp8_gemv_group<NJ8, T, P>(a.codes, (uint32_t)min(grp0 * 16 + m16, a.rows - 1), cols, &xs[0][0],
                                           m16, kq, x_setup);
    for (; grp < groups; grp += gridDim.x * 4) {
        if (grp != blockIdx.x * 4 + wave)
            acc = fp8_gemv_group<NJ8, T, P>(a.codes, (uint32_t)min(grp * 16 + m16, a.rows - 1), cols, &xs[0][0], m16,
                                            kq, [] {});
        // lane holds rows grp*16 + 4 kq + r of token n
        if (n < T) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int row = grp * 16 + 4 * kq + rr;
                if (row < a.rows) {
                    const float l = acc[rr] * a.wscale * a.iscale;
                    a.logits[(size_t)n * a.rows + row] = l;
                    const unsigned long long key =
                        ((unsigned long long)f32_order(l) << 32) | (unsigned long long)(0xffffffffu - (uint32_t)row);
                    best = key > best ? key : best;
                }
            }
        }
    }
    // per token: the lanes n, n+16, n+32, n+48 of every wave, then the block
    {
        unsigned long long o = __shfl_xor(best, 16, 64);
        best = o > best ? o : best;
        o = __shfl_xor(best, 32, 64);
        best = o > best ? o : best;
    }
    __shared__ unsigned long long sbest[4][T];
    if (lane < T) sbest[wave][lane] = best;
    __syncthreads();
    if (threadIdx.x < T) {
        unsigned long long v = 0ull;
        for (int wv = 0; wv < 4; ++wv) v = sbest[wv][threadIdx.x] > v ? sbest[wv][threadIdx.x] : v;
        a.keys[(size_t)blockIdx.x * T + threadIdx.x] = v;
    }
}

}  // namespace q4moe
