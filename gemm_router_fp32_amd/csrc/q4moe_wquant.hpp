// NVFP4 weight quantizer on gfx950: bf16 weights -> E2M1 codes, an E4M3FN
// scale per block of 16 and an fp32 scale per tensor ("Let's optimize
// Nemotron 3.5 Lightning - a worklog", Step 1: NVFP4 weights; the recipe
// table's weight-scale selection: max-based, or an MSE per-block search over
// FP8 scale values).
//
// Definitions (the same as the decoders use: weight = e2m1 * e4m3(b) * g):
//   g = fl32(amax / 2688), 2688 = 6 * 448 (1 for an all-zero tensor);
//   eff(b) = fl32(e4m3(b) * g); the code of w under b is the E2M1 magnitude
//   nearest the exact quotient |w| / eff(b), ties to the even code,
//   saturating at 6, with w's sign bit;
//   max-based: b = E4M3FN nearest-even of fl32(bamax / fl32(6 g));
//   MSE: b in 0x01..0x7E minimising the block's squared error, summed in
//   element order with every step rounded to fp32 (no fused operations), the
//   lowest byte among equal minima; an all-zero block takes b = 0.
//
// Two launches: per-workgroup maxima, then one thread per block of 16 (each
// workgroup first reduces the maxima to g).  The comparisons |w| against
// mid * eff are exact: the sign of fma(mid, eff, -|w|) is the sign of the
// exact difference, and it is zero only when the difference is.
#pragma once

#include "q4moe_device.hpp"

namespace q4moe {

constexpr int kWqMaxBlocks = 1024;  // workgroups of the maximum pass

__global__ __launch_bounds__(256) void k_wq_amax(const uint4* w, size_t n8, float* partial) {
    float m = 0.f;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (size_t)gridDim.x * 256) {
        const uint4 v = w[i];
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k)
            m = fmaxf(m, fmaxf(fabsf(bf16_bits_to_f32(d[k] & 0xffffu)), fabsf(bf16_bits_to_f32(d[k] >> 16))));
    }
    __shared__ float s_m[4];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if ((threadIdx.x & 63) == 0) s_m[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) partial[blockIdx.x] = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
}

// Magnitude code of the exact quotient mag / eff (binary search over the
// midpoints; a tie goes up at an odd midpoint, down at an even one).
__device__ __forceinline__ uint32_t wq_code(float mag, float eff) {
    const float r3 = __builtin_fmaf(1.75f, eff, -mag);  // mid 3
    const uint32_t b2 = r3 <= 0.f ? 1u : 0u;
    const float r1 = __builtin_fmaf(b2 ? 3.5f : 0.75f, eff, -mag);  // mid 5 or mid 1
    const uint32_t b1 = r1 <= 0.f ? 1u : 0u;
    const float m0 = b2 ? (b1 ? 5.0f : 2.5f) : (b1 ? 1.25f : 0.25f);  // mid 6, 4, 2 or 0
    const uint32_t b0 = __builtin_fmaf(m0, eff, -mag) < 0.f ? 1u : 0u;
    return (b2 << 2) | (b1 << 1) | b0;
}

__device__ __forceinline__ float wq_grid(uint32_t c) {
    return fp4x2_f32<0>(c)[0];  // E2M1 magnitude of code c (< 8)
}

struct WqArgs {
    const uint4* w;        // bf16 [rows][cols], as 16-byte pieces
    size_t nblocks;        // rows * cols / 16
    const float* partial;  // [npartial] maxima of the first pass
    int npartial;
    int mse;
    uint8_t* codes;        // [nblocks][8]
    uint8_t* scales;       // [nblocks]
    float* gscale;         // [1]
};

template <bool MSE>
__global__ __launch_bounds__(256) void k_wq_quant(WqArgs a) {
    // every product and sum below rounds on its own (the error that decides
    // the MSE scale is defined that way; fused forms would round differently)
#pragma clang fp contract(off)
    __shared__ float s_g;
    if (threadIdx.x < 64) {
        float m = 0.f;
        for (int i = threadIdx.x; i < a.npartial; i += 64) m = fmaxf(m, a.partial[i]);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
        if (threadIdx.x == 0) {
            const float g = m > 0.f ? __fdiv_rn(m, 2688.0f) : 1.0f;
            s_g = g;
            if (blockIdx.x == 0) *a.gscale = g;
        }
    }
    __syncthreads();
    const float g = s_g;
    const size_t blk = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (blk >= a.nblocks) return;
    const uint4 v0 = a.w[2 * blk], v1 = a.w[2 * blk + 1];
    const uint32_t d[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    float mag[16];
    uint32_t sgn = 0;
    float bamax = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        mag[2 * k] = fabsf(bf16_bits_to_f32(d[k] & 0xffffu));
        mag[2 * k + 1] = fabsf(bf16_bits_to_f32(d[k] >> 16));
        sgn |= ((d[k] >> 15) & 1u) << (2 * k);
        sgn |= ((d[k] >> 31) & 1u) << (2 * k + 1);
        bamax = fmaxf(bamax, fmaxf(mag[2 * k], mag[2 * k + 1]));
    }
    uint32_t b = 0;
    if (bamax > 0.f) {
        b = e4m3fn_rne_sat(__fdiv_rn(bamax, 6.0f * g));
        if constexpr (MSE) {
            float best = __builtin_inff();
            for (uint32_t c = 1; c <= 0x7Eu; ++c) {
                const float eff = e4m3fn_to_f32(c) * g;
                float e = 0.f;
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    const float q = wq_grid(wq_code(mag[k], eff)) * eff;
                    const float df = mag[k] - q;
                    const float sq = df * df;
                    e = e + sq;
                }
                if (e < best) {
                    best = e;
                    b = c;
                }
            }
        }
    }
    const float eff = e4m3fn_to_f32(b) * g;
    uint32_t cw[2] = {0u, 0u};
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const uint32_t c = (b == 0u ? 0u : wq_code(mag[k], eff)) | (((sgn >> k) & 1u) << 3);
        cw[k >> 3] |= c << (4 * (k & 7));
    }
    *reinterpret_cast<uint2*>(a.codes + 8 * blk) = make_uint2(cw[0], cw[1]);
    a.scales[blk] = (uint8_t)b;
}

}  // namespace q4moe
