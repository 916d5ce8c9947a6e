// Device helpers shared by the libq4moe kernels (gfx950, wave64).
//
// Element formats ("Let's optimize Nemotron 3.5 Lightning - a worklog",
// Step 1: NVFP4 with one scale per 16 weights; "NVIDIA-Nemotron-3.5-
// Lightning-30B-A3B-W4A16" README, What was changed: int4, group 64,
// symmetric): E2M1 codes are decoded by the gfx950 FP4 conversion
// instructions, E4M3FN scale bytes and int4 nibbles by integer arithmetic.
#pragma once

#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

namespace q4moe {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Element decoding
// ---------------------------------------------------------------------------

// E4M3FN byte -> fp32, exact: gfx950's fp8 converts use the OCP E4M3FN
// encoding (bias 7, subnormals m * 2^-9, S.1111.111 = NaN, no infinities),
// and with scale 1 the conversion is exact.  One instruction, no branches.
__device__ __forceinline__ float e4m3fn_to_f32(uint32_t b) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(b & 0xffu, 1.0f, false)[0];
}

// E4M3FN byte nearest (ties to even) to a finite d >= 0, saturating at 448.
__device__ __forceinline__ uint32_t e4m3fn_rne_sat(float d) {
    if (!(d < 448.0f)) return 0x7Eu;  // [448, inf) and NaN
    if (d < 0.015625f) {              // below 2^-6: subnormal steps of 2^-9
        return (uint32_t)__builtin_rintf(d * 512.0f);  // exact scaling; 8 -> 0x08 = 2^-6
    }
    const uint32_t u = __float_as_uint(d);
    int e = (int)(u >> 23) - 127;  // -6 .. 8
    uint32_t m = (u >> 20) & 7u;
    const uint32_t rem = u & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (m & 1u))) ++m;
    if (m == 8u) {
        m = 0u;
        ++e;
    }
    const uint32_t b = ((uint32_t)(e + 7) << 3) | m;
    return b > 0x7Eu ? 0x7Eu : b;
}

// Bytes 0 and 1 of v (two E4M3FN scales) -> fp32 pair, exact.
__device__ __forceinline__ f32x2 e4m3fn_x2_f32(uint32_t v) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v, 1.0f, false);
}

// Two E2M1 codes (byte `sel` of v: low nibble = first element) -> fp32 pair.
template <int sel>
__device__ __forceinline__ f32x2 fp4x2_f32(uint32_t v) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, sel);
}

// The E2M1 code of |v| on the grid scaled by s is the number of midpoints
// t_j = mids_j * s (exact: mids have at most 3 significant bits) that |v|
// passes, a tie going to the even code: up at an odd j, down at an even j.
// The thresholds increase, so three comparisons find the count (a binary
// search: j = 3, then 1 or 5, then 0, 2, 4 or 6).  Scale 0 gives code 0 for
// every value: the thresholds are then NaN and every comparison is false
// (as for a NaN value).
struct E2m1Thresholds {
    float t[7];
};
__device__ __forceinline__ E2m1Thresholds e2m1_thresholds(float s) {
    const float sc = s == 0.f ? __builtin_nanf("") : s;
    return {{0.25f * sc, 0.75f * sc, 1.25f * sc, 1.75f * sc, 2.5f * sc, 3.5f * sc, 5.0f * sc}};
}
__device__ __forceinline__ uint32_t e2m1_code(float mag, const E2m1Thresholds& th) {
    const uint32_t b2 = mag >= th.t[3] ? 1u : 0u;
    const uint32_t b1 = mag >= (b2 ? th.t[5] : th.t[1]) ? 1u : 0u;
    const float tl = b2 ? (b1 ? th.t[6] : th.t[4]) : (b1 ? th.t[2] : th.t[0]);
    const uint32_t b0 = mag > tl ? 1u : 0u;
    return (b2 << 2) | (b1 << 1) | b0;
}

// NVFP4 quantization of one block of 16 values (the activation quantizer:
// scale byte = E4M3FN nearest-even of fl32(amax / 6), saturating at 448;
// codes = nearest E2M1 of |v| / scale, ties to the even code, sign kept),
// codes packed low nibble first; and the block's dequantized values
// e2m1 * e4m3 (at most 6 significant bits: exact in fp32 and in bf16).
struct Nvfp4Block {
    uint32_t sb;
    uint32_t code[2];
};
__device__ __forceinline__ Nvfp4Block nvfp4_quant16(const float (&v)[16]) {
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) amax = fmaxf(amax, fabsf(v[k]));
    Nvfp4Block b;
    b.sb = e4m3fn_rne_sat(__fdiv_rn(amax, 6.0f));
    const E2m1Thresholds th = e2m1_thresholds(e4m3fn_to_f32(b.sb));
    b.code[0] = b.code[1] = 0u;
#pragma unroll
    for (int k = 0; k < 16; ++k)
        b.code[k >> 3] |= (e2m1_code(fabsf(v[k]), th) | ((__float_as_uint(v[k]) >> 31) << 3)) << (4 * (k & 7));
    return b;
}
// The same for half a block per lane: lanes 2k and 2k + 1 hold the two
// halves of one block (and are both active); the block maximum comes from
// the partner lane (quad_perm [1,0,3,2]).  code packs the lane's 8 codes.
struct Nvfp4Half {
    uint32_t sb, code;
};
__device__ __forceinline__ Nvfp4Half nvfp4_quant8_pair(const float (&v)[8]) {
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(v[k]));
    amax = fmaxf(amax, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, amax), 0xB1, 0xF, 0xF, true)));
    Nvfp4Half b;
    b.sb = e4m3fn_rne_sat(__fdiv_rn(amax, 6.0f));
    const E2m1Thresholds th = e2m1_thresholds(e4m3fn_to_f32(b.sb));
    b.code = 0u;
#pragma unroll
    for (int k = 0; k < 8; ++k) b.code |= (e2m1_code(fabsf(v[k]), th) | ((__float_as_uint(v[k]) >> 31) << 3)) << (4 * k);
    return b;
}
__device__ __forceinline__ void nvfp4_dequant8(const Nvfp4Half& b, float (&out)[8]) {
    const float s = e4m3fn_to_f32(b.sb);
    const f32x2 p[4] = {fp4x2_f32<0>(b.code), fp4x2_f32<1>(b.code), fp4x2_f32<2>(b.code), fp4x2_f32<3>(b.code)};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        out[2 * j] = p[j][0] * s;
        out[2 * j + 1] = p[j][1] * s;
    }
}
__device__ __forceinline__ void nvfp4_dequant16(const Nvfp4Block& b, float (&out)[16]) {
    const float s = e4m3fn_to_f32(b.sb);
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        const f32x2 p[4] = {fp4x2_f32<0>(b.code[w]), fp4x2_f32<1>(b.code[w]), fp4x2_f32<2>(b.code[w]),
                            fp4x2_f32<3>(b.code[w])};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            out[8 * w + 2 * j] = p[j][0] * s;
            out[8 * w + 2 * j + 1] = p[j][1] * s;
        }
    }
}


// Two E2M1 codes -> bf16 pair (every E2M1 value is exact in bf16).
template <int sel>
__device__ __forceinline__ bf16x2 fp4x2_bf16(uint32_t v) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, sel);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits) { return __uint_as_float(bits << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

__device__ __forceinline__ float dot2_bf16(bf16x2 a, bf16x2 b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}

// ---------------------------------------------------------------------------
// Cross-lane sums (DPP inside rows of 16 lanes, then lane permutes)
// ---------------------------------------------------------------------------

template <int ctrl>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), ctrl, 0xF, 0xF, true));
}

// Row-broadcast DPP step: rows in row_mask receive `src` from the row
// broadcast (row_bcast:15 = lane 15 of the row below, row_bcast:31 = lane 31),
// the others receive 0.
template <int ctrl, int row_mask>
__device__ __forceinline__ float dpp_bcast(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, row_mask, 0xF,
                                                                 false));
}

// Sum over aligned segments of SEG lanes (32 or 64) using DPP only; the sum
// lands in the LAST lane of each segment (lane 31 / 63), other lanes hold
// partial sums.
template <int SEG>
__device__ __forceinline__ float seg_sum_last(float v) {
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp<0x124>(v);  // row_ror:4
    v += dpp<0x128>(v);  // row_ror:8   (every lane: its row's sum)
    v += dpp_bcast<0x142, 0xA>(v);  // rows 1, 3 += rows 0, 2
    if constexpr (SEG == 64) v += dpp_bcast<0x143, 0x8>(v);  // row 3 += lane 31
    return v;
}

// Sum over aligned segments of SEG lanes (SEG in {16, 32, 64}); every lane of
// a segment receives the segment's sum.
template <int SEG>
__device__ __forceinline__ float seg_sum(float v) {
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp<0x124>(v);  // row_ror:4
    v += dpp<0x128>(v);  // row_ror:8
    if constexpr (SEG >= 32) v += __shfl_xor(v, 16, 64);
    if constexpr (SEG >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

// ---------------------------------------------------------------------------
// One 16-byte chunk (32 consecutive elements of a row) times activations.
// ---------------------------------------------------------------------------

// NVFP4 chunk . bf16 activations.  q: 4 code dwords; xa: 16 bf16 pairs
// (natural order: pair j = elements 2j, 2j+1); s0/s1: the two block scales.
__device__ __forceinline__ float nvfp4_chunk_bf16(const uint4 q, const uint32_t* xa, float s0, float s1) {
    float p0 = 0.f, p1 = 0.f;
    p0 = dot2_bf16(fp4x2_bf16<0>(q.x), as_bf16x2(xa[0]), p0);
    p0 = dot2_bf16(fp4x2_bf16<1>(q.x), as_bf16x2(xa[1]), p0);
    p0 = dot2_bf16(fp4x2_bf16<2>(q.x), as_bf16x2(xa[2]), p0);
    p0 = dot2_bf16(fp4x2_bf16<3>(q.x), as_bf16x2(xa[3]), p0);
    p0 = dot2_bf16(fp4x2_bf16<0>(q.y), as_bf16x2(xa[4]), p0);
    p0 = dot2_bf16(fp4x2_bf16<1>(q.y), as_bf16x2(xa[5]), p0);
    p0 = dot2_bf16(fp4x2_bf16<2>(q.y), as_bf16x2(xa[6]), p0);
    p0 = dot2_bf16(fp4x2_bf16<3>(q.y), as_bf16x2(xa[7]), p0);
    p1 = dot2_bf16(fp4x2_bf16<0>(q.z), as_bf16x2(xa[8]), p1);
    p1 = dot2_bf16(fp4x2_bf16<1>(q.z), as_bf16x2(xa[9]), p1);
    p1 = dot2_bf16(fp4x2_bf16<2>(q.z), as_bf16x2(xa[10]), p1);
    p1 = dot2_bf16(fp4x2_bf16<3>(q.z), as_bf16x2(xa[11]), p1);
    p1 = dot2_bf16(fp4x2_bf16<0>(q.w), as_bf16x2(xa[12]), p1);
    p1 = dot2_bf16(fp4x2_bf16<1>(q.w), as_bf16x2(xa[13]), p1);
    p1 = dot2_bf16(fp4x2_bf16<2>(q.w), as_bf16x2(xa[14]), p1);
    p1 = dot2_bf16(fp4x2_bf16<3>(q.w), as_bf16x2(xa[15]), p1);
    return p0 * s0 + p1 * s1;
}

// NVFP4 chunk . fp32 activations (h of the down projection).
template <int sel>
__device__ __forceinline__ float fp4_pair_fma(uint32_t v, const float* h, float acc) {
    const f32x2 w = fp4x2_f32<sel>(v);
    acc = __builtin_fmaf(w.x, h[2 * sel], acc);
    return __builtin_fmaf(w.y, h[2 * sel + 1], acc);
}

__device__ __forceinline__ float nvfp4_chunk_f32(const uint4 q, const float* h, float s0, float s1) {
    float p0 = 0.f, p1 = 0.f;
    p0 = fp4_pair_fma<0>(q.x, h + 0, p0);
    p0 = fp4_pair_fma<1>(q.x, h + 0, p0);
    p0 = fp4_pair_fma<2>(q.x, h + 0, p0);
    p0 = fp4_pair_fma<3>(q.x, h + 0, p0);
    p0 = fp4_pair_fma<0>(q.y, h + 8, p0);
    p0 = fp4_pair_fma<1>(q.y, h + 8, p0);
    p0 = fp4_pair_fma<2>(q.y, h + 8, p0);
    p0 = fp4_pair_fma<3>(q.y, h + 8, p0);
    p1 = fp4_pair_fma<0>(q.z, h + 16, p1);
    p1 = fp4_pair_fma<1>(q.z, h + 16, p1);
    p1 = fp4_pair_fma<2>(q.z, h + 16, p1);
    p1 = fp4_pair_fma<3>(q.z, h + 16, p1);
    p1 = fp4_pair_fma<0>(q.w, h + 24, p1);
    p1 = fp4_pair_fma<1>(q.w, h + 24, p1);
    p1 = fp4_pair_fma<2>(q.w, h + 24, p1);
    p1 = fp4_pair_fma<3>(q.w, h + 24, p1);
    return p0 * s0 + p1 * s1;
}

// The nibbles in bits 3..0 and 19..16 of v (two's complement codes c) as
// the bf16 pair 136 + c: the code's sign bit flipped gives the offset-binary
// c + 8 under the exponent of 128, in one and-xor.
__device__ __forceinline__ bf16x2 int4x2_bf16(uint32_t v) {
    return as_bf16x2((v & 0x000F000Fu) ^ 0x43084308u);
}

// int4 (two's complement nibbles) . bf16 activations.  Each code is turned
// into the bf16 number 136 + code (exact: an offset-binary nibble placed
// under the exponent of 128), so a dot2 gives sum (code + 136) * x and the
// caller subtracts 136 * sum(x).  xq holds the activation pairs in the order
// the unpacking produces: for dword d, (x0,x4), (x1,x5), (x2,x6), (x3,x7).
__device__ __forceinline__ float int4_chunk_bf16(const uint4 q, const uint32_t* xq) {
    float p = 0.f;
    const uint32_t v[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
        for (int s = 0; s < 4; ++s) p = dot2_bf16(int4x2_bf16(v[d] >> (4 * s)), as_bf16x2(xq[4 * d + s]), p);
    }
    return p;
}

// The same weights against fp32 activations held as bf16 hi + lo halves
// (hq, lq, in the unpacking order): each weight pair is unpacked once and
// meets both halves, so the sum carries about 17 bits of each activation.
__device__ __forceinline__ float int4_chunk_bf16_hl(const uint4 q, const uint32_t* hq, const uint32_t* lq) {
    float p = 0.f;
    const uint32_t v[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const bf16x2 w = int4x2_bf16(v[d] >> (4 * s));
            p = dot2_bf16(w, as_bf16x2(hq[4 * d + s]), p);
            p = dot2_bf16(w, as_bf16x2(lq[4 * d + s]), p);
        }
    }
    return p;
}

// Reorder the natural bf16 pairs of 8 elements (P0..P3 = (x0,x1)..(x6,x7))
// into the int4 unpacking order (x0,x4), (x1,x5), (x2,x6), (x3,x7).
__device__ __forceinline__ void int4_pair_order(const uint32_t* p, uint32_t* q) {
    q[0] = __builtin_amdgcn_perm(p[2], p[0], 0x05040100u);
    q[1] = __builtin_amdgcn_perm(p[2], p[0], 0x07060302u);
    q[2] = __builtin_amdgcn_perm(p[3], p[1], 0x05040100u);
    q[3] = __builtin_amdgcn_perm(p[3], p[1], 0x07060302u);
}

// Byte k of v as fp32 (the backend selects v_cvt_f32_ubyte<k>).
template <int k>
__device__ __forceinline__ float ubyte_f32(uint32_t v) { return (float)((v >> (8 * k)) & 0xffu); }

// int4 (two's complement nibbles) . fp32 activations: offset-binary bytes
// converted with the byte-to-float instructions; the caller subtracts
// 8 * sum(h).
__device__ __forceinline__ float int4_chunk_f32(const uint4 q, const float* h) {
    float p = 0.f;
    const uint32_t v[4] = {q.x ^ 0x88888888u, q.y ^ 0x88888888u, q.z ^ 0x88888888u, q.w ^ 0x88888888u};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t lo = v[d] & 0x0F0F0F0Fu, hi = (v[d] >> 4) & 0x0F0F0F0Fu;
        const float* hd = h + 8 * d;
        p = __builtin_fmaf(ubyte_f32<0>(lo), hd[0], p);
        p = __builtin_fmaf(ubyte_f32<0>(hi), hd[1], p);
        p = __builtin_fmaf(ubyte_f32<1>(lo), hd[2], p);
        p = __builtin_fmaf(ubyte_f32<1>(hi), hd[3], p);
        p = __builtin_fmaf(ubyte_f32<2>(lo), hd[4], p);
        p = __builtin_fmaf(ubyte_f32<2>(hi), hd[5], p);
        p = __builtin_fmaf(ubyte_f32<3>(lo), hd[6], p);
        p = __builtin_fmaf(ubyte_f32<3>(hi), hd[7], p);
    }
    return p;
}

__device__ __forceinline__ uint4 ldg16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

// Streaming (read-once) 16-byte load: non-temporal, so weight streams do not
// displace reused data (router weights, activations) from the caches.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// 8 and 16 bytes at an address that is only known to be 4-byte aligned
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
__device__ __forceinline__ u32x2 ldg8_a4(const uint8_t* p) { return *reinterpret_cast<const u32x2_a4*>(p); }
__device__ __forceinline__ u32x4 ldg16_a4(const uint8_t* p) { return *reinterpret_cast<const u32x4_a4*>(p); }
__device__ __forceinline__ uint4 ldg16_stream(const uint8_t* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Wave maximum of v, returned as a uniform value (DPP inside rows, row
// broadcasts across rows, then lane 63 read into a scalar).
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x124>(v));
    v = fmaxf(v, dpp<0x128>(v));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v),
                                                                      __builtin_bit_cast(int, v), 0x142, 0xA, 0xF,
                                                                      false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v),
                                                                      __builtin_bit_cast(int, v), 0x143, 0xC, 0xF,
                                                                      false)));
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}


typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Two E4M3FN bytes (bytes 0,1 of v, or 2,3 when HI) -> fp16 pair.  gfx950's
// fp8 converts use the OCP E4M3FN encoding; every E4M3FN value (NaN and -0
// included) is exact in fp16, and with scale 1 the conversion is exact.
template <bool HI>
__device__ __forceinline__ f16x2 e4m3x2_f16(uint32_t v) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, 1.0f, HI);
}

// Eight E2M1 codes (one dword) times their block scale, as fp16.  e2m1 *
// e4m3 has at most six significant bits and lies in [2^-10, 2688]: exact.
__device__ __forceinline__ f16x8 fp4x8_f16(uint32_t w, f16x2 s) {
    const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
    const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
    const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
    const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
    return f16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// Order-preserving int32 image of an fp32 key: for keys that are not NaN,
// a < b exactly when key_order(a) < key_order(b), and -0 and +0 map alike to
// 0.  NaN maps to INT_MIN, below every key.
__device__ __forceinline__ int key_order(float f) {
    int b = __builtin_bit_cast(int, f);
    if ((b << 1) == 0) b = 0;
    return f != f ? INT_MIN : (b >= 0 ? b : b ^ 0x7fffffff);
}

// Maximum over the 64 lanes of a wave (DPP only), returned to every lane.
__device__ __forceinline__ int wave_max_i32(int v) {
    v = max(v, __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true));   // quad_perm [1,0,3,2]
    v = max(v, __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true));   // quad_perm [2,3,0,1]
    v = max(v, __builtin_amdgcn_mov_dpp(v, 0x124, 0xF, 0xF, true));  // row_ror:4
    v = max(v, __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, true));  // row_ror:8 (every lane: its row's max)
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x142, 0xA, 0xF, false));  // rows 1, 3 take rows 0, 2 in
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x143, 0xC, 0xF, false));  // row 3 takes lane 31 in
    return __builtin_amdgcn_readlane(v, 63);
}

}  // namespace q4moe
