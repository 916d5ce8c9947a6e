// W4A4 routed-MoE chunk on gfx950: many tokens through one layer whose
// routed experts take 4-bit weights AND 4-bit activations ("Let's optimize
// Nemotron 3.5 Lightning - a worklog", Step 3: routed experts W4A4 with a
// dynamic NVFP4 input quantizer; the prefill comparison of Marlin W4A16 and
// CUTLASS FP4 grouped GEMMs).
//
// Pipeline (one stream, no host synchronisation):
//   router GEMM (fp32) -> top-k -> dispatch (per-expert token lists, stable
//   in token order) -> NVFP4 quantization of x -> grouped up GEMM on MFMA
//   (epilogue h = relu(g u)^2) -> NVFP4 quantization of h -> grouped down
//   GEMM on MFMA (epilogue w g z per (token, slot) row) -> combine over the
//   slots in slot order.
//
// gfx950's 4-bit MFMA takes power-of-two (E8M0) scales per 32 elements and
// cannot express NVFP4's E4M3 scale per 16, so both operands are decoded to
// bf16 while they are staged in LDS: e2m1 * e4m3 has at most six significant
// bits, so every decoded operand is exact in bf16 and every MFMA product is
// exact in fp32; only the fp32 accumulation rounds.
#pragma once

#include "q4moe_kernels.hpp"

namespace q4moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// Router logits for many tokens on fp32 MFMA (v_mfma_f32_32x32x2_f32):
// a workgroup computes a 32-token x 32-expert tile; its 8 waves split the
// hidden dimension and their partial tiles are summed in LDS in wave order.
// Lane l feeds token/expert row l % 32 and, for each group of 8 k-values,
// k-values 4 (l / 32) .. +3 (one per MFMA; A and B use the same k order).
// ---------------------------------------------------------------------------
typedef float f32x16r __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(512) void k_router_gemm(RouterArgs a) {
    __shared__ float part[8][32][33];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e0 = blockIdx.x * 32, t0 = blockIdx.y * 32;
    const int row = lane & 31, kq = lane >> 5;
    const int t = min(t0 + row, a.T - 1), e = min(e0 + row, a.E - 1);
    const uint16_t* xr = a.x + (size_t)t * a.H + 4 * kq;
    const float* wr = a.wg + (size_t)e * a.H + 4 * kq;
    const int nblk = a.H / 8;
    const int b0 = wave * nblk / 8, b1 = (wave + 1) * nblk / 8;
    f32x16r acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    for (int b = b0; b < b1; ++b) {
        const uint2 xv = *reinterpret_cast<const uint2*>(xr + 8 * b);
        const float4 wv = *reinterpret_cast<const float4*>(wr + 8 * b);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(bf16_bits_to_f32(xv.x & 0xffffu), wv.x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(bf16_bits_to_f32(xv.x >> 16), wv.y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(bf16_bits_to_f32(xv.y & 0xffffu), wv.z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(bf16_bits_to_f32(xv.y >> 16), wv.w, acc, 0, 0, 0);
    }
    // lane holds column j = lane % 32 (expert) and rows 8 (r/4) + 4 (lane/32) + r % 4 (tokens)
#pragma unroll
    for (int r = 0; r < 16; ++r) part[wave][8 * (r / 4) + 4 * kq + (r % 4)][row] = acc[r];
    __syncthreads();
    for (int idx = threadIdx.x; idx < 32 * 32; idx += 512) {
        const int i = idx >> 5, j = idx & 31;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < 8; ++w) v += part[w][i][j];
        const int tt = t0 + i, ee = e0 + j;
        if (tt < a.T && ee < a.E) {
            a.logits[(size_t)tt * a.E + ee] = v;
            if (a.logits_out) a.logits_out[(size_t)tt * a.E + ee] = v;
        }
    }
}

// ---------------------------------------------------------------------------
// Dispatch: expert e's (token, slot) pairs in token order.  One wave per
// expert scans the routing table 64 tokens at a time (a token selects an
// expert at most once).
// ---------------------------------------------------------------------------
struct DispatchArgs {
    const int32_t* ids;  // [T][K]
    int T, K, E;
    int32_t* counts;     // [E]
    int32_t* lists;      // [E][T]  pair index t*K + slot
    int32_t* offsets;    // [E+1]
    int32_t* perm;       // [T*K]   dispatch row -> pair
    int32_t* inv;        // [T*K]   pair -> dispatch row
};

__global__ __launch_bounds__(64) void k_dispatch(DispatchArgs a) {
    const int e = blockIdx.x, lane = threadIdx.x;
    int base = 0;
    for (int t0 = 0; t0 < a.T; t0 += 64) {
        const int t = t0 + lane;
        int pair = -1;
        if (t < a.T)
            for (int s = 0; s < a.K; ++s)
                if (a.ids[(size_t)t * a.K + s] == e) pair = t * a.K + s;
        const unsigned long long m = __ballot(pair >= 0);
        if (pair >= 0) {
            const int before = __popcll(m & ((1ull << lane) - 1ull));
            a.lists[(size_t)e * a.T + base + before] = pair;
        }
        base += __popcll(m);
    }
    if (lane == 0) a.counts[e] = base;
}

// Offsets (exclusive scan of the counts), the dispatch permutation and its
// inverse.  Workgroup e (grid E) loads all counts, scans them in LDS and
// writes expert e's part of the permutation.
__global__ __launch_bounds__(256) void k_dispatch_scan(DispatchArgs a) {
    __shared__ int s_cnt[256], s_off[257];
    const int e = blockIdx.x;
    for (int i = threadIdx.x; i < a.E; i += 256) s_cnt[i] = a.counts[i];
    __syncthreads();
    if (threadIdx.x == 0) {
        int o = 0;
        for (int i = 0; i < a.E; ++i) {
            s_off[i] = o;
            o += s_cnt[i];
        }
        s_off[a.E] = o;
    }
    __syncthreads();
    if (e == 0)
        for (int i = threadIdx.x; i <= a.E; i += 256) a.offsets[i] = s_off[i];
    const int n = s_cnt[e];
    for (int i = threadIdx.x; i < n; i += 256) {
        const int pair = a.lists[(size_t)e * a.T + i];
        a.perm[s_off[e] + i] = pair;
        a.inv[pair] = s_off[e] + i;
    }
}

// ---------------------------------------------------------------------------
// NVFP4 activation quantizer: per row, per block of 16, scale = E4M3FN
// nearest-even of fl32(amax / 6) (saturating at 448); code = nearest E2M1
// magnitude of |v| / scale, ties to the even code, saturating at 6; sign bit
// of v kept; scale 0 gives magnitude 0.
// ---------------------------------------------------------------------------

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

// E2M1 magnitude code of |v| on the grid scaled by s (ties to even codes).
__device__ __forceinline__ uint32_t e2m1_code(float mag, float s) {
    if (s == 0.f) return 0u;
    const float mids[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
    uint32_t idx = 0;
#pragma unroll
    for (int j = 0; j < 7; ++j) {
        const float t = mids[j] * s;  // exact
        const bool up = mag > t || (mag == t && ((j + 1) & 1) == 0);
        idx += (up && idx == (uint32_t)j) ? 1u : 0u;
    }
    return idx;
}

struct QuantArgs {
    int rows, cols;
    const void* v;      // bf16 bits (BF16_IN) or fp32
    uint8_t* codes;     // [rows][cols/2]
    uint8_t* scales;    // [rows][cols/16]
};

template <bool BF16_IN>
__global__ __launch_bounds__(256) void k_quant_nvfp4(QuantArgs a) {
    const size_t blk = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t nb_row = (size_t)a.cols / 16;
    if (blk >= (size_t)a.rows * nb_row) return;
    const size_t r = blk / nb_row, b = blk % nb_row;
    float v[16];
    if constexpr (BF16_IN) {
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.v) + r * a.cols + b * 16);
        const uint4 q0 = p[0], q1 = p[1];
        const uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            v[2 * j] = bf16_bits_to_f32(w[j] & 0xffffu);
            v[2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
        }
    } else {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(a.v) + r * a.cols + b * 16);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float4 q = p[k];
            v[4 * k] = q.x;
            v[4 * k + 1] = q.y;
            v[4 * k + 2] = q.z;
            v[4 * k + 3] = q.w;
        }
    }
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(v[j]));
    const uint32_t sb = e4m3fn_rne_sat(__fdiv_rn(amax, 6.0f));
    const float s = e4m3fn_to_f32(sb);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const uint32_t c = e2m1_code(fabsf(v[j]), s) | ((__float_as_uint(v[j]) >> 31) << 3);
        if (j < 8)
            lo |= c << (4 * j);
        else
            hi |= c << (4 * (j - 8));
    }
    *reinterpret_cast<uint2*>(a.codes + r * (a.cols / 2) + b * 8) = make_uint2(lo, hi);
    a.scales[r * nb_row + b] = (uint8_t)sb;
}

// ---------------------------------------------------------------------------
// Grouped GEMM on MFMA: for expert e and a 128-column output tile,
// out[m][n] = sum_k A[m][k] * W_e[n][k] over the expert's rows m, with both
// operands NVFP4 (codes + E4M3 scale per 16 along k) decoded into LDS as bf16.
// Workgroup: 4 waves; wave w owns output columns 32w..32w+31 and up to four
// 32-row subtiles (128 rows) of M, one v_mfma_f32_32x32x16_bf16 accumulator
// each.  K advances 64 per step; the next step's global loads are in flight
// while the current step's MFMAs run.
// ---------------------------------------------------------------------------
enum : int { EPI_UP = 0, EPI_DOWN = 1 };
constexpr int kGemmBN = 128, kGemmBM = 128, kGemmBK = 64, kLdsPitch = kGemmBK + 8;  // bf16 elements

struct GemmArgs {
    int N, Kd;                 // output columns (rows of W_e), reduction length
    const uint8_t* wc;         // W codes  [E][N][Kd/2]
    const uint8_t* wsc;        // W scales [E][N][Kd/16]
    const float* wg;           // per-expert fp32 scale [E]
    const uint8_t* ac;         // A codes  [rows][Kd/2]
    const uint8_t* asc;        // A scales [rows][Kd/16]
    const int32_t* offsets;    // [E+1] dispatch rows of each expert
    const int32_t* perm;       // dispatch row -> pair t*K + slot
    int K;                     // top-k (pair -> token = pair / K)
    int a_by_token;            // 1: A row = token of the pair (up), 0: A row = dispatch row (down)
    const float* wgate;        // [T*K] gates by pair (down epilogue)
    float* out;                // [rows][N] fp32, dispatch order
};

// Decode 32 NVFP4 elements (16 code bytes, two E4M3 scale bytes) to bf16 in LDS.
__device__ __forceinline__ void decode32_to_lds(uint4 q, uint32_t sb, uint16_t* dst) {
    const float s0 = e4m3fn_to_f32(sb & 0xffu), s1 = e4m3fn_to_f32((sb >> 8) & 0xffu);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    uint32_t o[16];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const float s = d < 2 ? s0 : s1;
        const f32x2 p0 = fp4x2_f32<0>(w[d]), p1 = fp4x2_f32<1>(w[d]), p2 = fp4x2_f32<2>(w[d]),
                    p3 = fp4x2_f32<3>(w[d]);
        // products are exact and representable in bf16: truncation is exact
        o[4 * d + 0] = (__float_as_uint(p0.x * s) >> 16) | (__float_as_uint(p0.y * s) & 0xffff0000u);
        o[4 * d + 1] = (__float_as_uint(p1.x * s) >> 16) | (__float_as_uint(p1.y * s) & 0xffff0000u);
        o[4 * d + 2] = (__float_as_uint(p2.x * s) >> 16) | (__float_as_uint(p2.y * s) & 0xffff0000u);
        o[4 * d + 3] = (__float_as_uint(p3.x * s) >> 16) | (__float_as_uint(p3.y * s) & 0xffff0000u);
    }
    uint4* d4 = reinterpret_cast<uint4*>(dst);
    d4[0] = make_uint4(o[0], o[1], o[2], o[3]);
    d4[1] = make_uint4(o[4], o[5], o[6], o[7]);
    d4[2] = make_uint4(o[8], o[9], o[10], o[11]);
    d4[3] = make_uint4(o[12], o[13], o[14], o[15]);
}

template <int EPI>
__global__ __launch_bounds__(256, 2) void k_grouped_gemm(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t As[kGemmBM][kLdsPitch];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[kGemmBN][kLdsPitch];
    const int e = blockIdx.y;
    const int row0 = a.offsets[e], n_e = a.offsets[e + 1] - row0;
    const int n0 = blockIdx.x * kGemmBN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nk = a.Kd / kGemmBK;
    // staging role: row tid/2 of the A and B tiles, k half (tid & 1) * 32
    const int sr = threadIdx.x >> 1, sh = threadIdx.x & 1;
    const uint8_t* wrow_c = a.wc + ((size_t)e * a.N + min(n0 + sr, a.N - 1)) * (a.Kd / 2);
    const uint8_t* wrow_s = a.wsc + ((size_t)e * a.N + min(n0 + sr, a.N - 1)) * (a.Kd / 16);
    const float g = a.wg[e];

    for (int m0 = 0; m0 < n_e; m0 += kGemmBM) {
        const int mv = min(kGemmBM, n_e - m0);  // valid rows in this chunk
        const int ms = (mv + 31) / 32;          // 32-row subtiles in use
        // A row of this thread's staging row (clamped to a valid row)
        const int am = min(sr, mv - 1);
        const int drow = row0 + m0 + am;
        const size_t arow = a.a_by_token ? (size_t)(a.perm[drow] / a.K) : (size_t)drow;
        const uint8_t* arow_c = a.ac + arow * (a.Kd / 2);
        const uint8_t* arow_s = a.asc + arow * (a.Kd / 16);
        const bool stage_a = sr < mv;

        f32x16 acc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

        // operands of the next kPre k-steps are in flight in a register ring
        constexpr int kPre = 4;
        uint4 qb[kPre], qa[kPre];
        uint32_t sbb[kPre], sba[kPre];
#pragma unroll
        for (int j = 0; j < kPre; ++j) {
            if (j < nk) {
                const int kb = j * kGemmBK;
                qb[j] = ldg16_stream(wrow_c + kb / 2 + sh * 16);
                sbb[j] = *reinterpret_cast<const uint16_t*>(wrow_s + kb / 16 + sh * 2);
                qa[j] = ldg16(arow_c + kb / 2 + sh * 16);
                sba[j] = *reinterpret_cast<const uint16_t*>(arow_s + kb / 16 + sh * 2);
            }
        }
        for (int ks0 = 0; ks0 < nk; ks0 += kPre) {
#pragma unroll
            for (int j = 0; j < kPre; ++j) {
                const int ks = ks0 + j;
                if (ks < nk) {  // uniform
                    __syncthreads();  // previous step's MFMAs are done with the tiles
                    decode32_to_lds(qb[j], sbb[j], &Bs[sr][sh * 32]);
                    if (stage_a) decode32_to_lds(qa[j], sba[j], &As[sr][sh * 32]);
                    __syncthreads();
                    if (ks + kPre < nk) {
                        const int kb = (ks + kPre) * kGemmBK;
                        qb[j] = ldg16_stream(wrow_c + kb / 2 + sh * 16);
                        sbb[j] = *reinterpret_cast<const uint16_t*>(wrow_s + kb / 16 + sh * 2);
                        qa[j] = ldg16(arow_c + kb / 2 + sh * 16);
                        sba[j] = *reinterpret_cast<const uint16_t*>(arow_s + kb / 16 + sh * 2);
                    }
#pragma unroll
                    for (int kk = 0; kk < kGemmBK; kk += 16) {
                        const bf16x8 bfrag =
                            *reinterpret_cast<const bf16x8*>(&Bs[32 * wave + (lane & 31)][kk + 8 * (lane >> 5)]);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            if (i < ms) {
                                const bf16x8 afrag = *reinterpret_cast<const bf16x8*>(
                                    &As[32 * i + (lane & 31)][kk + 8 * (lane >> 5)]);
                                acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag, bfrag, acc[i], 0, 0, 0);
                            }
                        }
                    }
                }
            }
        }
        // epilogue: lane holds column n = n0 + 32 wave + (lane & 31) and rows
        // 32 i + 8 (r / 4) + 4 (lane / 32) + r % 4
        const int n = n0 + 32 * wave + (lane & 31);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i < ms) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = 32 * i + 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
                    if (m < mv && n < a.N) {
                        const int p = row0 + m0 + m;
                        float v = acc[i][r] * g;
                        if constexpr (EPI == EPI_UP) {
                            v = fmaxf(v, 0.f);
                            v = v * v;
                        } else {
                            v = a.wgate[a.perm[p]] * v;
                        }
                        a.out[(size_t)p * a.N + n] = v;
                    }
                }
            }
        }
    }
}

// y32[t][n] = sum over slots s (in order) of zw[inv[t*K + s]][n]; y = bf16.
__global__ __launch_bounds__(256) void k_combine(int T, int K, int H, const int32_t* inv, const float* zw,
                                                 float* y32, uint16_t* y) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (size_t)T * H) return;
    const size_t t = i / H, n = i % H;
    float acc = 0.f;
    for (int s = 0; s < K; ++s) acc += zw[(size_t)inv[t * K + s] * H + n];
    y32[i] = acc;
    y[i] = (uint16_t)f32_to_bf16_rne(acc);
}

}  // namespace q4moe
