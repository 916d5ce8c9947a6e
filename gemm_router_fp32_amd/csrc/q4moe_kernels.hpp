// libq4moe kernels for gfx950: router top-k, reference dequantization,
// W4A16 decode (up GEMV + relu^2, down GEMV + weighted combine) and the
// NVFP4 lm_head GEMV with argmax.
//
// Batch-1 decode is a pure weight read ("Let's optimize Nemotron 3.5
// Lightning - a worklog", Interlude): every kernel streams its 4-bit codes
// with 16-byte loads (one 16-byte chunk = 32 consecutive elements of a row,
// two NVFP4 blocks or half an int4 group), decodes them in registers and
// reduces rows across lane segments.
#pragma once

#include "q4moe_device.hpp"

namespace q4moe {

enum : int { FMT_NVFP4 = 1, FMT_INT4 = 2, FMT_FP8 = 3 };

// Control words at the start of every workspace.
enum : int { CTRL_TICKET = 0, CTRL_FLAGS = 1, CTRL_WORDS = 1024 };

// ---------------------------------------------------------------------------
// Router ("Quantization (PTQ + QAD)", Precision Recipes: router compute FP32;
// "NVIDIA-Nemotron-3.5-Lightning-30B-A3B-W4A16" README, Left at bfloat16:
// fp32 e_score_correction_bias)
// ---------------------------------------------------------------------------

struct RouterArgs {
    const float* wg;
    const float* bias;
    const uint16_t* x;
    int E, H, T, K;
    float* logits;      // [T][E]
    int32_t* ids;       // [T][K] (workspace copy)
    float* w;           // [T][K]
    int32_t* ids_out;   // nullable
    float* w_out;       // nullable
    float* logits_out;  // nullable
};

// logits[t][e] = sum_c W_g[e][c] * x[t][c]: one workgroup per expert and up
// to four tokens, grid (E, ceil(T/4)), 256 threads.  Thread i takes the
// 4-column pieces i, i + 256, ... (H <= 4096: at most four), all loads issued
// before any use; the partial sums meet in LDS in a fixed order.
__global__ __launch_bounds__(256) void k_router_logits(RouterArgs a) {
    constexpr int kPieces = 4;  // 4096 / 4 / 256
    __shared__ float part[4][4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e = blockIdx.x, t0 = blockIdx.y * 4;
    const int nt = min(4, a.T - t0);
    const int np = a.H / 4;
    const float4* wr = reinterpret_cast<const float4*>(a.wg + (size_t)e * a.H);
    float4 wv[kPieces];
    uint2 xb[kPieces][4];
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
        const int j = min((int)threadIdx.x + 256 * i, np - 1);  // clamped: unused pieces are masked below
        wv[i] = wr[j];
#pragma unroll
        for (int t = 0; t < 4; ++t)
            xb[i][t] = *reinterpret_cast<const uint2*>(a.x + (size_t)(t0 + min(t, nt - 1)) * a.H + 4 * j);
    }
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
        if ((int)threadIdx.x + 256 * i < np) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                acc[t] = __builtin_fmaf(wv[i].x, bf16_bits_to_f32(xb[i][t].x & 0xffffu), acc[t]);
                acc[t] = __builtin_fmaf(wv[i].y, bf16_bits_to_f32(xb[i][t].x >> 16), acc[t]);
                acc[t] = __builtin_fmaf(wv[i].z, bf16_bits_to_f32(xb[i][t].y & 0xffffu), acc[t]);
                acc[t] = __builtin_fmaf(wv[i].w, bf16_bits_to_f32(xb[i][t].y >> 16), acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const float l = seg_sum<64>(acc[t]);
        if (lane == 0) part[wave][t] = l;
    }
    __syncthreads();
    if (threadIdx.x < nt) {
        const int t = threadIdx.x;
        const float l = (part[0][t] + part[1][t]) + (part[2][t] + part[3][t]);
        a.logits[(size_t)(t0 + t) * a.E + e] = l;
        if (a.logits_out) a.logits_out[(size_t)(t0 + t) * a.E + e] = l;
    }
}

// Sigmoid scores, selection key score + bias, top-K by key (largest first,
// equal keys -> lower index), gates = selected scores / their sum, for token
// t by one wave (E <= 256: four experts per lane).  Writes a.ids / a.w (and
// the caller's copies) when `global`, and lds_ids / lds_w when not null.
__device__ __forceinline__ void topk_token(const RouterArgs& a, int t, bool global, int32_t* lds_ids,
                                           float* lds_w) {
    const int lane = threadIdx.x & 63;
    float s[4], key[4];
    bool live[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = lane + kWave * q;
        live[q] = e < a.E;
        const float l = live[q] ? a.logits[(size_t)t * a.E + e] : 0.f;
        s[q] = 1.0f / (1.0f + expf(-l));
        key[q] = s[q] + (live[q] ? a.bias[e] : 0.f);
    }
    // Each round: the wave maximum (DPP), then the lowest expert index holding
    // it (ballot + find-first-set), so equal keys go to the lower index.  The
    // loop is unrolled (K <= 8) so the selections stay in registers.
#pragma unroll
    for (int q = 0; q < 4; ++q)
        if (!live[q]) key[q] = -__builtin_inff();
    float sel_s[8];
    int sel_i[8];
    float ssum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        sel_s[i] = 0.f;
        sel_i[i] = 0;
        if (i >= a.K) continue;
        const float m = wave_max(fmaxf(fmaxf(key[0], key[1]), fmaxf(key[2], key[3])));
        int best = 0x7fffffff;
        float bs = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const unsigned long long hit = __ballot(key[q] == m);
            if (hit && best == 0x7fffffff) {
                const int l = (int)__builtin_ctzll(hit);
                best = l + kWave * q;
                bs = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s[q]), l));
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (lane + kWave * q == best) key[q] = -__builtin_inff();
        if (best >= a.E) {  // no finite key left (NaN logits): keep ids inside the bank
            best = 0;
            bs = 0.f;
        }
        sel_s[i] = bs;
        sel_i[i] = best;
        ssum += bs;
    }
    if (lane < a.K) {
        float ws = 0.f;
        int wi = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i == lane) {
                ws = sel_s[i];
                wi = sel_i[i];
            }
        const float wv = ws / ssum;
        const size_t o = (size_t)t * a.K + lane;
        if (global) {
            a.ids[o] = wi;
            a.w[o] = wv;
            if (a.ids_out) a.ids_out[o] = wi;
            if (a.w_out) a.w_out[o] = wv;
        }
        if (lds_ids) {
            lds_ids[lane] = wi;
            lds_w[lane] = wv;
        }
    }
}

// One wave per token; grid ceil(T/4).
__global__ __launch_bounds__(256) void k_topk(RouterArgs a) {
    const int t = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    if (t >= a.T) return;  // wave-uniform
    topk_token(a, t, true, nullptr, nullptr);
}

// ---------------------------------------------------------------------------
// Reference dequantization: one thread per code dword (8 elements).
// NVFP4: fl32((e2m1 * e4m3fn) * g); INT4_G64: int4 * bf16 (exact in fp32).
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_dequant(int fmt, int rows, int cols, const uint8_t* codes,
                                                 const void* scales, const float* gscale, float* out) {
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t dw_per_row = (size_t)cols / 8;
    if (idx >= (size_t)rows * dw_per_row) return;
    const size_t r = idx / dw_per_row;
    const int c0 = (int)(idx % dw_per_row) * 8;
    const uint32_t v = reinterpret_cast<const uint32_t*>(codes)[idx];
    float o[8];
    if (fmt == FMT_NVFP4) {
        const uint8_t* sc = reinterpret_cast<const uint8_t*>(scales);
        const float s = e4m3fn_to_f32(sc[r * (cols / 16) + c0 / 16]);
        const float g = *gscale;
        const f32x2 p0 = fp4x2_f32<0>(v), p1 = fp4x2_f32<1>(v), p2 = fp4x2_f32<2>(v), p3 = fp4x2_f32<3>(v);
        const float e2[8] = {p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = __fmul_rn(__fmul_rn(e2[j], s), g);
    } else {
        const uint16_t* sc = reinterpret_cast<const uint16_t*>(scales);
        const float s = bf16_bits_to_f32(sc[r * (cols / 64) + c0 / 64]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int n = (int)((v >> (4 * j)) & 15u);
            o[j] = __fmul_rn((float)(n >= 8 ? n - 16 : n), s);
        }
    }
    float4* dst = reinterpret_cast<float4*>(out + r * cols + c0);
    dst[0] = make_float4(o[0], o[1], o[2], o[3]);
    dst[1] = make_float4(o[4], o[5], o[6], o[7]);
}

// ---------------------------------------------------------------------------
// W4A16 decode ("Let's optimize Nemotron 3.5 Lightning - a worklog", Step 1:
// 4-bit weights dequantized inside the kernel, 16-bit activations;
// "NVIDIA-Nemotron-3.5-Lightning-30B-A3B-W4A16" README, Checkpoint layout:
// per-expert up_proj and down_proj)
// ---------------------------------------------------------------------------

struct MoeArgs {
    int fmt, E, H, I, K, T;
    const uint8_t* upc;
    const void* ups;
    const float* upg;
    const uint8_t* dnc;
    const void* dns;
    const float* dng;
    const uint16_t* x;   // [T][H] bf16
    const int32_t* ids;  // [T][K]
    const float* w;      // [T][K]
    float* h;            // [T*K][I]
    float* y32;          // [T][H]
    uint16_t* y;         // [T][H] bf16
};

// Load the bf16 activations of chunk `ch` (32 elements) as 16 natural pairs.
__device__ __forceinline__ void load_x_chunk(const uint16_t* xrow, int ch, uint32_t* xa) {
    const uint4* p = reinterpret_cast<const uint4*>(xrow + ch * 32);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint4 v = p[k];
        xa[4 * k + 0] = v.x;
        xa[4 * k + 1] = v.y;
        xa[4 * k + 2] = v.z;
        xa[4 * k + 3] = v.w;
    }
}

__device__ __forceinline__ float pair_sum_bf16(const uint32_t* xa) {
    // one dot2 with (1, 1) per pair: 16 instructions instead of 64 converts
    // and adds (the products are exact, the sum is fp32)
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) s = dot2_bf16(as_bf16x2(xa[j]), as_bf16x2(0x3F803F80u), s);
    return s;
}

// u = W_up[e] x_t for rows of expert e = ids[p], h[p][r] = relu(u)^2.
// 32-lane segments, one row per segment: lane li holds chunks li*C .. li*C+C-1
// of the row.  Grid (ceil(I/8), T*K), 256 threads: 8 rows per block.
template <int C, int FMT>
__global__ __launch_bounds__(256) void k_up(MoeArgs a) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int seg = lane >> 5, li = lane & 31;
    const int p = blockIdx.y;
    const int t = p / a.K;
    const int e = min(max(a.ids[p], 0), a.E - 1);  // routing ids are always in range; never read outside the bank
    const int r = blockIdx.x * 8 + wave * 2 + seg;
    const int nch = a.H / 32;
    const bool rowok = r < a.I;
    const uint16_t* xrow = a.x + (size_t)t * a.H;

    uint32_t xa[C][16];
    float xs[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int ch = li * C + c;
        if (ch < nch) {
            uint32_t nat[16];
            load_x_chunk(xrow, ch, nat);
            if constexpr (FMT == FMT_NVFP4) {
#pragma unroll
                for (int j = 0; j < 16; ++j) xa[c][j] = nat[j];
                xs[c] = 0.f;
            } else {
#pragma unroll
                for (int d = 0; d < 4; ++d) int4_pair_order(nat + 4 * d, xa[c] + 4 * d);
                xs[c] = pair_sum_bf16(nat);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) xa[c][j] = 0u;
            xs[c] = 0.f;
        }
    }

    float acc = 0.f;
    if (rowok) {
        const size_t row = (size_t)e * a.I + r;
        const uint8_t* rc = a.upc + row * (a.H / 2);
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int ch = li * C + c;
            if (ch < nch) {
                const uint4 q = ldg16(rc + ch * 16);
                if constexpr (FMT == FMT_NVFP4) {
                    const uint8_t* sc = reinterpret_cast<const uint8_t*>(a.ups) + row * (a.H / 16) + ch * 2;
                    const uint32_t sb = *reinterpret_cast<const uint16_t*>(sc);
                    const f32x2 sp = e4m3fn_x2_f32(sb);
                    acc += nvfp4_chunk_bf16(q, xa[c], sp[0], sp[1]);
                } else {
                    const uint16_t* sc = reinterpret_cast<const uint16_t*>(a.ups) + row * (a.H / 64);
                    const float sg = bf16_bits_to_f32(sc[ch >> 1]);
                    acc = __builtin_fmaf(sg, int4_chunk_bf16(q, xa[c]) - 136.0f * xs[c], acc);
                }
            }
        }
    }
    acc = seg_sum<32>(acc);
    if (li == 0 && rowok) {
        const float u = (FMT == FMT_NVFP4) ? acc * a.upg[e] : acc;
        const float rl = fmaxf(u, 0.f);
        a.h[(size_t)p * a.I + r] = rl * rl;
    }
}

// z = W_down[e] h_p for all pairs p of every token, y[t][r] = sum_i w_i z_i.
// 64-lane segments, one row per wave at a time, 4 rows per wave; lane l holds
// chunks l*C .. l*C+C-1 of h.  Grid ceil(H/16), 256 threads.
template <int C, int FMT, int T>
__global__ __launch_bounds__(256) void k_down(MoeArgs a) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r0 = (blockIdx.x * 4 + wave) * 4;
    const int nch = a.I / 32;
    float acc[4][T];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
#pragma unroll
        for (int t = 0; t < T; ++t) acc[rr][t] = 0.f;

    for (int p = 0; p < T * a.K; ++p) {
        const int t = p / a.K;
        const int e = min(max(a.ids[p], 0), a.E - 1);
        const float wgt = a.w[p] * ((FMT == FMT_NVFP4) ? a.dng[e] : 1.0f);
        float hv[C][32];
        float hs[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int ch = lane * C + c;
            hs[c] = 0.f;
            if (ch < nch) {
                const float4* hp = reinterpret_cast<const float4*>(a.h + (size_t)p * a.I + ch * 32);
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float4 v = hp[k];
                    hv[c][4 * k + 0] = v.x;
                    hv[c][4 * k + 1] = v.y;
                    hv[c][4 * k + 2] = v.z;
                    hv[c][4 * k + 3] = v.w;
                }
                if constexpr (FMT == FMT_INT4) {
#pragma unroll
                    for (int j = 0; j < 32; ++j) hs[c] += hv[c][j];
                }
            } else {
#pragma unroll
                for (int j = 0; j < 32; ++j) hv[c][j] = 0.f;
            }
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int r = r0 + rr;
            if (r >= a.H) break;  // wave-uniform
            const size_t row = (size_t)e * a.H + r;
            const uint8_t* rc = a.dnc + row * (a.I / 2);
            float z = 0.f;
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const int ch = lane * C + c;
                if (ch < nch) {
                    const uint4 q = ldg16(rc + ch * 16);
                    if constexpr (FMT == FMT_NVFP4) {
                        const uint8_t* sc = reinterpret_cast<const uint8_t*>(a.dns) + row * (a.I / 16) + ch * 2;
                        const uint32_t sb = *reinterpret_cast<const uint16_t*>(sc);
                        const f32x2 sp = e4m3fn_x2_f32(sb);
                        z += nvfp4_chunk_f32(q, hv[c], sp[0], sp[1]);
                    } else {
                        const uint16_t* sc = reinterpret_cast<const uint16_t*>(a.dns) + row * (a.I / 64);
                        const float sg = bf16_bits_to_f32(sc[ch >> 1]);
                        z = __builtin_fmaf(sg, int4_chunk_f32(q, hv[c]) - 8.0f * hs[c], z);
                    }
                }
            }
            z = seg_sum<64>(z);
#pragma unroll
            for (int tt = 0; tt < T; ++tt)
                if (tt == t) acc[rr][tt] = __builtin_fmaf(wgt, z, acc[rr][tt]);
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int r = r0 + rr;
            if (r >= a.H) break;
#pragma unroll
            for (int t = 0; t < T; ++t) {
                a.y32[(size_t)t * a.H + r] = acc[rr][t];
                a.y[(size_t)t * a.H + r] = (uint16_t)f32_to_bf16_rne(acc[rr][t]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// NVFP4 W4A16 GEMV + argmax ("Let's optimize Nemotron 3.5 Lightning - a
// worklog", Step 4: the NVFP4 lm_head; Step 5: four tokens verified per step)
// ---------------------------------------------------------------------------

struct GemvArgs {
    int rows, cols, T;
    const uint8_t* codes;
    const uint8_t* scales;
    const float* gscale;
    const uint16_t* x;
    float* logits;           // [T][rows]
    int32_t* argmax;         // nullable
    unsigned long long* keys;  // [gridDim][T] workspace: each workgroup's best key per token
};

// Order-preserving map of fp32 onto uint32 (larger float -> larger integer;
// -0 and +0 are equal numbers and map alike).
__device__ __forceinline__ uint32_t f32_order(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u << 1) == 0u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exponent s of the power of two 2^s that puts a row's largest magnitude mx
// in [2^14, 2^15) before the row is rounded to fp16 (0 for a zero, infinite
// or NaN maximum).  s is at most 127 so that 2^s stays finite in fp32: a row
// of bf16 subnormals (multiples of 2^-133) then lands on multiples of 2^-6,
// still exact in fp16.  Results are scaled back by ldexp(result, -s) before
// any other factor, so the way back is exact unless the result itself
// underflows.
__device__ __forceinline__ int fp16_stage_exp(float mx) {
    return (mx > 0.f && mx < __builtin_inff()) ? min(14 - ilogbf(mx), 127) : 0;
}

typedef float f32x4g __attribute__((ext_vector_type(4)));

// One group of 16 NVFP4 rows against up to 16 LDS columns on fp16 MFMA
// (v_mfma_f32_16x16x32_f16): returns D[4 kq + r][n] for n = lane % 16, where
// the 16-row operand is rows (row of lane (m16, kq)) and column n of the other
// operand is LDS row n of xs (pitch P fp16; columns n >= NT are zero).  Lane
// (m16, kq) reads bytes 64 j + 16 kq .. +15 of its row for j < NJ (k 128 j +
// 32 kq .. +31) and MFMA step (j, d) sums k 128 j + 32 kq + 8 d .. +7 on both
// operands.  Weights decode exactly to fp16 (e2m1 * e4m3 has at most six
// significant bits).  Loads go in batches of seven pieces, batch b+1 issued
// before batch b is computed; `after_first_issue` runs (in every thread)
// once the first batch is in flight.  Pieces past `cols` reread the row's
// last bytes with scale 0 and read LDS columns that must hold zeros up to
// 128 NJ.
// A full group (all 16 rows r0 .. r0 + 15 inside the matrix, `full`) has its
// block scales, one contiguous run of 16 * cols / 16 bytes, copied with
// 16-byte loads into the wave's LDS slice sblk (at least cols bytes) and read
// from there: per piece a lane would otherwise gather 2 bytes from each of 16
// rows.  Other groups load each scale pair from memory.
// Offsets are 32-bit from the uniform bases (codes under 4 GiB).
template <int NJ, int NT, int P, typename F>
__device__ __forceinline__ f32x4g mfma_gemv_group(const uint8_t* codes, const uint8_t* scales, uint32_t r, int cols,
                                                  const _Float16* xs, int m16, int kq, F&& after_first_issue,
                                                  uint8_t* sblk, uint32_t r0, bool full) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const uint32_t rc = r * (uint32_t)(cols / 2), rs = r * (uint32_t)(cols / 16);
    const int rb = cols / 16;  // scale bytes per row; 16 rows are rb 16-byte pieces
    const int lane = threadIdx.x & 63;
    constexpr int kB = 7;
    uint4 q[NJ];
    uint32_t sc[NJ];
    uint4 sv[4];  // cols <= 4096: at most 256 pieces, 4 per lane
    if (full) {
        const uint4* src = reinterpret_cast<const uint4*>(scales + r0 * (uint32_t)rb);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int pc = lane + 64 * i;
            sv[i] = pc < rb ? src[pc] : make_uint4(0u, 0u, 0u, 0u);
        }
    }
    auto issue = [&](int j0) {
#pragma unroll
        for (int j = j0; j < (j0 + kB < NJ ? j0 + kB : NJ); ++j) {
            const bool ok = 128 * j + 32 * kq < cols;
            q[j] = ldg16(codes + (rc + (ok ? 64 * j + 16 * kq : cols / 2 - 16)));
            if (!full) sc[j] = *reinterpret_cast<const uint16_t*>(scales + (rs + (ok ? 8 * j + 2 * kq : cols / 16 - 2)));
        }
    };
    f32x4g acc = {0.f, 0.f, 0.f, 0.f};
    issue(0);
    // (the caller may fill xs here, while the first batch is in flight)
    __builtin_amdgcn_sched_barrier(0);
    after_first_issue();
    if (full) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int pc = lane + 64 * i;
            if (pc < rb) reinterpret_cast<uint4*>(sblk)[pc] = sv[i];
        }
    }
    const uint8_t* srow = sblk + (r - r0) * (uint32_t)rb;  // (full groups only)
#pragma unroll
    for (int j0 = 0; j0 < NJ; j0 += kB) {
        __builtin_amdgcn_sched_barrier(0);
        if (j0 + kB < NJ) issue(j0 + kB);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = j0; j < (j0 + kB < NJ ? j0 + kB : NJ); ++j) {
            const bool ok = 128 * j + 32 * kq < cols;
            const uint32_t scj = full ? (uint32_t)*reinterpret_cast<const uint16_t*>(srow + (ok ? 8 * j + 2 * kq : 0)) : sc[j];
            const h2 sp = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(ok ? scj : 0u, 1.0f, false);
            const uint32_t w4[4] = {q[j].x, q[j].y, q[j].z, q[j].w};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const h2 s = (d < 2) ? h2{sp.x, sp.x} : h2{sp.y, sp.y};
                const h2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w4[d], 1.0f, 0) * s;
                const h2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w4[d], 1.0f, 1) * s;
                const h2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w4[d], 1.0f, 2) * s;
                const h2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w4[d], 1.0f, 3) * s;
                const h8 wf = {p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
                h8 xf = {0, 0, 0, 0, 0, 0, 0, 0};
                if (m16 < NT) xf = *reinterpret_cast<const h8*>(xs + m16 * P + 128 * j + 32 * kq + 8 * d);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf, xf, acc, 0, 0, 0);
            }
        }
    }
    return acc;
}

// NVFP4 GEMV on MFMA for up to four tokens: logits[t][v] = g * sum_k W[v][k] x[t][k].
// v_mfma_f32_16x16x32_f16 with the weight rows as the 16-row operand and the
// tokens as the 16-column operand (columns past T are zero).  A wave owns a
// group of 16 rows at a time and issues every load of the group (NJ 16-byte
// code pieces and NJ scale pairs per lane) before it computes; lane (m, kq)
// takes bytes 64 j + 16 kq .. +15 of row m (k 128 j + 32 kq .. +31), and MFMA
// step (j, d) sums k 128 j + 32 kq + 8 d .. +7 on both operands.  Weights
// decode exactly to fp16 (e2m1 * e4m3 has at most six significant bits).
// x sits in LDS as fp16 after scaling token t by a power of two that puts
// its largest magnitude in [2^14, 2^15): no fp16 overflow, every bf16 value
// at least 2^-28 of that maximum is exact, and the result is scaled back
// exactly.  Persistent grid: wave w of workgroup b takes groups b*4+w,
// stepping by 4*gridDim.  Each workgroup leaves its best (logit, row) key
// per token in the workspace for k_argmax_reduce.
constexpr int kGemvMaxCols = 4096;
template <int NJ, int T>
__global__ __launch_bounds__(256, 3) void k_gemv_mfma(GemvArgs a) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    typedef float f4 __attribute__((ext_vector_type(4)));
    __shared__ __attribute__((aligned(16))) _Float16 xs[T][kGemvMaxCols + 8];
    static_assert(128 * (NJ - 1) + 32 * 3 + 8 * 3 + 8 <= kGemvMaxCols + 8, "LDS reads stay in the row");
    __shared__ float s_amax[4][T];
    __shared__ int s_exp[T];
    __shared__ __attribute__((aligned(16))) uint4 s_sblk[4][kGemvMaxCols / 16];  // each wave's group scales
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int cols = a.cols;
    uint8_t* sblk = reinterpret_cast<uint8_t*>(&s_sblk[wave][0]);

    // x -> registers in 16-byte pieces (one pass, every load in flight at
    // once), per-token largest magnitude, power-of-two scale, fp16 into LDS;
    // it runs once the first weight batch of the wave's first group is in
    // flight, so the weight stream starts at the first instruction
    auto x_setup = [&]()
    {
        constexpr int kXP = (T * kGemvMaxCols / 8 + 255) / 256;
        const int per_t = cols / 8, total = T * per_t;
        uint4 xv[kXP];
#pragma unroll
        for (int i = 0; i < kXP; ++i) {
            const int p = threadIdx.x + 256 * i;
            xv[i] = p < total ? *reinterpret_cast<const uint4*>(a.x + (size_t)p * 8) : make_uint4(0u, 0u, 0u, 0u);
        }
        float m[T];
#pragma unroll
        for (int t = 0; t < T; ++t) m[t] = 0.f;
#pragma unroll
        for (int i = 0; i < kXP; ++i) {
            const int p = threadIdx.x + 256 * i;
            const int tp = p / per_t;
            const uint32_t w[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
            float mx = 0.f;
#pragma unroll
            for (int d = 0; d < 4; ++d)
                mx = fmaxf(mx, fmaxf(fabsf(bf16_bits_to_f32(w[d] & 0xffffu)), fabsf(bf16_bits_to_f32(w[d] >> 16))));
#pragma unroll
            for (int t = 0; t < T; ++t)
                if (tp == t) m[t] = fmaxf(m[t], mx);
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) m[t] = fmaxf(m[t], __shfl_xor(m[t], o, 64));
            if (lane == 0) s_amax[wave][t] = m[t];
        }
        __syncthreads();
        if (threadIdx.x < T) {
            const float mx = fmaxf(fmaxf(s_amax[0][threadIdx.x], s_amax[1][threadIdx.x]),
                                   fmaxf(s_amax[2][threadIdx.x], s_amax[3][threadIdx.x]));
            s_exp[threadIdx.x] = fp16_stage_exp(mx);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kXP; ++i) {
            const int p = threadIdx.x + 256 * i;
            if (p < total) {
                const int tp = p / per_t, k0 = (p - tp * per_t) * 8;
                const float sc = ldexpf(1.0f, s_exp[tp]);
                const uint32_t w[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
                h8 hv;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    hv[2 * d] = (_Float16)(bf16_bits_to_f32(w[d] & 0xffffu) * sc);
                    hv[2 * d + 1] = (_Float16)(bf16_bits_to_f32(w[d] >> 16) * sc);
                }
                *reinterpret_cast<h8*>(&xs[tp][k0]) = hv;
            }
        }
        // zeros past the row: reads of pieces past the end stay finite
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll 1
            for (int k = cols + threadIdx.x; k < kGemvMaxCols + 8; k += 256) xs[t][k] = (_Float16)0.f;
        __syncthreads();
    };
    const int m16 = lane & 15, kq = lane >> 4;
    const int n = m16;  // token column of this lane in the 16-column operand
    unsigned long long best = 0ull;
    const int groups = (a.rows + 15) / 16;
    // every wave takes part in x_setup's barriers: a wave without a group of
    // its own computes the last group and stores nothing
    int grp = blockIdx.x * 4 + wave;
    const bool first_own = grp < groups;
    const int grp0 = first_own ? grp : groups - 1;
    f4 acc = mfma_gemv_group<NJ, T, kGemvMaxCols + 8>(a.codes, a.scales, (uint32_t)min(grp0 * 16 + m16, a.rows - 1),
                                                      cols, &xs[0][0], m16, kq, x_setup, sblk, (uint32_t)(grp0 * 16),
                                                      grp0 * 16 + 16 <= a.rows);
    const float g = *a.gscale;
    int unexp = 0;
#pragma unroll
    for (int t = 0; t < T; ++t)
        if (n == t) unexp = -s_exp[t];
    for (; grp < groups; grp += gridDim.x * 4) {
        if (grp != blockIdx.x * 4 + wave) {
            const uint32_t r = (uint32_t)min(grp * 16 + m16, a.rows - 1);
            acc = mfma_gemv_group<NJ, T, kGemvMaxCols + 8>(a.codes, a.scales, r, cols, &xs[0][0], m16, kq, [] {}, sblk,
                                                           (uint32_t)(grp * 16), grp * 16 + 16 <= a.rows);
        }
        // lane holds rows grp*16 + 4 kq + r of token n
        if (n < T) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int row = grp * 16 + 4 * kq + rr;
                if (row < a.rows) {
                    const float l = ldexpf(acc[rr], unexp) * g;
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
    // this workgroup's best key per token; k_argmax_reduce merges them after
    // the launch (a kernel boundary orders the stores: no fences, no atomics)
    if (threadIdx.x < T) {
        unsigned long long v = 0ull;
        for (int wv = 0; wv < 4; ++wv) v = sbest[wv][threadIdx.x] > v ? sbest[wv][threadIdx.x] : v;
        a.keys[(size_t)blockIdx.x * T + threadIdx.x] = v;
    }
}

// argmax[t] = the row of the largest key over the nblocks per-workgroup keys
// (key = order(logit) << 32 | ~row: the largest logit, then the lowest row).
__global__ __launch_bounds__(256) void k_argmax_reduce(const unsigned long long* keys, int nblocks, int T,
                                                       int32_t* argmax) {
    __shared__ unsigned long long sm[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int t = 0; t < T; ++t) {
        unsigned long long v = 0ull;
        for (int b = threadIdx.x; b < nblocks; b += 256) {
            const unsigned long long k = keys[(size_t)b * T + t];
            v = k > v ? k : v;
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const unsigned long long w = __shfl_xor(v, o, 64);
            v = w > v ? w : v;
        }
        if (lane == 0) sm[wave] = v;
        __syncthreads();
        if (threadIdx.x == 0) {
            unsigned long long m = sm[0];
            for (int i = 1; i < 4; ++i) m = sm[i] > m ? sm[i] : m;
            argmax[t] = (int32_t)(0xffffffffu - (uint32_t)(m & 0xffffffffull));
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Routed MoE for 2..8 tokens on MFMA (the four-token verify step of "Let's
// optimize Nemotron 3.5 Lightning - a worklog", Step 5, and a few concurrent
// sequences), NVFP4 weights.  Each distinct selected expert is streamed
// once: the block set of the first (token, slot) pair that selected it
// computes the expert for every token (MFMA columns are free up to 16) and
// writes the results of every pair that selected it.  TM (4 or 8) is the
// instance's token capacity.  A4: the W4A4 form (Step 3: activations
// quantized to NVFP4 on the fly): x and h are quantized per 16-block and
// their decoded values (e2m1 * e4m3, exact in fp16) are the MFMA columns.
// ---------------------------------------------------------------------------
constexpr int kSmallT = 4;   // tokens at most for the small-batch W4A16 path
constexpr int kSmallT8 = 8;  // capacity of the wider instances

struct SmallMoeArgs {
    int E, H, I, K, T;
    const uint8_t* upc;
    const uint8_t* ups;
    const float* upg;
    const uint8_t* dnc;
    const uint8_t* dns;
    const float* dng;
    const uint16_t* x;   // [T][H] bf16
    const int32_t* ids;  // [T][K]
    const float* w;      // [T][K]
    float* h;            // [T*K][I] fp32
    float* zw;           // [T*K][H] fp32: w * g * z per pair
    float* y32;          // [T][H]
    uint16_t* y;         // [T][H] bf16
    // routing done by k_small_up itself from the logits (the top-k of every
    // token in every workgroup; workgroup (0, 0) stores it for the others)
    RouterArgs ra;
    const float* zsh;    // [T][H] the shared expert's output (nullable)
    // A4 code taps: x codes [T][H/2] and scales [T][H/16], h codes
    // [T*K][I/2] and scales [T*K][I/16] (unused otherwise)
    uint8_t* xq_codes;
    uint8_t* xq_scales;
    uint8_t* hq_codes;
    uint8_t* hq_scales;
};

// The expert of pair p, and whether p is the first pair that selected it.
__device__ __forceinline__ int small_expert(const SmallMoeArgs& a, const int32_t* ids, int p, bool& leader) {
    const int e = min(max(ids[p], 0), a.E - 1);  // routing ids are always in range; never read outside the bank
    leader = true;
    for (int q = 0; q < p; ++q)
        if (min(max(ids[q], 0), a.E - 1) == e) leader = false;
    return e;
}

// Largest magnitude of each of TM rows' values (per-thread partials ->
// block), turned into the row's fp16 staging exponent.
template <int TM>
__device__ __forceinline__ void block_amax(float (&m)[TM], float (*s_amax)[TM], int* s_exp) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int t = 0; t < TM; ++t) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) m[t] = fmaxf(m[t], __shfl_xor(m[t], o, 64));
        if (lane == 0) s_amax[wave][t] = m[t];
    }
    __syncthreads();
    if (threadIdx.x < TM) {
        const float mx = fmaxf(fmaxf(s_amax[0][threadIdx.x], s_amax[1][threadIdx.x]),
                               fmaxf(s_amax[2][threadIdx.x], s_amax[3][threadIdx.x]));
        s_exp[threadIdx.x] = fp16_stage_exp(mx);
    }
    __syncthreads();
}

// NVFP4 quantization of a block of 16 values held by four adjacent lanes
// (4 values each, the block's first lane at a multiple of 4): the block
// maximum over the quad (quad_perm [1,0,3,2], then [2,3,0,1]); code packs
// the lane's 4 codes.  The same rule as nvfp4_quant16.
struct Nvfp4Quarter {
    uint32_t sb, code;
};
__device__ __forceinline__ Nvfp4Quarter nvfp4_quant4_quad(const float (&v)[4]) {
    float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    amax = fmaxf(amax, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, amax), 0xB1, 0xF, 0xF, true)));
    amax = fmaxf(amax, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, amax), 0x4E, 0xF, 0xF, true)));
    Nvfp4Quarter b;
    b.sb = e4m3fn_rne_sat(__fdiv_rn(amax, 6.0f));
    const E2m1Thresholds th = e2m1_thresholds(e4m3fn_to_f32(b.sb));
    b.code = 0u;
#pragma unroll
    for (int k = 0; k < 4; ++k) b.code |= (e2m1_code(fabsf(v[k]), th) | ((__float_as_uint(v[k]) >> 31) << 3)) << (4 * k);
    return b;
}

// Rows 0..TM-1 of an LDS operand (pitch P fp16) from up to TM bf16 rows of
// `cols` values (row t at src + t * cols); rows past `rows` and columns past
// `cols` are zero.  One pass of 16-byte loads, all in flight at once.
//  - W4A16: row t is scaled by 2^s_exp[t], the power of two that puts its
//    largest magnitude in [2^14, 2^15), and rounded to fp16 (exact for every
//    bf16 value at least 2^-28 of that maximum);
//  - A4: each 16-block is quantized to NVFP4 (two adjacent lanes per block)
//    and its decoded values stored (exact in fp16); s_exp = 0; codes and
//    scales go to xq_codes / xq_scales when they are not null.
template <int P, int TM, bool A4>
__device__ __forceinline__ void stage_bf16_rows(const uint16_t* src, int rows, int cols, _Float16* xs,
                                                float (*s_amax)[TM], int* s_exp, uint8_t* xq_codes,
                                                uint8_t* xq_scales) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    constexpr int kXP = (TM * (P / 8) + 255) / 256;
    const int per = cols / 8, total = rows * per;
    uint4 v[kXP];
#pragma unroll
    for (int i = 0; i < kXP; ++i) {
        const int p = threadIdx.x + 256 * i;
        v[i] = p < total ? *reinterpret_cast<const uint4*>(src + (size_t)p * 8) : make_uint4(0u, 0u, 0u, 0u);
    }
    if constexpr (A4) {
        if (threadIdx.x < TM) s_exp[threadIdx.x] = 0;
#pragma unroll
        for (int i = 0; i < kXP; ++i) {
            const int p = threadIdx.x + 256 * i;
            const int t = p / per, k0 = (p - t * per) * 8;
            const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
            float f[8];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                f[2 * d] = bf16_bits_to_f32(w[d] & 0xffffu);
                f[2 * d + 1] = bf16_bits_to_f32(w[d] >> 16);
            }
            const Nvfp4Half b = nvfp4_quant8_pair(f);  // (both lanes of a block run it)
            float dq[8];
            nvfp4_dequant8(b, dq);
            if (p < total) {
                h8 hv;
#pragma unroll
                for (int d = 0; d < 8; ++d) hv[d] = (_Float16)dq[d];
                *reinterpret_cast<h8*>(xs + t * P + k0) = hv;
                if (xq_codes) {
                    *reinterpret_cast<uint32_t*>(xq_codes + (size_t)t * (cols / 2) + k0 / 2) = b.code;
                    if ((p & 1) == 0) xq_scales[(size_t)t * (cols / 16) + k0 / 16] = (uint8_t)b.sb;
                }
            }
        }
    } else {
        float m[TM];
#pragma unroll
        for (int t = 0; t < TM; ++t) m[t] = 0.f;
#pragma unroll
        for (int i = 0; i < kXP; ++i) {
            const int t = (threadIdx.x + 256 * i) / per;
            const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
            float mx = 0.f;
#pragma unroll
            for (int d = 0; d < 4; ++d)
                mx = fmaxf(mx, fmaxf(fabsf(bf16_bits_to_f32(w[d] & 0xffffu)), fabsf(bf16_bits_to_f32(w[d] >> 16))));
#pragma unroll
            for (int tt = 0; tt < TM; ++tt)
                if (t == tt) m[tt] = fmaxf(m[tt], mx);
        }
        block_amax<TM>(m, s_amax, s_exp);
#pragma unroll
        for (int i = 0; i < kXP; ++i) {
            const int p = threadIdx.x + 256 * i;
            if (p < total) {
                const int t = p / per, k0 = (p - t * per) * 8;
                const float sc = ldexpf(1.0f, s_exp[t]);
                const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
                h8 hv;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    hv[2 * d] = (_Float16)(bf16_bits_to_f32(w[d] & 0xffffu) * sc);
                    hv[2 * d + 1] = (_Float16)(bf16_bits_to_f32(w[d] >> 16) * sc);
                }
                *reinterpret_cast<h8*>(xs + t * P + k0) = hv;
            }
        }
    }
    // zeros: rows past `rows`, and columns past `cols` (8-aligned pieces)
    const h8 z = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int i = threadIdx.x; i < TM * (P / 8); i += 256) {
        const int t = i / (P / 8), k0 = (i - t * (P / 8)) * 8;
        if (t >= rows || k0 >= cols) *reinterpret_cast<h8*>(xs + t * P + k0) = z;
    }
    __syncthreads();
}

// Columns c < nc of an LDS operand as fp16 hi (row c) and lo (row TM + c)
// parts of the fp32 rows src + col_off[c] (`cols` values); other rows and
// columns past `cols` are zero.
//  - W4A16: row c is scaled by 2^s_exp[c] (largest magnitude into [2^14,
//    2^15)); hi = fp16(v), lo = fp16(v - hi), so hi + lo carries v to about
//    2^-22;
//  - A4: each 16-block is quantized to NVFP4 (four adjacent lanes per block)
//    and hi holds its decoded values (exact in fp16), lo zero; s_exp = 0;
//    codes and scales of column c go to row pair[c] of hq_codes / hq_scales
//    when they are not null.
template <int P, int TM, bool A4>
__device__ __forceinline__ void stage_f32_hilo(const float* src, const size_t (&col_off)[TM], int nc, int cols,
                                               _Float16* hs, float (*s_amax)[TM], int* s_exp,
                                               const int (&pair)[TM], uint8_t* hq_codes, uint8_t* hq_scales) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    constexpr int kXP = (TM * (P / 4) + 255) / 256;
    const int per = cols / 4, total = nc * per;
    float4 v[kXP];
#pragma unroll
    for (int i = 0; i < kXP; ++i) {
        const int p = threadIdx.x + 256 * i;
        const int c = p / per;
        size_t off = col_off[0];
#pragma unroll
        for (int cc = 1; cc < TM; ++cc)
            if (c == cc) off = col_off[cc];
        v[i] = p < total ? *reinterpret_cast<const float4*>(src + off + (size_t)(p - c * per) * 4)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const h4 z = {0, 0, 0, 0};
    if constexpr (A4) {
        if (threadIdx.x < TM) s_exp[threadIdx.x] = 0;
#pragma unroll
        for (int i = 0; i < kXP; ++i) {
            const int p = threadIdx.x + 256 * i;
            const int c = p / per, k0 = (p - c * per) * 4;
            const float f[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
            const Nvfp4Quarter b = nvfp4_quant4_quad(f);  // (all four lanes of a block run it)
            if (p < total) {
                const float s = e4m3fn_to_f32(b.sb);
                const f32x2 d0 = fp4x2_f32<0>(b.code), d1 = fp4x2_f32<1>(b.code);
                const h4 hv = {(_Float16)(d0[0] * s), (_Float16)(d0[1] * s), (_Float16)(d1[0] * s),
                               (_Float16)(d1[1] * s)};
                *reinterpret_cast<h4*>(hs + c * P + k0) = hv;
                *reinterpret_cast<h4*>(hs + (TM + c) * P + k0) = z;
                if (hq_codes) {
                    int pr = pair[0];
#pragma unroll
                    for (int cc = 1; cc < TM; ++cc)
                        if (c == cc) pr = pair[cc];
                    *reinterpret_cast<uint16_t*>(hq_codes + (size_t)pr * (cols / 2) + k0 / 2) = (uint16_t)b.code;
                    if ((p & 3) == 0) hq_scales[(size_t)pr * (cols / 16) + k0 / 16] = (uint8_t)b.sb;
                }
            }
        }
        __syncthreads();  // (s_exp)
    } else {
        float m[TM];
#pragma unroll
        for (int t = 0; t < TM; ++t) m[t] = 0.f;
#pragma unroll
        for (int i = 0; i < kXP; ++i) {
            const int c = (threadIdx.x + 256 * i) / per;
            const float mx = fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w)));
#pragma unroll
            for (int cc = 0; cc < TM; ++cc)
                if (c == cc) m[cc] = fmaxf(m[cc], mx);
        }
        block_amax<TM>(m, s_amax, s_exp);
#pragma unroll
        for (int i = 0; i < kXP; ++i) {
            const int p = threadIdx.x + 256 * i;
            if (p < total) {
                const int c = p / per, k0 = (p - c * per) * 4;
                const float sc = ldexpf(1.0f, s_exp[c]);
                const float f[4] = {v[i].x * sc, v[i].y * sc, v[i].z * sc, v[i].w * sc};
                h4 hi, lo;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    hi[d] = (_Float16)f[d];
                    lo[d] = (_Float16)(f[d] - (float)hi[d]);
                }
                *reinterpret_cast<h4*>(hs + c * P + k0) = hi;
                *reinterpret_cast<h4*>(hs + (TM + c) * P + k0) = lo;
            }
        }
    }
    for (int i = threadIdx.x; i < 2 * TM * (P / 4); i += 256) {
        const int rr = i / (P / 4), k0 = (i - rr * (P / 4)) * 4;
        if ((rr % TM) >= nc || k0 >= cols) *reinterpret_cast<h4*>(hs + rr * P + k0) = z;
    }
    __syncthreads();
}

// up: u = W_up[e] x_t for all tokens t, h[pair] = relu(g u)^2 for every pair
// (t, slot) that selected e.  Grid (ceil(I/64), T*K): 64 rows per block, one
// 16-row group per wave.  x goes to LDS as fp16 (scaled per token by a power
// of two, as in the lm_head GEMV; A4: NVFP4-quantized and decoded).
template <int NJ, int TM, bool A4>
__global__ __launch_bounds__(256, 2) void k_small_up(SmallMoeArgs a) {
    constexpr int P = 128 * NJ + 8;
    __shared__ __attribute__((aligned(16))) _Float16 xs[TM][P];
    __shared__ float s_amax[4][TM];
    __shared__ int s_exp[TM];
    __shared__ __attribute__((aligned(16))) uint4 s_sblk[4][NJ * 8];  // each wave's group scales (16 rows)
    __shared__ int32_t s_ids[TM * 8];
    __shared__ float s_w[TM * 8];
    // routing: wave w takes tokens w, w + 4 (every workgroup, so no top-k launch)
    for (int t = (int)(threadIdx.x >> 6); t < a.T; t += 4)
        topk_token(a.ra, t, blockIdx.x == 0 && blockIdx.y == 0, &s_ids[t * a.K], &s_w[t * a.K]);
    __syncthreads();
    bool leader;
    const int e = small_expert(a, s_ids, blockIdx.y, leader);
    if (!leader) return;  // uniform
    const bool tap = A4 && blockIdx.x == 0 && blockIdx.y == 0;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m16 = lane & 15, kq = lane >> 4;
    const int row = blockIdx.x * 64 + wave * 16 + m16;
    const uint32_t wrow = (uint32_t)e * a.I + min(row, a.I - 1);
    const int row0 = blockIdx.x * 64 + wave * 16;
    // x goes to LDS while the first weight batch is in flight
    const f32x4g acc = mfma_gemv_group<NJ, TM, P>(
        a.upc, a.ups, wrow, a.H, &xs[0][0], m16, kq,
        [&] {
            stage_bf16_rows<P, TM, A4>(a.x, a.T, a.H, &xs[0][0], s_amax, s_exp, tap ? a.xq_codes : nullptr,
                                       tap ? a.xq_scales : nullptr);
        },
        reinterpret_cast<uint8_t*>(&s_sblk[wave][0]), (uint32_t)e * a.I + (uint32_t)row0, row0 + 16 <= a.I);
    // lane (n = m16, kq) holds rows 4 kq + r of token n
    const int n = m16;
    if (n < a.T) {
        int pp = -1;
        for (int sl = 0; sl < a.K; ++sl)
            if (min(max(s_ids[n * a.K + sl], 0), a.E - 1) == e) pp = n * a.K + sl;
        if (pp >= 0) {
            const float ge = a.upg[e];
            const int unexp = -s_exp[n];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rr = blockIdx.x * 64 + wave * 16 + 4 * kq + r;
                if (rr < a.I) {
                    const float u = fmaxf(ldexpf(acc[r], unexp) * ge, 0.f);
                    a.h[(size_t)pp * a.I + rr] = u * u;
                }
            }
        }
    }
}

// down: z = W_down[e] h_pair for every pair that selected e, zw[pair] =
// w * g * z.  Grid (ceil(H/64), T*K).  Each pair's fp32 h is scaled by a power
// of two and split into fp16 hi + lo (h' = hi + lo to about 2^-22), columns c
// and TM + c of the same MFMA, so h keeps nearly fp32 precision at no extra
// MFMA cost (A4: the decoded NVFP4 h in column c, column TM + c zero).
template <int NJ, int TM, bool A4>
__global__ __launch_bounds__(256, 2) void k_small_down(SmallMoeArgs a) {
    constexpr int P = 128 * NJ + 8;
    __shared__ __attribute__((aligned(16))) _Float16 hs[2 * TM][P];
    __shared__ float s_amax[4][TM];
    __shared__ int s_exp[TM];
    // each wave's group scales (16 rows), where the instance has room for them
    constexpr bool kScaleLds = NJ <= 24;
    __shared__ __attribute__((aligned(16))) uint4 s_sblk[4][kScaleLds ? NJ * 8 : 1];
    bool leader;
    const int e = small_expert(a, a.ids, blockIdx.y, leader);
    if (!leader) return;  // uniform
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m16 = lane & 15, kq = lane >> 4;
    const int row = blockIdx.x * 64 + wave * 16 + m16;
    const uint32_t wrow = (uint32_t)e * a.H + min(row, a.H - 1);
    // columns: the pairs that selected e, in pair order (one per token at most)
    // (static indices only, so the list stays in registers)
    int cols[TM];
#pragma unroll
    for (int c = 0; c < TM; ++c) cols[c] = 0;
    int nc = 0;
    for (int pp = 0; pp < a.T * a.K; ++pp) {
        if (min(max(a.ids[pp], 0), a.E - 1) == e) {
#pragma unroll
            for (int c = 0; c < TM; ++c)
                if (c == nc) cols[c] = pp;
            nc = min(nc + 1, TM);
        }
    }
    size_t col_off[TM];
#pragma unroll
    for (int c = 0; c < TM; ++c) col_off[c] = (size_t)cols[c] * a.I;
    const bool tap = A4 && blockIdx.x == 0;
    // h goes to LDS while the first weight batch is in flight
    // (the widest instances have no LDS left for the scale slice: their
    // scales load per piece)
    const int row0 = blockIdx.x * 64 + wave * 16;
    const f32x4g acc = mfma_gemv_group<NJ, 2 * TM, P>(
        a.dnc, a.dns, wrow, a.I, &hs[0][0], m16, kq,
        [&] {
            stage_f32_hilo<P, TM, A4>(a.h, col_off, nc, a.I, &hs[0][0], s_amax, s_exp, cols,
                                      tap ? a.hq_codes : nullptr, tap ? a.hq_scales : nullptr);
        },
        reinterpret_cast<uint8_t*>(&s_sblk[wave][0]), (uint32_t)e * a.H + (uint32_t)row0,
        kScaleLds && row0 + 16 <= a.H);
    // lane (n, kq) holds column n: hi for n < TM, lo for n >= TM; add lane n + TM's lo
    const int n = m16;
    float z[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) z[r] = acc[r] + __shfl(acc[r], (n < TM) ? lane + TM : lane, 64);
    if (n < nc) {
        int pp = cols[0];
#pragma unroll
        for (int c = 1; c < TM; ++c)
            if (c == n) pp = cols[c];
        const float wg = a.w[pp] * a.dng[e];
        const int unexp = -s_exp[n];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rr = blockIdx.x * 64 + wave * 16 + 4 * kq + r;
            if (rr < a.H) a.zw[(size_t)pp * a.H + rr] = ldexpf(z[r], unexp) * wg;
        }
    }
}

// y32[t][r] = sum over slots s (in order) of zw[t*K + s][r]; y = bf16 (RNE).
__global__ __launch_bounds__(256) void k_small_combine(SmallMoeArgs a) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= a.T * a.H) return;
    const int t = i / a.H, r = i - t * a.H;
    float acc = 0.f;
    for (int sl = 0; sl < a.K; ++sl) acc += a.zw[(size_t)(t * a.K + sl) * a.H + r];
    if (a.zsh) acc += a.zsh[i];  // the shared expert, after the routed slots
    a.y32[i] = acc;
    a.y[i] = (uint16_t)f32_to_bf16_rne(acc);
}

// Zero fill (used instead of a memset so a caller may capture it in a graph).
__global__ __launch_bounds__(256) void k_zero(uint4* p, size_t n16) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace q4moe
