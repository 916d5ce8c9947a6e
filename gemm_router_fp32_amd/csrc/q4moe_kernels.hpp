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

enum : int { FMT_NVFP4 = 1, FMT_INT4 = 2 };

// Control words at the start of every workspace.
enum : int { CTRL_TICKET = 0, CTRL_FLAGS = 1, CTRL_WORDS = 256 };

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

// logits[t][e] = sum_c W_g[e][c] * x[t][c]: one wave per expert and up to
// four tokens; grid (ceil(E/4), ceil(T/4)), 256 threads.
__global__ __launch_bounds__(256) void k_router_logits(RouterArgs a) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e = blockIdx.x * 4 + wave;
    const int t0 = blockIdx.y * 4;
    if (e >= a.E) return;  // wave-uniform
    const int nt = min(4, a.T - t0);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    const float4* wr = reinterpret_cast<const float4*>(a.wg + (size_t)e * a.H);
    for (int j = lane; j < a.H / 4; j += kWave) {
        const float4 wv = wr[j];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (t < nt) {
                const uint2 xb = *reinterpret_cast<const uint2*>(a.x + (size_t)(t0 + t) * a.H + 4 * j);
                acc[t] = __builtin_fmaf(wv.x, bf16_bits_to_f32(xb.x & 0xffffu), acc[t]);
                acc[t] = __builtin_fmaf(wv.y, bf16_bits_to_f32(xb.x >> 16), acc[t]);
                acc[t] = __builtin_fmaf(wv.z, bf16_bits_to_f32(xb.y & 0xffffu), acc[t]);
                acc[t] = __builtin_fmaf(wv.w, bf16_bits_to_f32(xb.y >> 16), acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const float l = seg_sum<64>(acc[t]);
        if (lane == 0 && t < nt) {
            a.logits[(size_t)(t0 + t) * a.E + e] = l;
            if (a.logits_out) a.logits_out[(size_t)(t0 + t) * a.E + e] = l;
        }
    }
}

// Sigmoid scores, selection key score + bias, top-K by key (largest first,
// equal keys -> lower index), gates = selected scores / their sum.
// One wave per token (E <= 256: four experts per lane); grid ceil(T/4).
__global__ __launch_bounds__(256) void k_topk(RouterArgs a) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wave;
    if (t >= a.T) return;  // wave-uniform
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
    float sel_s[8];
    int sel_i[8];
    float ssum = 0.f;
    for (int i = 0; i < a.K; ++i) {
        float bk = -__builtin_inff();
        int bi = 0x7fffffff;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = lane + kWave * q;
            if (live[q] && (key[q] > bk || (key[q] == bk && e < bi))) {
                bk = key[q];
                bi = e;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ok = __shfl_xor(bk, off, 64);
            const int oi = __shfl_xor(bi, off, 64);
            if (ok > bk || (ok == bk && oi < bi)) {
                bk = ok;
                bi = oi;
            }
        }
        const int owner = bi & 63, slot = bi >> 6;
        float mine = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (lane == owner && slot == q) {
                mine = s[q];
                live[q] = false;
            }
        const float sb = __shfl(mine, owner, 64);
        sel_s[i] = sb;
        sel_i[i] = bi;
        ssum += sb;
    }
    if (lane < a.K) {
        float ws = 0.f;
        int wi = 0;
        for (int i = 0; i < a.K; ++i)
            if (i == lane) {
                ws = sel_s[i];
                wi = sel_i[i];
            }
        const float wv = ws / ssum;
        const size_t o = (size_t)t * a.K + lane;
        a.ids[o] = wi;
        a.w[o] = wv;
        if (a.ids_out) a.ids_out[o] = wi;
        if (a.w_out) a.w_out[o] = wv;
    }
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
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) s += bf16_bits_to_f32(xa[j] & 0xffffu) + bf16_bits_to_f32(xa[j] >> 16);
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
                    acc += nvfp4_chunk_bf16(q, xa[c], e4m3fn_to_f32(sb & 0xffu), e4m3fn_to_f32(sb >> 8));
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
                        z += nvfp4_chunk_f32(q, hv[c], e4m3fn_to_f32(sb & 0xffu), e4m3fn_to_f32(sb >> 8));
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
    unsigned long long* keys;  // [T] workspace, zero between calls
    uint32_t* ctrl;          // workspace control words
};

// Order-preserving map of fp32 onto uint32 (larger float -> larger integer).
__device__ __forceinline__ uint32_t f32_order(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 32-lane segments, two rows per wave per pass, 8 passes: 64 rows per block.
template <int C, int T>
__global__ __launch_bounds__(256) void k_gemv(GemvArgs a) {
    constexpr int kPasses = 8;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int seg = lane >> 5, li = lane & 31;
    const int nch = a.cols / 32;
    uint32_t xa[T][C][16];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int ch = li * C + c;
            if (ch < nch)
                load_x_chunk(a.x + (size_t)t * a.cols, ch, xa[t][c]);
            else
#pragma unroll
                for (int j = 0; j < 16; ++j) xa[t][c][j] = 0u;
        }
    const float g = *a.gscale;
    unsigned long long best[T];
#pragma unroll
    for (int t = 0; t < T; ++t) best[t] = 0ull;

    for (int ps = 0; ps < kPasses; ++ps) {
        const int r = (blockIdx.x * kPasses + ps) * 8 + wave * 2 + seg;
        const bool rowok = r < a.rows;
        float acc[T];
#pragma unroll
        for (int t = 0; t < T; ++t) acc[t] = 0.f;
        if (rowok) {
            const uint8_t* rc = a.codes + (size_t)r * (a.cols / 2);
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const int ch = li * C + c;
                if (ch < nch) {
                    const uint4 q = ldg16(rc + ch * 16);
                    const uint32_t sb =
                        *reinterpret_cast<const uint16_t*>(a.scales + (size_t)r * (a.cols / 16) + ch * 2);
                    const float s0 = e4m3fn_to_f32(sb & 0xffu), s1 = e4m3fn_to_f32(sb >> 8);
#pragma unroll
                    for (int t = 0; t < T; ++t) acc[t] += nvfp4_chunk_bf16(q, xa[t][c], s0, s1);
                }
            }
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const float l = seg_sum<32>(acc[t]) * g;
            if (li == 0 && rowok) {
                a.logits[(size_t)t * a.rows + r] = l;
                const unsigned long long key =
                    ((unsigned long long)f32_order(l) << 32) | (unsigned long long)(0xffffffffu - (uint32_t)r);
                best[t] = key > best[t] ? key : best[t];
            }
        }
    }
    // block-level maximum of the keys, then one atomic per token per block
    __shared__ unsigned long long sbest[8][T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        unsigned long long v = best[t];
        const unsigned long long o = __shfl_xor(v, 32, 64);
        v = o > v ? o : v;
        if (lane == 0) sbest[wave][t] = v;
    }
    __syncthreads();
    if (threadIdx.x < T) {
        unsigned long long v = 0ull;
        for (int wv = 0; wv < 4; ++wv) v = sbest[wv][threadIdx.x] > v ? sbest[wv][threadIdx.x] : v;
        atomicMax(a.keys + threadIdx.x, v);
    }
    // the last block to finish publishes the argmax and clears the keys
    __shared__ bool last;
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) last = atomicAdd(a.ctrl + CTRL_TICKET, 1u) == gridDim.x - 1;
    __syncthreads();
    if (last) {
        __threadfence();
        if (threadIdx.x < T) {
            const unsigned long long k = atomicExch(a.keys + threadIdx.x, 0ull);
            if (a.argmax) a.argmax[threadIdx.x] = (int32_t)(0xffffffffu - (uint32_t)(k & 0xffffffffull));
        }
        if (threadIdx.x == 0) atomicExch(a.ctrl + CTRL_TICKET, 0u);
    }
}

// Zero fill (used instead of a memset so a caller may capture it in a graph).
__global__ __launch_bounds__(256) void k_zero(uint4* p, size_t n16) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace q4moe
