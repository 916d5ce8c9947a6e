// W4A16 routed-MoE for many tokens on gfx950 (mid-batch decode: several
// concurrent sequences through one layer; "Let's optimize Nemotron 3.5
// Lightning - a worklog", "Coming in Part 2: filling the GPU", and
// "Quantization (PTQ + QAD)", "Deployment and Serving": the GEMM backend is
// chosen per batch size).  The weights are NVFP4 or int4-g64 and the
// activations stay at 16 bits or better: x is bf16, h is fp32.
//
// Pipeline (one stream, no host synchronisation):
//   router -> dispatch (per-expert token lists, stable in token order, and
//   the list of experts that have rows) -> x to fp16 -> grouped up GEMM on
//   MFMA (epilogue h = relu(g u)^2, fp32, by (token, slot) pair) -> h to
//   fp16 hi + lo -> grouped down GEMM on MFMA (epilogue w g z per pair) ->
//   sum over the slots in slot order.
//
// Both MFMA operands are fp16 (v_mfma_f32_32x32x16_f16, fp32 accumulate):
//  - x row t is scaled by a power of two 2^s_t that puts its largest
//    magnitude in [2^14, 2^15) and rounded to fp16: exact for every bf16
//    value down to about 2^-28 of the row's maximum;
//  - h row p is scaled the same way and split into hi = fp16(v) and lo =
//    fp16(v - hi), two A rows whose products are summed in the epilogue, so
//    h carries about 22 bits;
//  - NVFP4 weights decode exactly (e2m1 * e4m3 has at most six significant
//    bits in [2^-10, 2688]); the per-tensor g is applied in the epilogue;
//  - int4 weights are code * bf16 group scale; a weight row's scales are
//    first scaled by the power of two 2^sigma that puts their largest
//    magnitude in [2^11, 2^12), so code * scale (at most 11 significant
//    bits, magnitude below 2^15) is exact in fp16 for every scale down to
//    about 2^-25 of the row's largest;
//  - the epilogue undoes every power of two exactly.
#pragma once

#include "q4moe_fused.hpp"
#include "q4moe_w4a4.hpp"

namespace q4moe {

// ---------------------------------------------------------------------------
// fp16 staging of activation rows (one workgroup per row, cols <= 4096).
// ---------------------------------------------------------------------------
struct StageArgs {
    int cols;
    const uint16_t* xb;  // bf16 rows (k_stage_x16, k_stage_fp8<true>)
    const float* hf;     // fp32 rows (k_stage_h16, k_stage_fp8<false>)
    _Float16* out;       // x: [rows][cols]; h: [2 rows][cols], hi then lo of each row (FP8: [rows][cols])
    int32_t* exps;       // [rows]: the power of two each row was scaled by (FP8: 0)
    float iscale;        // FP8: the static input scale
    uint8_t* codes;      // FP8: the E4M3FN codes [rows][cols] (nullable tap)
};

// Largest of the 256 threads' values, returned to every thread.
__device__ __forceinline__ float block_max256(float v, float* s_red) {
    v = wave_max(v);
    if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = v;
    __syncthreads();
    return fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
}

__global__ __launch_bounds__(256) void k_stage_x16(StageArgs a) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    __shared__ float s_red[4];
    const int r = blockIdx.x, per = a.cols / 8;  // 8-value pieces, at most 512
    const uint16_t* src = a.xb + (size_t)r * a.cols;
    uint4 v[2];
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int p = threadIdx.x + 256 * i;
        v[i] = p < per ? *reinterpret_cast<const uint4*>(src + 8 * p) : make_uint4(0u, 0u, 0u, 0u);
        const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
        for (int d = 0; d < 4; ++d)
            mx = fmaxf(mx, fmaxf(fabsf(bf16_bits_to_f32(w[d] & 0xffffu)), fabsf(bf16_bits_to_f32(w[d] >> 16))));
    }
    const int s = fp16_stage_exp(block_max256(mx, s_red));
    if (threadIdx.x == 0) a.exps[r] = s;
    const float sc = ldexpf(1.0f, s);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int p = threadIdx.x + 256 * i;
        if (p < per) {
            const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
            h8 hv;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                hv[2 * d] = (_Float16)(bf16_bits_to_f32(w[d] & 0xffffu) * sc);
                hv[2 * d + 1] = (_Float16)(bf16_bits_to_f32(w[d] >> 16) * sc);
            }
            *reinterpret_cast<h8*>(a.out + (size_t)r * a.cols + 8 * p) = hv;
        }
    }
}

__global__ __launch_bounds__(256) void k_stage_h16(StageArgs a) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    __shared__ float s_red[4];
    const int r = blockIdx.x, per = a.cols / 4;  // 4-value pieces, at most 1024
    const float* src = a.hf + (size_t)r * a.cols;
    float4 v[4];
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = threadIdx.x + 256 * i;
        v[i] = p < per ? *reinterpret_cast<const float4*>(src + 4 * p) : make_float4(0.f, 0.f, 0.f, 0.f);
        mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
    }
    const int s = fp16_stage_exp(block_max256(mx, s_red));
    if (threadIdx.x == 0) a.exps[r] = s;
    const float sc = ldexpf(1.0f, s);
    _Float16* hi_row = a.out + (size_t)(2 * r) * a.cols;
    _Float16* lo_row = hi_row + a.cols;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = threadIdx.x + 256 * i;
        if (p < per) {
            const float f[4] = {v[i].x * sc, v[i].y * sc, v[i].z * sc, v[i].w * sc};
            h4 hi, lo;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                hi[d] = (_Float16)f[d];
                lo[d] = (_Float16)(f[d] - (float)hi[d]);
            }
            *reinterpret_cast<h4*>(hi_row + 4 * p) = hi;
            *reinterpret_cast<h4*>(lo_row + 4 * p) = lo;
        }
    }
}

// FP8 per-tensor activation coding (the shared expert's W8A8 form): each
// value v becomes the E4M3FN code of fl32(v / iscale) (nearest-even,
// saturating at 448, sign kept), staged as its exact fp16 value; one
// workgroup per row, 8 values per thread and pass.
template <bool BF16_IN>
__global__ __launch_bounds__(256) void k_stage_fp8(StageArgs a) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    const int r = blockIdx.x, per = a.cols / 8;
    if (threadIdx.x == 0) a.exps[r] = 0;
    for (int p = threadIdx.x; p < per; p += 256) {
        float v[8];
        if constexpr (BF16_IN) {
            const uint4 q = *reinterpret_cast<const uint4*>(a.xb + (size_t)r * a.cols + 8 * p);
            const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                v[2 * d] = bf16_bits_to_f32(w[d] & 0xffffu);
                v[2 * d + 1] = bf16_bits_to_f32(w[d] >> 16);
            }
        } else {
            const float4 q0 = *reinterpret_cast<const float4*>(a.hf + (size_t)r * a.cols + 8 * p);
            const float4 q1 = *reinterpret_cast<const float4*>(a.hf + (size_t)r * a.cols + 8 * p + 4);
            v[0] = q0.x; v[1] = q0.y; v[2] = q0.z; v[3] = q0.w;
            v[4] = q1.x; v[5] = q1.y; v[6] = q1.z; v[7] = q1.w;
        }
        h8 hv;
        uint32_t cw[2] = {0u, 0u};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t c = fp8_act_code(v[k], a.iscale);
            hv[k] = (_Float16)e4m3fn_to_f32(c);
            cw[k >> 2] |= c << (8 * (k & 3));
        }
        *reinterpret_cast<h8*>(a.out + (size_t)r * a.cols + 8 * p) = hv;
        if (a.codes) *reinterpret_cast<uint2*>(a.codes + (size_t)r * a.cols + 8 * p) = make_uint2(cw[0], cw[1]);
    }
}

// A dense layer as a one-expert dispatch: every token is a row of expert 0
// with gate 1 (the shared expert through the grouped GEMMs).
__global__ __launch_bounds__(256) void k_dispatch_all(int T, int4* act, int32_t* n_act, int32_t* perm, float* gate) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t == 0) {
        act[0] = make_int4(0, 0, T, 0);
        n_act[0] = 1;
    }
    if (t < T) {
        perm[t] = t;
        gate[t] = 1.0f;
    }
}

// ---------------------------------------------------------------------------
// Grouped GEMM with fp16 activations: for expert e and a 128-column output
// tile, out[pair][n] = epi(sum_k A[row][k] W_e[n][k]).  Workgroup: 4 waves,
// wave w owns columns 32w..32w+31 (lane l: column l % 32, k half l / 32 of
// each 256-wide chunk) and one 32-row A tile (v_mfma_f32_32x32x16_f16), in
// M-tiles over the expert's rows: 32 rows per tile, or 16 pairs (32 hi/lo
// rows) for the down GEMM of the 16-bit path.
//
// Weights stream straight into registers, two chunks ahead in a three-slot
// ring (every weight row contributes one 128-byte line per chunk, two for
// FP8); the A pieces (64 bytes of a row per thread and chunk) ride a ring of
// their own and are copied into LDS once per workgroup.  MFMA step j (0..15)
// of a chunk sums k 8j..8j+7 (lanes 0..31) and 128+8j..+7 (lanes 32..63) of
// both operands.  int4 codes unpack as the pairs (e0,e4), (e1,e5), (e2,e6),
// (e3,e7) of each 8-code dword, so the A pieces are stored in that order.
// The block scales of the workgroup's 128 weight rows are copied into LDS
// once (FP8 has one scale per tensor).  Loads past the end of a row (last
// chunk, and the prefetches of the last two chunks) reread the row's last
// bytes and are given scale 0 (B) or zeroed (A).  Workgroups map to the
// experts that have rows (the dispatch's list), expert-major on the XCDs;
// the rest exit at once.
// ---------------------------------------------------------------------------
struct GemmA16Args {
    int N, Kd, K;              // output columns (rows of W_e), reduction length, top-k
    const uint8_t* wc;         // W codes [E][N][Kd/2] (FP8: [E][N][Kd])
    const uint8_t* wsc;        // W scales: E4M3 [E][N][Kd/16] (NVFP4) or bf16 [E][N][Kd/64] (int4)
    const float* wg;           // NVFP4 per-expert fp32 scale [E]
    float gs;                  // FP8: the weight scale times the input scale
    const _Float16* a16;       // A rows: x [T][Kd] (up) or h [T K][Kd] (down; hi/lo [2 T K][Kd] but FP8)
    const int32_t* aexp;       // power of two of each staged row: [T] (up) or [T K] (down)
    const int4* act;           // experts with rows: (e, first dispatch row, rows, 0)
    const int32_t* n_act;      // their number
    const int32_t* perm;       // dispatch row -> pair t K + slot
    const float* gate;         // [T K] gate weight of each pair (down)
    float* out;                // [T K][N] fp32, by pair
};

struct A16Ctx {
    int row0, n_e, hk, nch, n, ap, ar, sigma;
    uint32_t wc_off, sc_row;
    float g;
};

// Eight int4 codes (one dword, two's complement nibbles) times the fp16
// scale s, in the pair order (e0,e4), (e1,e5), (e2,e6), (e3,e7): a nibble
// with its sign bit flipped, placed under the fp16 exponent of 1024, is
// 1032 + code exactly.
__device__ __forceinline__ f16x8 int4x8_f16(uint32_t w, f16x2 s) {
    const f16x2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
    f16x2 p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = (__builtin_bit_cast(f16x2, ((w >> (4 * i)) & 0x000F000Fu) ^ 0x64086408u) - off) * s;
    return f16x8{p[0].x, p[0].y, p[1].x, p[1].y, p[2].x, p[2].y, p[3].x, p[3].y};
}

// Eight E4M3FN bytes (two dwords, natural order) as fp16, exact.
__device__ __forceinline__ f16x8 fp8x8_f16(uint32_t w0, uint32_t w1) {
    const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
    const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
    const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
    const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
    return f16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

template <int NP>
struct BChunkN {
    uint4 q[NP];
};

template <int EPI, int WF, typename F>
__device__ __forceinline__ void a16_tile(const GemmA16Args& a, A16Ctx& x, int m0, int mv,
                                         _Float16 (*As)[kApitch], F&& after_first_issue) {
    // HILO: the A rows come in hi/lo pairs (the 16-bit path's h); FP8
    // weights: 16-byte pieces of 16 values, 8 per lane and chunk
    constexpr bool HILO = EPI == EPI_DOWN && WF != FMT_FP8;
    constexpr bool F8 = WF == FMT_FP8;
    constexpr int NP = F8 ? 8 : 4, KPP = F8 ? 16 : 32;
    const int lane = threadIdx.x & 63;
    const uint32_t row_bytes = F8 ? (uint32_t)a.Kd : (uint32_t)(a.Kd / 2);
    // the A row this thread stages (rows past the tile's last repeat it)
    const int dr = x.row0 + m0 + min(HILO ? (x.ar >> 1) : x.ar, mv - 1);
    const int pr = a.perm[dr];
    // weight pieces of chunk c (this lane's half), in the B ring
    auto valid_pieces = [&](int c) { return min(NP, max(0, (a.Kd - c * kGemmBK - 128 * x.hk) / KPP)); };
    auto load_b = [&](int c, BChunkN<NP>& b) {
        const int v = valid_pieces(c);
        const uint32_t c_last = x.wc_off + row_bytes - 16;
        const uint32_t base = x.wc_off + (uint32_t)c * (F8 ? kGemmBK : kGemmBK / 2) + (F8 ? 128 : 64) * x.hk;
#pragma unroll
        for (int i = 0; i < NP; ++i) b.q[i] = ldg16(a.wc + (i < v ? base + 16 * i : c_last));
    };
    BChunkN<NP> bb[3];
    load_b(0, bb[0]);
    __builtin_amdgcn_sched_barrier(0);
    load_b(1, bb[1]);
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t arow = EPI == EPI_UP ? (uint32_t)(pr / a.K) : HILO ? (uint32_t)(2 * pr + (x.ar & 1)) : (uint32_t)pr;
    const _Float16* asrc = a.a16 + (size_t)arow * a.Kd;
    uint4 qa[3][4];
    auto load_a = [&](int c, uint4 (&q)[4]) {
        const int k0 = c * kGemmBK + 32 * x.ap;
        const _Float16* p = asrc + (k0 < a.Kd ? k0 : a.Kd - 32);
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = *reinterpret_cast<const uint4*>(p + 8 * i);
    };
    load_a(0, qa[0]);
    __builtin_amdgcn_sched_barrier(0);
    load_a(1, qa[1]);
    __builtin_amdgcn_sched_barrier(0);
    after_first_issue();

    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;

    auto step = [&](const int c, const BChunkN<NP>& bc, BChunkN<NP>& bn, const uint4 (&qc)[4], uint4 (&qn)[4]) {
        __syncthreads();  // every wave is done with the last chunk's A
        const bool a_ok = c * kGemmBK + 32 * x.ap < a.Kd;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint4 v = a_ok ? qc[i] : make_uint4(0u, 0u, 0u, 0u);
            if constexpr (WF == FMT_INT4) {
                const uint32_t p[4] = {v.x, v.y, v.z, v.w};
                uint32_t q[4];
                int4_pair_order(p, q);
                v = make_uint4(q[0], q[1], q[2], q[3]);
            }
            *reinterpret_cast<uint4*>(&As[x.ar][a_col(4 * x.ap + i)]) = v;
        }
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        load_b(c + 2, bn);
        __builtin_amdgcn_sched_barrier(0);
        load_a(c + 2, qn);
        __builtin_amdgcn_sched_barrier(0);
        const int valid = valid_pieces(c);
        f16x2 sc[4];
        if constexpr (WF == FMT_NVFP4) {
            const int so = c * 16 + 8 * x.hk;
            const uint32_t s0 = *reinterpret_cast<const uint32_t*>(g_gemm_sct + x.sc_row + (valid > 0 ? so : 0));
            const uint32_t s1 = *reinterpret_cast<const uint32_t*>(g_gemm_sct + x.sc_row + (valid > 2 ? so + 4 : 0));
            sc[0] = e4m3x2_f16<false>(s0);
            sc[1] = e4m3x2_f16<true>(s0);
            sc[2] = e4m3x2_f16<false>(s1);
            sc[3] = e4m3x2_f16<true>(s1);
        } else if constexpr (WF == FMT_INT4) {
            // groups 4c + 2hk and 4c + 2hk + 1 (pieces 0-1 and 2-3)
            const int grp = 4 * c + 2 * x.hk;
            const uint16_t* srow = reinterpret_cast<const uint16_t*>(g_gemm_sct + x.sc_row);
            const _Float16 g0 = (_Float16)ldexpf(bf16_bits_to_f32(srow[valid > 0 ? grp : 0]), x.sigma);
            const _Float16 g1 = (_Float16)ldexpf(bf16_bits_to_f32(srow[valid > 2 ? grp + 1 : 0]), x.sigma);
            sc[0] = sc[1] = f16x2{g0, g0};
            sc[2] = sc[3] = f16x2{g1, g1};
        }
        if constexpr (!F8) {
#pragma unroll
            for (int pc = 0; pc < 4; ++pc)
                if (pc >= valid) sc[pc] = f16x2{0, 0};
        }
        uint32_t w[4 * NP];
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            w[4 * i] = bc.q[i].x;
            w[4 * i + 1] = bc.q[i].y;
            w[4 * i + 2] = bc.q[i].z;
            w[4 * i + 3] = bc.q[i].w;
        }
        const _Float16* arow_l = &As[lane & 31][0];
        f16x8 af[2];
        af[0] = *reinterpret_cast<const f16x8*>(arow_l + a_col(16 * x.hk));
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if (j + 1 < 16) af[(j + 1) & 1] = *reinterpret_cast<const f16x8*>(arow_l + a_col(16 * x.hk + j + 1));
            f16x8 bfrag;
            if constexpr (WF == FMT_NVFP4) {
                // dword j: k 8j..8j+7 of the lane's half, block j / 2, piece j / 4
                const f16x2 sp = sc[j / 4];
                bfrag = fp4x8_f16(w[j], (j & 2) ? f16x2{sp.y, sp.y} : f16x2{sp.x, sp.x});
            } else if constexpr (WF == FMT_INT4) {
                bfrag = int4x8_f16(w[j], sc[j / 4]);
            } else {
                // dwords 2j, 2j + 1: k 8j..8j+7 of the lane's half, piece j / 2
                bfrag = fp8x8_f16(w[2 * j], w[2 * j + 1]);
                if (j / 2 >= valid) bfrag = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
            }
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[j & 1], bfrag, acc, 0, 0, 0);
        }
    };
    int c = 0;
    for (; c + 3 <= x.nch; c += 3) {
        step(c, bb[0], bb[2], qa[0], qa[2]);
        step(c + 1, bb[1], bb[0], qa[1], qa[0]);
        step(c + 2, bb[2], bb[1], qa[2], qa[1]);
    }
    if (c < x.nch) step(c, bb[0], bb[2], qa[0], qa[2]);
    if (c + 1 < x.nch) step(c + 1, bb[1], bb[0], qa[1], qa[0]);

    // epilogue: lane holds column n and rows 8 (r / 4) + 4 (lane / 32) + r % 4
    if (x.n >= a.N) return;
    if constexpr (EPI == EPI_UP) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
            if (m < mv) {
                const int p = a.perm[x.row0 + m0 + m];
                const float u = fmaxf(ldexpf(acc[r], -(x.sigma + a.aexp[p / a.K])) * x.g, 0.f);
                a.out[(size_t)p * a.N + x.n] = u * u;
            }
        }
    } else if constexpr (HILO) {
        // rows 2j (hi) and 2j + 1 (lo) of pair j sit in registers r and r + 1
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const int j = (8 * (r / 4) + 4 * (lane >> 5) + (r % 4)) >> 1;
            if (j < mv) {
                const int p = a.perm[x.row0 + m0 + j];
                const float z = acc[r] + acc[r + 1];
                a.out[(size_t)p * a.N + x.n] = ldexpf(z, -(x.sigma + a.aexp[p])) * (a.gate[p] * x.g);
            }
        }
    } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
            if (m < mv) {
                const int p = a.perm[x.row0 + m0 + m];
                a.out[(size_t)p * a.N + x.n] = ldexpf(acc[r], -(x.sigma + a.aexp[p])) * (a.gate[p] * x.g);
            }
        }
    }
}

template <int EPI, int WF>
__global__ __launch_bounds__(256, 2) void k_grouped_a16(GemmA16Args a) {
    __shared__ __attribute__((aligned(16))) _Float16 As[32][kApitch];
    // (active expert j, column tile): expert-major on the XCDs as in
    // k_grouped_gemm (workgroup b runs on XCD b % 8)
    const int ntiles = gridDim.x;
    int tile = blockIdx.x, j = blockIdx.y;
    if (gridDim.y % 8 == 0) {
        const int b = blockIdx.y * ntiles + blockIdx.x;
        const int q = b / 8;
        j = b % 8 + 8 * (q / ntiles);
        tile = q % ntiles;
    }
    if (j >= a.n_act[0]) return;  // uniform
    const int4 ae = a.act[j];
    const int e = ae.x;
    A16Ctx x;
    x.row0 = ae.y;
    x.n_e = ae.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // this tile's block scales (contiguous rows), one dword per thread and pass
    const int rb = WF == FMT_NVFP4 ? a.Kd / 16 : WF == FMT_INT4 ? a.Kd / 32 : 0;  // scale bytes per weight row
    const int sc_ndw = min(kGemmBN, a.N - tile * kGemmBN) * rb / 4;
    uint32_t scv[32];
    if constexpr (WF != FMT_FP8) {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(a.wsc + ((uint32_t)e * a.N + tile * kGemmBN) * (uint32_t)rb);
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const int d = (int)threadIdx.x + 256 * i;
            scv[i] = d < sc_ndw ? src[d] : 0u;
        }
    }
    x.hk = lane >> 5;
    x.nch = (a.Kd + kGemmBK - 1) / kGemmBK;
    x.n = tile * kGemmBN + 32 * wave + (lane & 31);
    x.wc_off = ((uint32_t)e * a.N + min(x.n, a.N - 1)) * (uint32_t)(WF == FMT_FP8 ? a.Kd : a.Kd / 2);
    x.sc_row = (uint32_t)((32 * wave + (lane & 31)) * rb);
    x.g = WF == FMT_NVFP4 ? a.wg[e] : WF == FMT_INT4 ? 1.0f : a.gs;
    x.sigma = 0;
    x.ap = threadIdx.x & 7;
    x.ar = threadIdx.x >> 3;
    const int step = (EPI == EPI_DOWN && WF != FMT_FP8) ? 16 : 32;
    // the first M-tile's first loads leave before the scales are stored
    auto scales_in = [&] {
        if constexpr (WF != FMT_FP8) {
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                const int d = (int)threadIdx.x + 256 * i;
                if (d < sc_ndw) reinterpret_cast<uint32_t*>(g_gemm_sct)[d] = scv[i];
            }
        }
        if constexpr (WF == FMT_INT4) {
            __syncthreads();
            const uint16_t* srow = reinterpret_cast<const uint16_t*>(g_gemm_sct + x.sc_row);
            float mx = 0.f;
            for (int q = 0; q < a.Kd / 64; ++q) mx = fmaxf(mx, fabsf(bf16_bits_to_f32(srow[q])));
            x.sigma = (mx > 0.f && mx < __builtin_inff()) ? 11 - ilogbf(mx) : 0;
        }
    };
    a16_tile<EPI, WF>(a, x, 0, min(step, x.n_e), As, scales_in);
    for (int m0 = step; m0 < x.n_e; m0 += step) a16_tile<EPI, WF>(a, x, m0, min(step, x.n_e - m0), As, [] {});
}

}  // namespace q4moe
