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
// fp16 (the activations while they are staged in LDS, the weights in
// registers): e2m1 * e4m3 has at most six significant bits and lies in
// [2^-10, 2688], so every decoded operand is exact in fp16 and every MFMA
// product is exact in fp32; only the fp32 accumulation rounds.
#pragma once

#include "q4moe_kernels.hpp"

namespace q4moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// Router logits for many tokens on fp32 MFMA (v_mfma_f32_16x16x4_f32): a
// workgroup computes a (16 TB)-token x 16-expert tile; its 8 waves split the
// hidden dimension, and their partial tiles are summed in LDS in wave order.
// Each wave runs the TB token blocks of its part of the hidden dimension
// side by side: one router-weight fragment feeds TB MFMAs.  A wider token
// tile cuts the re-reads of the fp32 router matrix, which dominate the
// kernel's L2 traffic (every token tile reads all of it).  Each (token
// block, expert block, wave) runs the same MFMA sequence at any TB, so the
// logits do not depend on TB.  Lane l feeds token/expert row l % 16 and,
// for each block of 16 k-values, k-values 4 (l / 16) .. +3 (one per MFMA; A
// and B use the same k order).  The grid is (token tiles, expert tiles):
// workgroup b runs on XCD b % 8, so all expert tiles of a token tile share
// one XCD and read its x rows from HBM once.
// ---------------------------------------------------------------------------
constexpr int kRouterTile = 16;

template <int TB>
__global__ __launch_bounds__(512) void k_router_gemm(RouterArgs a) {
    __shared__ float part[8][16 * TB][17];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * kRouterTile * TB, e0 = blockIdx.y * kRouterTile;
    const int row = lane & 15, kq = lane >> 4;
    const int e = min(e0 + row, a.E - 1);
    const uint16_t* xr[TB];
#pragma unroll
    for (int j = 0; j < TB; ++j) xr[j] = a.x + (size_t)min(t0 + 16 * j + row, a.T - 1) * a.H + 4 * kq;
    const float* wr = a.wg + (size_t)e * a.H + 4 * kq;
    const int nblk = a.H / 16;
    const int b0 = wave * nblk / 8, b1 = (wave + 1) * nblk / 8;
    f32x4g acc[TB];
#pragma unroll
    for (int j = 0; j < TB; ++j) acc[j] = f32x4g{0.f, 0.f, 0.f, 0.f};
    // kRouterBatch blocks' loads leave before their MFMAs (blocks past b1 are
    // clamped to b1 - 1 and skipped)
    constexpr int kRouterBatch = 7;
    for (int bb = b0; bb < b1; bb += kRouterBatch) {
        uint2 xv[kRouterBatch][TB];
        float4 wv[kRouterBatch];
#pragma unroll
        for (int i = 0; i < kRouterBatch; ++i) {
            const int b = min(bb + i, b1 - 1);
            wv[i] = *reinterpret_cast<const float4*>(wr + 16 * b);
#pragma unroll
            for (int j = 0; j < TB; ++j) xv[i][j] = *reinterpret_cast<const uint2*>(xr[j] + 16 * b);
        }
#pragma unroll
        for (int i = 0; i < kRouterBatch; ++i) {
            if (bb + i < b1) {
#pragma unroll
                for (int j = 0; j < TB; ++j) {
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(bf16_bits_to_f32(xv[i][j].x & 0xffffu), wv[i].x, acc[j], 0, 0, 0);
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(bf16_bits_to_f32(xv[i][j].x >> 16), wv[i].y, acc[j], 0, 0, 0);
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(bf16_bits_to_f32(xv[i][j].y & 0xffffu), wv[i].z, acc[j], 0, 0, 0);
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(bf16_bits_to_f32(xv[i][j].y >> 16), wv[i].w, acc[j], 0, 0, 0);
                }
            }
        }
    }
    // lane holds column lane % 16 (expert) and rows 4 (lane / 16) + i (tokens)
#pragma unroll
    for (int j = 0; j < TB; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) part[wave][16 * j + 4 * kq + i][row] = acc[j][i];
    __syncthreads();
    for (int u = threadIdx.x; u < 16 * TB * kRouterTile; u += 512) {
        const int i = u >> 4, j = u & 15;
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
    // (nullable) the experts with at least one row, in expert order:
    // act[j] = (expert, first dispatch row, rows, 0) for j < n_act[0]
    int4* act;
    int32_t* n_act;
};

__global__ __launch_bounds__(64) void k_dispatch(DispatchArgs a) {
    const int e = blockIdx.x, lane = threadIdx.x;
    int base = 0;
    // four chunks of 64 tokens per round: all their id loads leave before
    // any is compared.  Token and slot indices are clamped (K <= 8), so the
    // loads need no branch; slots past K are masked afterwards.  (A branch
    // around each load made every load wait for the one before it.)
    for (int t0 = 0; t0 < a.T; t0 += 256) {
        int idv[4][8];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int tc = min(t0 + 64 * c + lane, a.T - 1);
#pragma unroll
            for (int s = 0; s < 8; ++s) idv[c][s] = a.ids[(size_t)tc * a.K + min(s, a.K - 1)];
        }
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int s = 0; s < 8; ++s)
                if (s >= a.K) idv[c][s] = -1;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int t = t0 + 64 * c + lane;
            int pair = -1;
#pragma unroll
            for (int s = 0; s < 8; ++s)
                if (s < a.K && idv[c][s] == e && t < a.T) pair = t * a.K + s;
            const unsigned long long m = __ballot(pair >= 0);
            if (pair >= 0) {
                const int before = __popcll(m & ((1ull << lane) - 1ull));
                a.lists[(size_t)e * a.T + base + before] = pair;
            }
            base += __popcll(m);
        }
    }
    if (lane == 0) a.counts[e] = base;
}

// Offsets (exclusive scan of the counts), the dispatch permutation and its
// inverse, and (when asked) the list of experts that have rows.  Workgroup e
// (grid E <= 256) loads all counts, one per lane, scans them (and the
// has-rows flags) across its 256 lanes and writes expert e's part of the
// permutation and its entry of the list.
__global__ __launch_bounds__(256) void k_dispatch_scan(DispatchArgs a) {
    __shared__ int s_cnt[256], s_off[257], s_rank, s_nact, s_wc[4], s_wf[4];
    const int e = blockIdx.x;
    const int i = threadIdx.x, lane = i & 63, wave = i >> 6;
    const int c = i < a.E ? a.counts[i] : 0;
    const int f = c > 0 ? 1 : 0;
    s_cnt[i] = c;
    // inclusive scans of c and f: within the wave, then over the waves
    int sc = c, sf = f;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int tc = __shfl_up(sc, d, 64), tf = __shfl_up(sf, d, 64);
        if (lane >= d) {
            sc += tc;
            sf += tf;
        }
    }
    if (lane == 63) {
        s_wc[wave] = sc;
        s_wf[wave] = sf;
    }
    __syncthreads();
    for (int w = 0; w < wave; ++w) {
        sc += s_wc[w];
        sf += s_wf[w];
    }
    if (i < a.E) s_off[i] = sc - c;
    if (i == a.E - 1) {
        s_off[a.E] = sc;
        s_nact = sf;
    }
    if (i == e) s_rank = sf - f;
    __syncthreads();
    if (threadIdx.x == 0 && a.act) {
        if (s_cnt[e] > 0) a.act[s_rank] = make_int4(e, s_off[e], s_cnt[e], 0);
        if (e == 0) a.n_act[0] = s_nact;
    }
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

struct QuantArgs {
    int rows, cols;
    const void* v;      // bf16 bits (BF16_IN) or fp32
    uint8_t* codes;     // [rows][cols/2]
    uint8_t* scales;    // [rows][cols/16]
};

// One lane per 16-value block: it loads the block's 32 (bf16) or 64 (fp32)
// bytes as 16-byte pieces (all in flight at once), takes the block maximum
// in registers, and stores the block's 8 code bytes in one store and its
// scale byte.  Lanes past the end work on the last block and store nothing.
template <bool BF16_IN>
__global__ __launch_bounds__(256) void k_quant_nvfp4(QuantArgs a) {
    const size_t n_blocks = (size_t)a.rows * (size_t)a.cols / 16;
    const size_t gb = (size_t)blockIdx.x * 256 + threadIdx.x;
    const bool live = gb < n_blocks;
    const size_t bk = live ? gb : n_blocks - 1;
    float v[16];
    if constexpr (BF16_IN) {
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.v) + bk * 16);
        const uint4 q0 = src[0], q1 = src[1];
        const uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            v[2 * k] = bf16_bits_to_f32(w[k] & 0xffffu);
            v[2 * k + 1] = bf16_bits_to_f32(w[k] >> 16);
        }
    } else {
        const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(a.v) + bk * 16);
        float4 q[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) q[k] = src[k];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[4 * k + 0] = q[k].x;
            v[4 * k + 1] = q[k].y;
            v[4 * k + 2] = q[k].z;
            v[4 * k + 3] = q[k].w;
        }
    }
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) amax = fmaxf(amax, fabsf(v[k]));
    const uint32_t sb = e4m3fn_rne_sat(__fdiv_rn(amax, 6.0f));
    const E2m1Thresholds th = e2m1_thresholds(e4m3fn_to_f32(sb));
    uint32_t word[2] = {0u, 0u};
#pragma unroll
    for (int k = 0; k < 16; ++k)
        word[k >> 3] |= (e2m1_code(fabsf(v[k]), th) | ((__float_as_uint(v[k]) >> 31) << 3)) << (4 * (k & 7));
    if (live) {
        *reinterpret_cast<uint2*>(a.codes + bk * 8) = make_uint2(word[0], word[1]);
        a.scales[bk] = (uint8_t)sb;
    }
}

// ---------------------------------------------------------------------------
// Grouped GEMM on MFMA: for expert e and a 128-column output tile,
// out[m][n] = sum_k A[m][k] * W_e[n][k] over the expert's rows m, with both
// operands NVFP4 (codes + E4M3 scale per 16 along k), decoded exactly to
// fp16: A into LDS, W in registers.  Workgroup: 4 waves; wave w owns output
// columns 32w..32w+31 (two 16-column blocks) and up to four 16-row subtiles
// (64 rows) of M, one v_mfma_f32_16x16x32_f16 accumulator per (subtile,
// block).  K advances 256 per chunk (128 bytes of every weight row); a
// 3-slot register ring keeps two chunks of weight loads in flight while the
// current one computes.
// ---------------------------------------------------------------------------
enum : int { EPI_UP = 0, EPI_DOWN = 1 };
// Output columns (rows of W_e) per workgroup (4 waves x 32), A rows per
// M-tile (an expert's rows beyond it take further M-tiles), k per chunk (128
// bytes of every weight row), LDS pitch of A (fp16).  BM = 64 (four
// subtiles) keeps the kernel within the 256 registers of two workgroups per
// CU.  At 96 rows the six-subtile path pushed it over that limit: values
// spilled and reloaded ahead of each ring loop, and the first use of such
// a reload waits for every load issued before it.  That emptied the ring
// once per turn.
constexpr int kGemmBN = 128, kGemmBM = 64, kGemmBK = 256, kApitch = kGemmBK + 8;

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
    float* out;                // [rows][N] fp32, dispatch order
};

// Pieces of the grouped GEMM below (k_grouped_gemm describes the whole).
// A chunk's weights of one lane: q[2 nb + h] = bytes 64 h + 16 kq .. +15 of
// the chunk in the lane's row of block nb.
struct BChunk {
    uint4 q[4];
};

// Block scales of the workgroup's 128 weight rows (row-major, Kd / 16 bytes a
// row), staged once per workgroup: per chunk a lane then reads its bytes
// from LDS instead of scattered loads from its rows.
extern __shared__ __attribute__((aligned(16))) uint8_t g_gemm_sct[];

// Per-workgroup constants of the grouped GEMM.  Lane (n16 = lane % 16, kq =
// lane / 16): n = column of its block-0 row (block 1: n + 16); wc_off[nb] /
// sc_row[nb] = byte offsets of its rows' codes / staged scales.
struct GemmCtx {
    int e, row0, n, kq, nch, ap, ar, rb;
    uint32_t wc_off[2], sc_row[2];
    float g;
};

// Piece (h, kq) of chunk c (k 256 c + 128 h + 32 kq .. +31) lies inside K.
__device__ __forceinline__ bool gemm_piece_ok(const GemmArgs& a, int c, int h, int kq) {
    return c * kGemmBK + 128 * h + 32 * kq < a.Kd;
}

// Pieces past the end of the row read the row's last 16 code bytes instead
// (their scales are zeroed where they are used).  Each load instruction of a
// wave reads 64 contiguous bytes of 16 rows: a wave load spread over 32 rows
// streams about a third slower.
__device__ __forceinline__ void gemm_load_b(const GemmArgs& a, const GemmCtx& x, int c, BChunk& b) {
    const uint32_t kb = (uint32_t)c * kGemmBK / 2;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const uint32_t c_last = x.wc_off[nb] + a.Kd / 2 - 16;
#pragma unroll
        for (int h = 0; h < 2; ++h)
            b.q[2 * nb + h] = ldg16(a.wc + (gemm_piece_ok(a, c, h, x.kq) ? x.wc_off[nb] + kb + 64 * h + 16 * x.kq
                                                                           : c_last));
    }
}

// A tile LDS column (fp16 elements) of 16-byte group g of a row: groups are
// XOR-swizzled so that the 8 threads staging one row (group 4 ap + i for
// piece ap, store i) write 8 different bank groups; the MFMA fragment reads
// (16 rows at one group, rows 528 bytes apart) stay conflict-free.
__device__ __forceinline__ int a_col(int g) { return 8 * (g ^ ((g >> 3) & 3)); }

// A compile-time switch for the chunk step: whether it loads chunk c + 2.
template <bool B> struct ChunkPrefetch {
    static constexpr bool value = B;
};

// One M-tile (rows m0 .. m0 + mv - 1 of expert e, MS = ceil(mv / 16)
// subtiles, staged in ceil(mv / 32) groups of 32 rows) against the
// workgroup's 128 columns.  FIRST: the workgroup's first M-tile, whose
// weight chunks 0 and 1 (bb[0], bb[1]) and A rows (arow) the kernel's
// prologue has already loaded; later M-tiles load their own.
template <int EPI, int MS, bool FIRST>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, const GemmCtx& x, int m0, int mv,
                                          _Float16 (*As)[kApitch], BChunk (&bb)[3],
                                          const uint32_t (&arow_first)[2]) {
    constexpr int MA = (MS + 1) / 2;  // staging groups of 32 rows
    static_assert(MA <= 2, "arow_first holds two staging groups");
    const int lane = threadIdx.x & 63, n16 = lane & 15;
    uint32_t ac_off[MA], as_off[MA];
#pragma unroll
    for (int q = 0; q < MA; ++q) {
        uint32_t arow;
        if constexpr (FIRST) {
            arow = arow_first[q];
        } else {
            const int drow = x.row0 + m0 + min(x.ar + 32 * q, mv - 1);
            arow = a.a_by_token ? (uint32_t)(a.perm[drow] / a.K) : (uint32_t)drow;
        }
        ac_off[q] = arow * (uint32_t)(a.Kd / 2);
        as_off[q] = arow * (uint32_t)(a.Kd / 16);
    }
    // A pieces in a three-slot register ring alongside B's: chunk c's A is
    // loaded two chunks ahead, into the slot chunk c - 1 staged from
    uint4 qa3[3][MA];
    uint32_t sa3[3][MA];
    auto load_a = [&](int c, uint4 (&qa)[MA], uint32_t (&sa)[MA]) {
        const int kb = c * kGemmBK;
        const bool ok = 32 * x.ap < a.Kd - kb;
#pragma unroll
        for (int q = 0; q < MA; ++q) {
            // past the end: the row's last piece (just read), with scale 0
            qa[q] = ldg16(a.ac + (ok ? ac_off[q] + kb / 2 + 16 * x.ap : ac_off[q] + a.Kd / 2 - 16));
            // (the scale of a piece past the end is zeroed where it is used:
            // touching a loaded value here would wait for every load before it)
            sa[q] = *reinterpret_cast<const uint16_t*>(
                a.asc + (ok ? as_off[q] + kb / 16 + 2 * x.ap : as_off[q] + a.Kd / 16 - 2));
        }
    };

    f32x4g acc[MS][2];
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[i][nb] = f32x4g{0.f, 0.f, 0.f, 0.f};

    // issue order = wait order (the scheduler may not mix the groups):
    // FIRST: (B0, B1 from the prologue) A0, A1; otherwise B0, A0, B1, A1
    if constexpr (!FIRST) gemm_load_b(a, x, 0, bb[0]);
    __builtin_amdgcn_sched_barrier(0);
    load_a(0, qa3[0], sa3[0]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!FIRST) gemm_load_b(a, x, 1, bb[1]);
    __builtin_amdgcn_sched_barrier(0);
    load_a(1, qa3[1], sa3[1]);
    __builtin_amdgcn_sched_barrier(0);
    // chunk c stages its A from (qa, sa), computes on bc, and (PF) loads
    // chunk c + 2 into (qn, sn) and bn, the slots chunk c - 1 used
    auto step = [&](auto pf, const int c, const BChunk& bc, BChunk& bn, const uint4 (&qa)[MA],
                    const uint32_t (&sa)[MA], uint4 (&qn)[MA], uint32_t (&sn)[MA]) {
            // this chunk's A into LDS (after every wave is done with the last one)
            __syncthreads();
            const bool a_ok = 32 * x.ap < a.Kd - c * kGemmBK;
#pragma unroll
            for (int q = 0; q < MA; ++q) {
                const f16x2 sp = e4m3x2_f16<false>(a_ok ? sa[q] : 0u);
                const f16x2 s_lo = {sp.x, sp.x}, s_hi = {sp.y, sp.y};
                _Float16* dst = &As[x.ar + 32 * q][0];
                *reinterpret_cast<f16x8*>(dst + a_col(4 * x.ap + 0)) = fp4x8_f16(qa[q].x, s_lo);
                *reinterpret_cast<f16x8*>(dst + a_col(4 * x.ap + 1)) = fp4x8_f16(qa[q].y, s_lo);
                *reinterpret_cast<f16x8*>(dst + a_col(4 * x.ap + 2)) = fp4x8_f16(qa[q].z, s_hi);
                *reinterpret_cast<f16x8*>(dst + a_col(4 * x.ap + 3)) = fp4x8_f16(qa[q].w, s_hi);
            }
            __syncthreads();
            // next loads: A and B of chunk c+2 into the free slots
            if constexpr (decltype(pf)::value) {
                __builtin_amdgcn_sched_barrier(0);
                load_a(c + 2, qn, sn);
                __builtin_amdgcn_sched_barrier(0);
                gemm_load_b(a, x, c + 2, bn);
                __builtin_amdgcn_sched_barrier(0);
            }
            // 8 MFMA steps (h, d) on chunk c: lane (n16, kq) takes dword d of
            // its piece h (k 128 h + 32 kq + 8 d .. +7 of the chunk) with
            // block scale 8 h + 2 kq + d / 2; pieces past the end get scale 0
            f16x2 sc[2][2];
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t sv = *reinterpret_cast<const uint16_t*>(g_gemm_sct + x.sc_row[nb] + c * 16 +
                                                                           8 * h + 2 * x.kq);
                    sc[nb][h] = e4m3x2_f16<false>(gemm_piece_ok(a, c, h, x.kq) ? sv : 0u);  // byte 0 is +0
                }
            // the A fragment of step (h, d): group 16 h + 4 kq + d of unit row 16 i + n16
            const _Float16* arow = &As[n16][0];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    f16x8 af[MS];
#pragma unroll
                    for (int i = 0; i < MS; ++i)
                        af[i] = *reinterpret_cast<const f16x8*>(arow + 16 * i * kApitch +
                                                                a_col(16 * h + 4 * x.kq + d));
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb) {
                        const uint4 pc = bc.q[2 * nb + h];
                        const uint32_t wd = d == 0 ? pc.x : d == 1 ? pc.y : d == 2 ? pc.z : pc.w;
                        const f16x2 sp = sc[nb][h];
                        const f16x8 bfrag = fp4x8_f16(wd, d < 2 ? f16x2{sp.x, sp.x} : f16x2{sp.y, sp.y});
#pragma unroll
                        for (int i = 0; i < MS; ++i)
                            acc[i][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bfrag, acc[i][nb], 0, 0, 0);
                    }
                }
            }
    };
    // Whole turns of the ring, then the one or two chunks left, which load
    // nothing (no exit from inside a turn).  A turn's loads past the end of
    // K read the rows' last bytes.  They come only when nch % 3 != 2, and
    // then they stay in flight into the epilogue, whose registers wait for
    // them.  Hidden 2688 and inter 1856 (11 and 8 chunks) have none.
    constexpr ChunkPrefetch<true> PF{};
    constexpr ChunkPrefetch<false> NP{};
    int c = 0;
    for (; c + 3 <= x.nch; c += 3) {
        step(PF, c, bb[0], bb[2], qa3[0], sa3[0], qa3[2], sa3[2]);
        step(PF, c + 1, bb[1], bb[0], qa3[1], sa3[1], qa3[0], sa3[0]);
        step(PF, c + 2, bb[2], bb[1], qa3[2], sa3[2], qa3[1], sa3[1]);
    }
    if (c < x.nch) step(NP, c, bb[0], bb[2], qa3[0], sa3[0], qa3[2], sa3[2]);
    if (c + 1 < x.nch) step(NP, c + 1, bb[1], bb[0], qa3[1], sa3[1], qa3[0], sa3[0]);
    // epilogue: lane (n16, kq) holds column n + 16 nb and rows 16 i + 4 kq + r
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int n = x.n + 16 * nb;
#pragma unroll
        for (int i = 0; i < MS; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 16 * i + 4 * x.kq + r;
                if (m < mv && n < a.N) {
                    const int p = x.row0 + m0 + m;
                    float v = acc[i][nb][r] * x.g;
                    if constexpr (EPI == EPI_UP) {
                        v = fmaxf(v, 0.f);
                        v = v * v;
                    }
                    a.out[(size_t)p * a.N + n] = v;
                }
            }
        }
    }
}

// Grouped GEMM over the experts' dispatch rows: out[row][n] = epi(sum_k
// A[row][k] W_e[n][k]) on fp16 MFMA (v_mfma_f32_16x16x32_f16) with both
// operands decoded exactly from NVFP4.  A workgroup takes 128 columns of one
// expert and all its rows in M-tiles of 64; wave w owns columns 32w..32w+31.
//
// The reduction runs in chunks of 256: every weight row contributes one whole
// 128-byte line per chunk, loaded straight into registers two chunks ahead in
// a three-slot ring (lane (n16, kq) of block nb: row 32 w + 16 nb + n16,
// bytes 64 h + 16 kq .. +15 for halves h = 0, 1: each load instruction
// covers 64 bytes of 16 rows); the A pieces of the chunk, loaded two chunks
// ahead in a ring of their own, are decoded into LDS once per workgroup.
// MFMA step (h, d) of a chunk sums k 128 h + 32 kq + 8 d .. +7 on lanes
// kq = 0..3: the same k order on both operands.  The block scales of the
// workgroup's 128 weight rows are copied into LDS once.  The prologue
// issues every load that does not wait on another before its first wait:
// weight chunks 0 and 1, the scale rows and the first M-tile's dispatch
// entries (the A rows of the up GEMM), so that the workgroup's start costs
// one memory round trip, then one more for the A pieces of chunks 0 and 1.
// The chunk loads are unconditional: pieces past the end of a row (in the
// last chunk, and a turn's loads of chunks past K) read the row's last
// bytes and get scale 0, so that every wait covers exactly the loads it
// needs.
// Offsets are 32-bit from the uniform bases: the argument limits (E <= 256,
// rows and columns <= 4096, T * K <= 2^19) keep every matrix under 2^31
// bytes.
template <int EPI>
__global__ __launch_bounds__(256, 2) void k_grouped_gemm(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) _Float16 As[kGemmBM][kApitch];
    GemmCtx x;
    // Expert-major placement on the XCDs: workgroup b runs on XCD b % 8, and
    // when E % 8 == 0 all column tiles of expert e go to XCD e % 8, so that
    // each XCD's L2 fetches an expert's A rows once.  With gridDim = (tiles,
    // E) the flat id b covers every (tile, expert) pair exactly once.
    const int ntiles = gridDim.x;
    int tile = blockIdx.x;
    x.e = blockIdx.y;
    if (gridDim.y % 8 == 0) {
        const int b = blockIdx.y * ntiles + blockIdx.x;
        const int j = b / 8;
        x.e = b % 8 + 8 * (j / ntiles);
        tile = j % ntiles;
    }
    x.row0 = a.offsets[x.e];
    const int n_e = a.offsets[x.e + 1] - x.row0;
    if (n_e == 0) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    x.kq = lane >> 4;
    x.nch = (a.Kd + kGemmBK - 1) / kGemmBK;
    x.n = tile * kGemmBN + 32 * wave + (lane & 15);
    const int sc_rb = a.Kd / 16;
    x.rb = sc_rb;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const uint32_t wrow = (uint32_t)x.e * a.N + min(x.n + 16 * nb, a.N - 1);
        x.wc_off[nb] = wrow * (uint32_t)(a.Kd / 2);
        x.sc_row[nb] = (uint32_t)((32 * wave + 16 * nb + (lane & 15)) * x.rb);
    }
    // A staging role: piece ap (k 32ap..32ap+31 of the chunk) of rows ar + 32q
    x.ap = threadIdx.x & 7;
    x.ar = threadIdx.x >> 3;
    // The prologue's loads, in wait order: weight chunks 0 and 1, the scale
    // rows of this tile (contiguous: rows e N + 128 tile .., one dword per
    // thread and pass), the dispatch entries of the first M-tile's rows.
    BChunk bb[3];
    gemm_load_b(a, x, 0, bb[0]);
    gemm_load_b(a, x, 1, bb[1]);
    const int sc_ndw = min(kGemmBN, a.N - tile * kGemmBN) * sc_rb / 4;
    uint32_t scv[32];
    {
        const uint32_t* src =
            reinterpret_cast<const uint32_t*>(a.wsc + ((uint32_t)x.e * a.N + tile * kGemmBN) * (uint32_t)sc_rb);
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const int i = (int)threadIdx.x + 256 * j;
            scv[j] = i < sc_ndw ? src[i] : 0u;
        }
    }
    const int mv0 = min(kGemmBM, n_e);
    uint32_t arow[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int drow = x.row0 + min(x.ar + 32 * q, mv0 - 1);
        arow[q] = a.a_by_token ? (uint32_t)(a.perm[drow] / a.K) : (uint32_t)drow;
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        const int i = (int)threadIdx.x + 256 * j;
        if (i < sc_ndw) reinterpret_cast<uint32_t*>(g_gemm_sct)[i] = scv[j];
    }
    x.g = a.wg[x.e];
    static_assert(kGemmBM == 64, "subtile dispatch below covers 1..4");
    switch ((mv0 + 15) / 16) {
        case 1: gemm_tile<EPI, 1, true>(a, x, 0, mv0, As, bb, arow); break;
        case 2: gemm_tile<EPI, 2, true>(a, x, 0, mv0, As, bb, arow); break;
        case 3: gemm_tile<EPI, 3, true>(a, x, 0, mv0, As, bb, arow); break;
        default: gemm_tile<EPI, 4, true>(a, x, 0, mv0, As, bb, arow); break;
    }
    // an expert's rows beyond the first 64 (rare at a few thousand tokens)
    for (int m0 = kGemmBM; m0 < n_e; m0 += kGemmBM)
        gemm_tile<EPI, 4, false>(a, x, m0, min(kGemmBM, n_e - m0), As, bb, arow);
}

// y32[t][n] = sum over slots s (in order) of w[t*K + s] * z[inv[t*K + s]][n]
// (the product rounded to fp32, then added); y = bf16.  One workgroup per
// token (H / 4 lanes rounded up to whole waves): the token's K rows and
// weights are uniform, read once through the scalar cache, and each lane
// takes 4 columns (H % 4 == 0), issuing its K row loads before summing them.
__global__ __launch_bounds__(1024) void k_combine(int T, int K, int H, const int32_t* inv, const float* w,
                                                  const float* z, float* y32, uint16_t* y) {
    const int t = blockIdx.x;
    const int n = 4 * (int)threadIdx.x;
    if (t >= T || n >= H) return;
    float4 v[8];
    float g[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        if (s < K) {
            v[s] = *reinterpret_cast<const float4*>(z + (size_t)inv[(size_t)t * K + s] * H + n);
            g[s] = w[(size_t)t * K + s];
        }
    }
    float4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        if (s < K) {
            acc.x += __fmul_rn(g[s], v[s].x);
            acc.y += __fmul_rn(g[s], v[s].y);
            acc.z += __fmul_rn(g[s], v[s].z);
            acc.w += __fmul_rn(g[s], v[s].w);
        }
    }
    const size_t i = (size_t)t * H + n;
    *reinterpret_cast<float4*>(y32 + i) = acc;
    uint2 b;
    b.x = f32_to_bf16_rne(acc.x) | (f32_to_bf16_rne(acc.y) << 16);
    b.y = f32_to_bf16_rne(acc.z) | (f32_to_bf16_rne(acc.w) << 16);
    *reinterpret_cast<uint2*>(y + i) = b;
}

}  // namespace q4moe
